// rotation.hip -- normalized Hadamard rotation around the cache: K and V rows are rotated
// before they are quantised, the query is rotated before attention, and the attention
// output is rotated back (page "KV Cache Quantization: What FP8 and q8_0 Cost in
// Accuracy", paragraph on the llama.cpp rotation merged on 2026-04-01: dot products are
// preserved while outliers spread across coordinates).  The Sylvester Hadamard matrix
// divided by sqrt(d) is symmetric and orthonormal, so one transform rotates both ways.
//
// A row of d values is held by d/8 consecutive lanes, 8 values each.  The fast
// Walsh-Hadamard butterflies run in the order h = 1, 2, ..., d/2: stages h < 8 combine
// values inside a lane, stages h >= 8 exchange with lane ^ (h/8).  Each butterfly output is
// one f32 add or subtract of the two inputs of that stage, so the result does not depend
// on which lane computes it; the scale (float)(1/sqrt(d)) follows as one f32 multiply.
// The write's codes are defined by exactly this f32 sequence.
#include "codec.h"
#include "hadamard.h"
#include "internal.h"

namespace fp8kv {
namespace {

// ---- rotated cache write: one lane per (token, kv head, 8 channels), d/8 lanes per row
template <int D, int C>
__global__ __launch_bounds__(256) void rotate_write_kernel(CacheWriteParams p, float rscale) {
    constexpr bool FP8 = C != kCodecBF16;  // one-byte codes
    constexpr int CH = D / 8;
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t total = (int64_t)p.num_tokens * p.num_kv_heads * CH;
    // whole rows exit together (a row's lanes are consecutive and CH divides 64)
    if (gid >= total) return;
    const int c = (int)(gid % CH);
    const int64_t th = gid / CH;                  // token * Hkv + head
    const int h = (int)(th % p.num_kv_heads);
    const int64_t t = th / p.num_kv_heads;
    float k[8], v[8];
    bf16x8_to_f32(*reinterpret_cast<const uint4*>(p.key + th * D + c * 8), k);
    bf16x8_to_f32(*reinterpret_cast<const uint4*>(p.value + th * D + c * 8), v);
    hadamard_row<D>(k, c, rscale);
    hadamard_row<D>(v, c, rscale);
    const int64_t slot = p.slot_mapping[t];
    if (slot >= (int64_t)p.num_blocks * kBlockSize && c == 0 && h == 0) report_error(p.err, kErrSlot);
    if (slot < 0 || slot >= (int64_t)p.num_blocks * kBlockSize) return;
    const int64_t blk = slot / kBlockSize;
    const int off = (int)(slot % kBlockSize);
    const int64_t tile = (blk * p.num_kv_heads + h) * (int64_t)kBlockSize * D;   // elements
    if constexpr (FP8) {
        uint8_t* kc = static_cast<uint8_t*>(p.key_cache);
        uint8_t* vc = static_cast<uint8_t*>(p.value_cache);
        uint32_t ck[4], cv[4];
        // the head's scales (per-kv-head arrays when given, else the per-tensor pair); h
        // differs between the rows of a wave, so these are vector loads
        const float ksc = p.k_scales != nullptr ? p.k_scales[h] : p.k_scale;
        const float vsc = p.v_scales != nullptr ? p.v_scales[h] : p.v_scale;
#pragma unroll
        for (int j = 0; j < 4; ++j) {   // IEEE f32 division by the scale, then the cast
            ck[j] = pack2<C>(k[2 * j] / ksc, k[2 * j + 1] / ksc);
            cv[j] = pack2<C>(v[2 * j] / vsc, v[2 * j + 1] / vsc);
        }
        *reinterpret_cast<uint2*>(kc + tile + key_chunk_offset<D, 1>(off, c * 8)) =
            make_uint2(ck[0] | (ck[1] << 16), ck[2] | (ck[3] << 16));
        uint8_t* vdst = vc + tile + (int64_t)(c * 8) * kBlockSize + off;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            vdst[(2 * j) * kBlockSize] = (uint8_t)(cv[j] & 0xFFu);
            vdst[(2 * j + 1) * kBlockSize] = (uint8_t)(cv[j] >> 8);
        }
    } else {
        uint16_t* kc = static_cast<uint16_t*>(p.key_cache);
        uint16_t* vc = static_cast<uint16_t*>(p.value_cache);
        *reinterpret_cast<uint4*>(kc + tile + key_chunk_offset<D, 2>(off, c * 8) / 2) =
            make_uint4(pack_bf16x2(k[0], k[1]), pack_bf16x2(k[2], k[3]), pack_bf16x2(k[4], k[5]),
                       pack_bf16x2(k[6], k[7]));
        uint16_t* vdst = vc + tile + (int64_t)(c * 8) * kBlockSize + off;
#pragma unroll
        for (int j = 0; j < 8; ++j)
            vdst[j * kBlockSize] = __builtin_bit_cast(uint16_t, (__bf16)v[j]);
    }
}

// ---- query rotation: q [rows][D] bf16 -> rotated q as hi + lo bf16 terms
template <int D>
__global__ __launch_bounds__(256) void rotate_query_kernel(const uint16_t* q, uint16_t* q_hi,
                                                           uint16_t* q_lo, int64_t rows,
                                                           float rscale) {
    constexpr int CH = D / 8;
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (gid >= rows * CH) return;
    const int c = (int)(gid % CH);
    const int64_t r = gid / CH;
    float v[8];
    bf16x8_to_f32(*reinterpret_cast<const uint4*>(q + r * D + c * 8), v);
    hadamard_row<D>(v, c, rscale);
    uint32_t hi[4], lo[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        hi[j] = pack_bf16x2(v[2 * j], v[2 * j + 1]);
        const float h0 = __uint_as_float(hi[j] << 16), h1 = __uint_as_float(hi[j] & 0xFFFF0000u);
        lo[j] = pack_bf16x2(v[2 * j] - h0, v[2 * j + 1] - h1);
    }
    *reinterpret_cast<uint4*>(q_hi + r * D + c * 8) = make_uint4(hi[0], hi[1], hi[2], hi[3]);
    *reinterpret_cast<uint4*>(q_lo + r * D + c * 8) = make_uint4(lo[0], lo[1], lo[2], lo[3]);
}

// ---- output rotation back: f32 [rows][D] -> out (bf16 or f32)
template <int D>
__global__ __launch_bounds__(256) void rotate_out_kernel(const float* in, void* out, int out_f32,
                                                         int64_t rows, float rscale) {
    constexpr int CH = D / 8;
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (gid >= rows * CH) return;
    const int c = (int)(gid % CH);
    const int64_t r = gid / CH;
    float v[8];
    const float4 a = *reinterpret_cast<const float4*>(in + r * D + c * 8);
    const float4 b = *reinterpret_cast<const float4*>(in + r * D + c * 8 + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    hadamard_row<D>(v, c, rscale);
    if (out_f32) {
        float* o = static_cast<float*>(out) + r * D + c * 8;
        *reinterpret_cast<float4*>(o) = make_float4(v[0], v[1], v[2], v[3]);
        *reinterpret_cast<float4*>(o + 4) = make_float4(v[4], v[5], v[6], v[7]);
    } else {
        uint16_t* o = static_cast<uint16_t*>(out) + r * D + c * 8;
        *reinterpret_cast<uint4*>(o) = make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]),
                                                  pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7]));
    }
}

inline float rotation_scale(int d) { return (float)(1.0 / sqrt((double)d)); }

// Launch `kernel` over threads_total threads (256 per workgroup) and return the status of
// this launch alone.
template <typename... A>
hipError_t launch_rows(void (*kernel)(A...), int64_t threads_total, hipStream_t s, A... args) {
    const int64_t blocks = (threads_total + 255) / 256;
    if (blocks <= 0) return hipSuccess;
    if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
    void* argv[] = {static_cast<void*>(&args)...};
    return hipLaunchKernel(reinterpret_cast<const void*>(kernel), dim3((unsigned)blocks), dim3(256),
                           argv, 0, s);
}

}  // namespace

template <int D>
hipError_t launch_rotate_write_d(const CacheWriteParams& p, Codec codec, int64_t total, float rs,
                                 hipStream_t s) {
    switch (codec) {
        case kCodecE4M3: return launch_rows(rotate_write_kernel<D, kCodecE4M3>, total, s, p, rs);
        case kCodecBF16: return launch_rows(rotate_write_kernel<D, kCodecBF16>, total, s, p, rs);
        case kCodecE5M2: return launch_rows(rotate_write_kernel<D, kCodecE5M2>, total, s, p, rs);
        case kCodecINT8: return launch_rows(rotate_write_kernel<D, kCodecINT8>, total, s, p, rs);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_rotate_write(const CacheWriteParams& p, Codec codec, int head_dim, hipStream_t s) {
    const int64_t total = (int64_t)p.num_tokens * p.num_kv_heads * (head_dim / 8);
    const float rs = rotation_scale(head_dim);
    switch (head_dim) {
        case 64: return launch_rotate_write_d<64>(p, codec, total, rs, s);
        case 128: return launch_rotate_write_d<128>(p, codec, total, rs, s);
        case 256: return launch_rotate_write_d<256>(p, codec, total, rs, s);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_rotate_query(const uint16_t* q, uint16_t* q_hi, uint16_t* q_lo, int64_t rows,
                               int head_dim, hipStream_t s) {
    const int64_t total = rows * (head_dim / 8);
    const float rs = rotation_scale(head_dim);
    switch (head_dim) {
        case 64: return launch_rows(rotate_query_kernel<64>, total, s, q, q_hi, q_lo, rows, rs);
        case 128: return launch_rows(rotate_query_kernel<128>, total, s, q, q_hi, q_lo, rows, rs);
        case 256: return launch_rows(rotate_query_kernel<256>, total, s, q, q_hi, q_lo, rows, rs);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_rotate_out(const float* in, void* out, int out_f32, int64_t rows, int head_dim,
                             hipStream_t s) {
    const int64_t total = rows * (head_dim / 8);
    const float rs = rotation_scale(head_dim);
    switch (head_dim) {
        case 64: return launch_rows(rotate_out_kernel<64>, total, s, in, out, out_f32, rows, rs);
        case 128: return launch_rows(rotate_out_kernel<128>, total, s, in, out, out_f32, rows, rs);
        case 256: return launch_rows(rotate_out_kernel<256>, total, s, in, out, out_f32, rows, rs);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace fp8kv
