// cache_write.hip -- quantise-on-write of new K/V rows into the paged caches.
//
// Each element is divided by its tensor's scale -- or its kv head's, with per-attention-head
// scales (same page and section) -- in IEEE binary32 and cast once to OCP
// E4M3 (page "FP8 KV Cache Quantization: Capacity Gains and Accuracy Risk", section
// "Scales and calibration"); the bytes are scattered by slot into 16-token blocks
// (same page, "Why the KV cache sets long-context capacity").  Values land in
// channel-major tiles [block][kv_head][dim][slot], the layout the decode kernel's P.V
// matrix-core operand reads with one 16-byte load per lane.  Keys land in tiles of
// 16-byte chunks ordered (slot quad, chunk, slot in quad, channel quarter), so that each
// key load instruction of the decode kernel reads whole 256-byte runs of a tile.
//
// One thread handles 8 consecutive channels of 4 consecutive input tokens of one kv head:
// four 16-byte bf16 loads per tensor, 64 f32 divisions (multiplies when both scales are
// powers of two, with the same result), then the stores.  When the four
// tokens go to four consecutive slots starting at a multiple of 4 (what a prefill or any
// in-order write of a sequence produces, except at its two ends) the four value bytes of
// one channel are adjacent in the channel-major tile: a 4 x 8 byte transpose in registers
// (byte permutes) turns the thread's codes into 8 four-byte channel stores, and the keys
// go out as 4 eight-byte stores.  Any other quad (scattered slots, the decode step's one
// token per sequence, a tail) takes the per-token path: 8-byte key stores and single-byte
// value stores.  Lanes are ordered (token quad, channel chunk, kv head, group of 4 quads),
// quad fastest, so the 4 lanes that complete one 16-byte channel row of a tile are
// adjacent.  Rows of tokens past the end are loaded clamped (in bounds) and never stored.
#include "codec.h"
#include "internal.h"

#include <type_traits>

namespace fp8kv {
namespace {

// In: a[k] = 4 one-byte codes (channels 0..3) of token k.  Out: r[c] = the 4 tokens'
// codes of channel c (token k in byte k).  Plain shifts and masks; the compiler turns them
// into byte permutes.
__device__ inline void transpose4x4(const uint32_t a[4], uint32_t r[4]) {
#pragma unroll
    for (int c = 0; c < 4; ++c)
        r[c] = ((a[0] >> (8 * c)) & 0xFFu) | (((a[1] >> (8 * c)) & 0xFFu) << 8) |
               (((a[2] >> (8 * c)) & 0xFFu) << 16) | (((a[3] >> (8 * c)) & 0xFFu) << 24);
}

// f(k) for k = 0..3 as compile-time constants: register arrays indexed by k stay in
// registers.
template <typename F>
__device__ inline void for4(F f) {
    f(std::integral_constant<int, 0>{});
    f(std::integral_constant<int, 1>{});
    f(std::integral_constant<int, 2>{});
    f(std::integral_constant<int, 3>{});
}

// 16 bytes as a native vector: copies of it stay in registers (copies of the uint4 struct
// wrapper are lowered as memory copies, which can move the arrays below out of registers).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ inline uint32_t dword(const u32x4& v, int i) {
    return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

// A scale that is a power of two, s = 2^k with s normal, has an exact reciprocal (2^-k,
// possibly subnormal), so x * (1 / s) and x / s are the same real number and IEEE
// rounding gives the same binary32 result, overflow and underflow included: the codes can
// be formed with a multiply.  Other scales take the division.
__device__ inline bool exact_reciprocal(float s) {
    const uint32_t b = __float_as_uint(s);
    return (b & 0x007FFFFFu) == 0 && (b & 0x7F800000u) != 0 && (b & 0x7F800000u) != 0x7F800000u;
}

// Eight bf16 (as 4 dwords) multiplied by the exact reciprocal of a power-of-two scale and
// cast: the same 8 codes as quantize8 with that scale.
template <int C>
__device__ inline uint2 quantize8_pow2(uint4 x, float rcp) {
    const uint32_t w[4] = {x.x, x.y, x.z, x.w};
    uint32_t c[4];
#pragma unroll
    for (int k = 0; k < 4; ++k)
        c[k] = pack2<C>(bf16_bits_to_f32(w[k] & 0xFFFFu) * rcp, bf16_bits_to_f32(w[k] >> 16) * rcp);
    return make_uint2(c[0] | (c[1] << 16), c[2] | (c[3] << 16));
}

template <int D, int C>
__global__ __launch_bounds__(256) void cache_write_kernel(CacheWriteParams p) {
    constexpr bool FP8 = C != kCodecBF16;         // one-byte codes (E4M3, E5M2 or INT8)
    constexpr int CH = D / 8;                     // 8-channel chunks per row
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t T = p.num_tokens;
    const int Hkv = p.num_kv_heads;
    const int64_t groups = (T + 15) / 16;
    if (gid >= groups * Hkv * CH * 4) return;
    const int tq = (int)(gid & 3);
    int64_t r = gid >> 2;
    const int c = (int)(r % CH);
    r /= CH;
    const int h = (int)(r % Hkv);
    const int64_t t0 = ((r / Hkv) * 4 + tq) * 4;  // first token of this thread's quad
    if (t0 >= T) return;

    // loads of clamped rows (always in bounds); only the stores below are guarded
    u32x4 xk[4], xv[4];
    int64_t sl[4];
    for4([&](auto kk) {
        constexpr int k = decltype(kk)::value;
        const int64_t tk = t0 + k < T ? t0 + k : T - 1;
        const int64_t row = (tk * Hkv + h) * D + c * 8;
        xk[k] = *reinterpret_cast<const u32x4*>(p.key + row);
        xv[k] = *reinterpret_cast<const u32x4*>(p.value + row);
        sl[k] = p.slot_mapping[tk];
    });
    const int64_t nslots = (int64_t)p.num_blocks * kBlockSize;
    // a slot past the cache is skipped, and reported (negative slots are padding by design)
    if (p.err != nullptr && c == 0 && h == 0) {
        bool bad = false;
        for4([&](auto kk) {
            constexpr int k = decltype(kk)::value;
            bad |= t0 + k < T && sl[k] >= nslots;
        });
        if (bad) report_error(p.err, kErrSlot);
    }
    const bool fast = t0 + 3 < T && sl[0] >= 0 && sl[0] < nslots && (sl[0] & 3) == 0 &&
                      sl[1] == sl[0] + 1 && sl[2] == sl[0] + 2 && sl[3] == sl[0] + 3;

    if constexpr (FP8) {
        uint8_t* kc = static_cast<uint8_t*>(p.key_cache);
        uint8_t* vc = static_cast<uint8_t*>(p.value_cache);
        const float ks = p.k_scales != nullptr ? p.k_scales[h] : p.k_scale;
        const float vs = p.v_scales != nullptr ? p.v_scales[h] : p.v_scale;
        uint2 qk[4], qv[4];
        if (exact_reciprocal(ks) && exact_reciprocal(vs)) {
            const float rk = 1.0f / ks, rv = 1.0f / vs;   // exact
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                qk[k] = quantize8_pow2<C>(make_uint4(xk[k].x, xk[k].y, xk[k].z, xk[k].w), rk);
                qv[k] = quantize8_pow2<C>(make_uint4(xv[k].x, xv[k].y, xv[k].z, xv[k].w), rv);
            }
        } else {
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                qk[k] = quantize8<C>(make_uint4(xk[k].x, xk[k].y, xk[k].z, xk[k].w), ks);
                qv[k] = quantize8<C>(make_uint4(xv[k].x, xv[k].y, xv[k].z, xv[k].w), vs);
            }
        }
        if (fast) {
            const int64_t blk = sl[0] / kBlockSize;
            const int off0 = (int)(sl[0] % kBlockSize);
            const int64_t tile = (blk * Hkv + h) * (int64_t)kBlockSize * D;
#pragma unroll
            for (int k = 0; k < 4; ++k)
                *reinterpret_cast<uint2*>(kc + tile + key_chunk_offset<D, 1>(off0 + k, c * 8)) = qk[k];
            const uint32_t lo[4] = {qv[0].x, qv[1].x, qv[2].x, qv[3].x};
            const uint32_t hi[4] = {qv[0].y, qv[1].y, qv[2].y, qv[3].y};
            uint32_t col[8];
            transpose4x4(lo, col);
            transpose4x4(hi, col + 4);
            uint8_t* vdst = vc + tile + (int64_t)(c * 8) * kBlockSize + off0;
#pragma unroll
            for (int j = 0; j < 8; ++j) *reinterpret_cast<uint32_t*>(vdst + j * kBlockSize) = col[j];
        } else {
            for4([&](auto kk) {
                constexpr int k = decltype(kk)::value;
                const int64_t slot = sl[k];
                if (t0 + k < T && slot >= 0 && slot < nslots) {
                    const int64_t blk = slot / kBlockSize;
                    const int off = (int)(slot % kBlockSize);
                    const int64_t tile = (blk * Hkv + h) * (int64_t)kBlockSize * D;
                    *reinterpret_cast<uint2*>(kc + tile + key_chunk_offset<D, 1>(off, c * 8)) = qk[k];
                    uint8_t* vdst = vc + tile + (int64_t)(c * 8) * kBlockSize + off;
#pragma unroll
                    for (int i = 0; i < 4; ++i) vdst[i * kBlockSize] = (uint8_t)(qv[k].x >> (8 * i));
#pragma unroll
                    for (int i = 0; i < 4; ++i) vdst[(i + 4) * kBlockSize] = (uint8_t)(qv[k].y >> (8 * i));
                }
            });
        }
    } else {
        uint16_t* kc = static_cast<uint16_t*>(p.key_cache);
        uint16_t* vc = static_cast<uint16_t*>(p.value_cache);
        if (fast) {
            const int64_t blk = sl[0] / kBlockSize;
            const int off0 = (int)(sl[0] % kBlockSize);
            const int64_t tile = (blk * Hkv + h) * (int64_t)kBlockSize * D;
#pragma unroll
            for (int k = 0; k < 4; ++k)
                *reinterpret_cast<u32x4*>(kc + tile + key_chunk_offset<D, 2>(off0 + k, c * 8) / 2) = xk[k];
            // channel 2i of token k is the low half of dword i of xv[k], channel 2i+1 the high
            uint16_t* vdst = vc + tile + (int64_t)(c * 8) * kBlockSize + off0;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t a0 = dword(xv[0], i), a1 = dword(xv[1], i);
                const uint32_t a2 = dword(xv[2], i), a3 = dword(xv[3], i);
                *reinterpret_cast<uint2*>(vdst + (2 * i) * kBlockSize) =
                    make_uint2((a0 & 0xFFFFu) | (a1 << 16), (a2 & 0xFFFFu) | (a3 << 16));
                *reinterpret_cast<uint2*>(vdst + (2 * i + 1) * kBlockSize) =
                    make_uint2((a0 >> 16) | (a1 & 0xFFFF0000u), (a2 >> 16) | (a3 & 0xFFFF0000u));
            }
        } else {
            for4([&](auto kk) {
                constexpr int k = decltype(kk)::value;
                const int64_t slot = sl[k];
                if (t0 + k < T && slot >= 0 && slot < nslots) {
                    const int64_t blk = slot / kBlockSize;
                    const int off = (int)(slot % kBlockSize);
                    const int64_t tile = (blk * Hkv + h) * (int64_t)kBlockSize * D;
                    *reinterpret_cast<u32x4*>(kc + tile + key_chunk_offset<D, 2>(off, c * 8) / 2) = xk[k];
                    uint16_t* vdst = vc + tile + (int64_t)(c * 8) * kBlockSize + off;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        vdst[(2 * i) * kBlockSize] = (uint16_t)(dword(xv[k], i) & 0xFFFFu);
                        vdst[(2 * i + 1) * kBlockSize] = (uint16_t)(dword(xv[k], i) >> 16);
                    }
                }
            });
        }
    }
}

template <int D>
hipError_t launch_d(const CacheWriteParams& p, Codec codec, hipStream_t s) {
    const int64_t total = (((int64_t)p.num_tokens + 15) / 16) * p.num_kv_heads * (D / 8) * 4;
    const int threads = 256;
    const int64_t blocks = (total + threads - 1) / threads;
    if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
    const void* fn;
    switch (codec) {
        case kCodecE4M3: fn = reinterpret_cast<const void*>(&cache_write_kernel<D, kCodecE4M3>); break;
        case kCodecBF16: fn = reinterpret_cast<const void*>(&cache_write_kernel<D, kCodecBF16>); break;
        case kCodecE5M2: fn = reinterpret_cast<const void*>(&cache_write_kernel<D, kCodecE5M2>); break;
        case kCodecINT8: fn = reinterpret_cast<const void*>(&cache_write_kernel<D, kCodecINT8>); break;
        default: return hipErrorInvalidValue;
    }
    return launch_kernel(fn, dim3((unsigned)blocks), dim3(threads), 0, s, p);
}

}  // namespace

hipError_t launch_cache_write(const CacheWriteParams& p, Codec codec, int head_dim, hipStream_t s) {
    switch (head_dim) {
        case 64: return launch_d<64>(p, codec, s);
        case 128: return launch_d<128>(p, codec, s);
        case 256: return launch_d<256>(p, codec, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace fp8kv
