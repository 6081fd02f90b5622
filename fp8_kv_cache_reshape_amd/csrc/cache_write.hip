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
// One thread handles 8 consecutive channels of one (token, kv head): a 16-byte bf16
// load per tensor, eight f32 divisions, four packed conversions, an 8-byte key store
// and eight strided value bytes.  At decode time the write moves a few KiB per step,
// so this kernel is sized for simplicity and exactness, not bandwidth.
#include "codec.h"
#include "internal.h"

namespace fp8kv {
namespace {

template <int D, bool FP8>
__global__ __launch_bounds__(256) void cache_write_kernel(CacheWriteParams p) {
    constexpr int CHUNKS = D / 8;
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t total = (int64_t)p.num_tokens * p.num_kv_heads * CHUNKS;
    if (gid >= total) return;
    const int c = (int)(gid % CHUNKS);
    const int64_t th = gid / CHUNKS;              // token * Hkv + head
    const int h = (int)(th % p.num_kv_heads);
    const int64_t t = th / p.num_kv_heads;
    // the row loads do not depend on the slot: issue them together with the slot load
    const uint4 xk = *reinterpret_cast<const uint4*>(p.key + th * D + c * 8);
    const uint4 xv = *reinterpret_cast<const uint4*>(p.value + th * D + c * 8);
    const int64_t slot = p.slot_mapping[t];
    if (slot < 0 || slot >= (int64_t)p.num_blocks * kBlockSize) return;
    const int64_t blk = slot / kBlockSize;
    const int off = (int)(slot % kBlockSize);
    const int64_t tile = (blk * p.num_kv_heads + h) * (int64_t)kBlockSize * D;   // elements
    if constexpr (FP8) {
        uint8_t* kc = static_cast<uint8_t*>(p.key_cache);
        uint8_t* vc = static_cast<uint8_t*>(p.value_cache);
        *reinterpret_cast<uint2*>(kc + tile + key_chunk_offset<D, 1>(off, c * 8)) =
            quantize8(xk, p.k_scales != nullptr ? p.k_scales[h] : p.k_scale);
        const uint2 qv = quantize8(xv, p.v_scales != nullptr ? p.v_scales[h] : p.v_scale);
        uint8_t* vdst = vc + tile + (int64_t)(c * 8) * kBlockSize + off;
#pragma unroll
        for (int i = 0; i < 4; ++i) vdst[i * kBlockSize] = (uint8_t)(qv.x >> (8 * i));
#pragma unroll
        for (int i = 0; i < 4; ++i) vdst[(i + 4) * kBlockSize] = (uint8_t)(qv.y >> (8 * i));
    } else {
        uint16_t* kc = static_cast<uint16_t*>(p.key_cache);
        uint16_t* vc = static_cast<uint16_t*>(p.value_cache);
        *reinterpret_cast<uint4*>(kc + tile + key_chunk_offset<D, 2>(off, c * 8) / 2) = xk;
        uint16_t* vdst = vc + tile + (int64_t)(c * 8) * kBlockSize + off;
        const uint32_t w[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            vdst[(2 * i) * kBlockSize] = (uint16_t)(w[i] & 0xFFFFu);
            vdst[(2 * i + 1) * kBlockSize] = (uint16_t)(w[i] >> 16);
        }
    }
}

template <int D>
hipError_t launch_d(const CacheWriteParams& p, bool fp8, hipStream_t s) {
    const int64_t total = (int64_t)p.num_tokens * p.num_kv_heads * (D / 8);
    const int threads = 256;
    const int64_t blocks = (total + threads - 1) / threads;
    if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
    const void* fn = fp8 ? reinterpret_cast<const void*>(&cache_write_kernel<D, true>)
                         : reinterpret_cast<const void*>(&cache_write_kernel<D, false>);
    return launch_kernel(fn, dim3((unsigned)blocks), dim3(threads), 0, s, p);
}

}  // namespace

hipError_t launch_cache_write(const CacheWriteParams& p, bool fp8, int head_dim, hipStream_t s) {
    switch (head_dim) {
        case 64: return launch_d<64>(p, fp8, s);
        case 128: return launch_d<128>(p, fp8, s);
        case 256: return launch_d<256>(p, fp8, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace fp8kv
