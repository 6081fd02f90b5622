// codec.h -- device-side E4M3 encoding shared by the cache write and the fused decode step.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8kv {

__device__ inline float bf16_bits_to_f32(uint32_t h16) { return __uint_as_float(h16 << 16); }

// RNE cast of two f32 values to E4M3 codes (low byte = a, next byte = b).  The hardware
// conversion rounds to nearest even; saturation and NaN are made explicit here:
// magnitudes >= 448 and infinities clamp to +-448, NaN becomes 0x7F with its sign.
__device__ inline uint32_t e4m3_pack2(float a, float b) {
    const float ca = fminf(fmaxf(a, -448.0f), 448.0f);
    const float cb = fminf(fmaxf(b, -448.0f), 448.0f);
    uint32_t r = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(ca, cb, 0, false) & 0xFFFFu;
    if (__builtin_isnan(a)) r = (r & 0xFF00u) | 0x7Fu | ((__float_as_uint(a) >> 24) & 0x80u);
    if (__builtin_isnan(b)) r = (r & 0x00FFu) | ((0x7Fu | ((__float_as_uint(b) >> 24) & 0x80u)) << 8);
    return r;
}

// Eight bf16 (as 4 dwords) divided by `scale` and cast: returns 8 codes in 2 dwords.
__device__ inline uint2 quantize8(uint4 x, float scale) {
    const uint32_t w[4] = {x.x, x.y, x.z, x.w};
    uint32_t c[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const float lo = bf16_bits_to_f32(w[k] & 0xFFFFu) / scale;   // IEEE binary32 division
        const float hi = bf16_bits_to_f32(w[k] >> 16) / scale;
        c[k] = e4m3_pack2(lo, hi);
    }
    return make_uint2(c[0] | (c[1] << 16), c[2] | (c[3] << 16));
}

}  // namespace fp8kv
