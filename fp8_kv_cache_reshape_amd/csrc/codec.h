// codec.h -- device-side encoding and decoding of the one-byte cache codecs (E4M3, E5M2,
// INT8), shared by the cache writes, the fused decode step, the decode and the prefill.
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

// Cache element codecs (the values of the C-ABI cache_dtype codes).
enum Codec : int { kCodecE4M3 = 0, kCodecBF16 = 1, kCodecE5M2 = 3, kCodecINT8 = 4 };

// RNE cast of two f32 values to OCP E5M2 codes (low byte = a): magnitudes >= 57344 and
// infinities clamp to +-57344, NaN becomes 0x7F with its sign.
__device__ inline uint32_t e5m2_pack2(float a, float b) {
    const float ca = fminf(fmaxf(a, -57344.0f), 57344.0f);
    const float cb = fminf(fmaxf(b, -57344.0f), 57344.0f);
    uint32_t r = (uint32_t)__builtin_amdgcn_cvt_pk_bf8_f32(ca, cb, 0, false) & 0xFFFFu;
    if (__builtin_isnan(a)) r = (r & 0xFF00u) | 0x7Fu | ((__float_as_uint(a) >> 24) & 0x80u);
    if (__builtin_isnan(b)) r = (r & 0x00FFu) | ((0x7Fu | ((__float_as_uint(b) >> 24) & 0x80u)) << 8);
    return r;
}

// Symmetric INT8 codes of two f32 values (low byte = a): nearest integer, ties to even,
// clamped to [-127, 127]; NaN becomes 0.
__device__ inline uint32_t int8_pack2(float a, float b) {
    auto one = [](float y) -> uint32_t {
        if (__builtin_isnan(y)) return 0u;
        const float r = fminf(fmaxf(__builtin_rintf(y), -127.0f), 127.0f);
        return (uint32_t)(int)r & 0xFFu;
    };
    return one(a) | (one(b) << 8);
}

template <int C>
__device__ inline uint32_t pack2(float a, float b) {
    if constexpr (C == kCodecE5M2) return e5m2_pack2(a, b);
    else if constexpr (C == kCodecINT8) return int8_pack2(a, b);
    else return e4m3_pack2(a, b);
}

// Eight bf16 (as 4 dwords) divided by `scale` and cast: returns 8 codes in 2 dwords.
template <int C = kCodecE4M3>
__device__ inline uint2 quantize8(uint4 x, float scale) {
    const uint32_t w[4] = {x.x, x.y, x.z, x.w};
    uint32_t c[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const float lo = bf16_bits_to_f32(w[k] & 0xFFFFu) / scale;   // IEEE binary32 division
        const float hi = bf16_bits_to_f32(w[k] >> 16) / scale;
        c[k] = pack2<C>(lo, hi);
    }
    return make_uint2(c[0] | (c[1] << 16), c[2] | (c[3] << 16));
}

// ---- decoding: 8 one-byte codes (bytes of lo then hi, memory order) -> 8 bf16, exactly
// (every E4M3, E5M2 and INT8 value is a bf16 value).
typedef __bf16 codec_bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 codec_bf16x2 __attribute__((ext_vector_type(2)));

template <int C>
__device__ inline codec_bf16x8 codes8_to_bf16x8(uint32_t lo, uint32_t hi) {
    if constexpr (C == kCodecINT8) {
        // signed byte -> f32 (exact) -> its upper half is the exact bf16
        uint32_t w[4];
        const uint32_t src[2] = {lo, hi};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const uint32_t d = src[k / 2];
            const int s = 16 * (k % 2);
            const float f0 = (float)(int)(int8_t)(d >> s);
            const float f1 = (float)(int)(int8_t)(d >> (s + 8));
            w[k] = (__float_as_uint(f0) >> 16) | (__float_as_uint(f1) & 0xFFFF0000u);
        }
        typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
        const u32x4_t v = {w[0], w[1], w[2], w[3]};
        return __builtin_bit_cast(codec_bf16x8, v);
    } else {
        codec_bf16x2 a, b, c, d;
        if constexpr (C == kCodecE5M2) {
            a = __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(lo, 1.0f, false);
            b = __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(lo, 1.0f, true);
            c = __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(hi, 1.0f, false);
            d = __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(hi, 1.0f, true);
        } else {
            a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false);
            b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true);
            c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false);
            d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true);
        }
        codec_bf16x8 r = {a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
        return r;
    }
}

// ---- 8 one-byte codes (bytes of lo then hi, memory order) -> 8 fp16, exactly: every E4M3
// value (|x| <= 448, steps >= 2^-9), every E5M2 value (E5M2 is fp16 with the low 8 bits
// dropped) and every INT8 value is an fp16 value.
typedef _Float16 codec_f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 codec_f16x2 __attribute__((ext_vector_type(2)));

template <int C>
__device__ inline codec_f16x8 codes8_to_f16x8(uint32_t lo, uint32_t hi) {
    static_assert(C != kCodecBF16, "one-byte codecs only");
    codec_f16x2 a, b, c, d;
    if constexpr (C == kCodecINT8) {
        const uint32_t src[2] = {lo, hi};
        codec_f16x2 w[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const uint32_t v = src[k / 2] >> (16 * (k % 2));
            const float f0 = (float)(int)(int8_t)v;              // exact
            const float f1 = (float)(int)(int8_t)(v >> 8);
            w[k] = codec_f16x2{(_Float16)f0, (_Float16)f1};      // exact (|x| <= 128)
        }
        a = w[0]; b = w[1]; c = w[2]; d = w[3];
    } else if constexpr (C == kCodecE5M2) {
        a = __builtin_amdgcn_cvt_scalef32_pk_f16_bf8(lo, 1.0f, false);
        b = __builtin_amdgcn_cvt_scalef32_pk_f16_bf8(lo, 1.0f, true);
        c = __builtin_amdgcn_cvt_scalef32_pk_f16_bf8(hi, 1.0f, false);
        d = __builtin_amdgcn_cvt_scalef32_pk_f16_bf8(hi, 1.0f, true);
    } else {
        a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 1.0f, false);
        b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 1.0f, true);
        c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 1.0f, false);
        d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 1.0f, true);
    }
    codec_f16x8 r = {a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
    return r;
}

}  // namespace fp8kv
