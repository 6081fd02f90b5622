// hadamard.h -- the normalized Hadamard rotation of one d-element row held by d/8
// consecutive lanes (8 values each), in f32, and the bf16 helpers around it; shared by the
// rotated cache write and the rotated decode.  The fast Walsh-Hadamard butterflies run in
// the order h = 1, 2, ..., d/2 (stages h < 8 inside a lane, stages h >= 8 with lane ^ (h/8));
// each butterfly output is one f32 add or subtract of that stage's two inputs, so the
// result does not depend on which lane computes it.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8kv {

// v[0..7] = channels 8c .. 8c+7 of a row whose d/8 lanes are consecutive (lane c of the
// row at lane offset c).  Rotates the row in place, f32, then multiplies by `scale`.
template <int D>
__device__ inline void hadamard_row(float (&v)[8], int c, float scale) {
#pragma unroll
    for (int h = 1; h < 8; h *= 2)
#pragma unroll
        for (int j = 0; j < 8; ++j)
            if ((j & h) == 0) {
                const float a = v[j], b = v[j + h];
                v[j] = a + b;
                v[j + h] = a - b;
            }
#pragma unroll
    for (int h = 8; h < D; h *= 2) {
        const int m = h / 8;                  // partner lane: c ^ m
        const bool upper = (c & m) != 0;      // this lane holds x[j + h] of each pair
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const float other = __shfl_xor(v[j], m);
            v[j] = upper ? other - v[j] : v[j] + other;
        }
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = v[j] * scale;
}

__device__ inline void bf16x8_to_f32(uint4 x, float (&v)[8]) {
    const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        v[2 * k] = __uint_as_float(w[k] << 16);
        v[2 * k + 1] = __uint_as_float(w[k] & 0xFFFF0000u);
    }
}

__device__ inline uint32_t pack_bf16x2(float a, float b) {
    const __bf16 x = (__bf16)a, y = (__bf16)b;   // round to nearest even
    return (uint32_t)__builtin_bit_cast(uint16_t, x) | ((uint32_t)__builtin_bit_cast(uint16_t, y) << 16);
}

}  // namespace fp8kv
