/*
 * oracle.c -- plain, slow, obviously-correct CPU reference for the fp8 KV-cache
 * hot path: the e4m3 codec, quantise-on-write into the paged cache, and GQA
 * decode attention over that cache in fp64.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path links, loads or calls
 * this file: only the tests, the smoke check and the benchmark's CPU-baseline
 * leg do.  It shares no code, header, table or constant with the HIP library.
 *
 * Citations name the source pages by title and section:
 *   [VLLM]  "The State of FP8 KV-Cache and Attention Quantization in vLLM"
 *           (vLLM project blog summary), keyed paragraphs such as
 *           "ACCURACY AT LONG CONTEXT" and "DECODE COST".
 *   [FLOPS] "ctx-fp8-kv-cache-long-context-accuracy" (arithmetic-intensity
 *           record), sections "Arithmetic intensity", "Workarounds", "notes".
 *   [CAP]   "FP8 KV Cache Quantization: Capacity Gains and Accuracy Risk"
 *           (GPU Smith), sections named where cited.
 *   [ACC]   "KV Cache Quantization: What FP8 and q8_0 Cost in Accuracy"
 *           (Particula Tech), cited by paragraph topic.
 *
 * Readings where the pages are silent (each also listed in the design notes):
 *   - fp8 flavour is OCP E4M3 ("fn"): bias 7, no infinities, S.1111.111 = NaN,
 *     largest finite 448 [CAP "What FP8 KV changes" / E4M3 vs E5M2].
 *   - the element is divided by the per-tensor scale in IEEE f32 and then cast
 *     once to e4m3 with round-to-nearest-even; magnitudes at or above 448 (and
 *     infinities) saturate to 448; NaN keeps its sign [CAP "Scales and
 *     calibration"]; rounding and saturation are not stated on the pages.
 *   - decoding multiplies the code's value by the same scale.
 *   - paged layout: one tile per (block, kv_head), tiles ordered [block][kv_head].
 *     Value tiles are channel-major: element (slot t, dim i) at i*bs + t.  Key tiles
 *     are 16-byte chunks ordered (slot quad, chunk, slot within quad, dim quarter):
 *     element (t, i) at byte ((t/4 * C + c) * 4 + t%4) * 4K + g*K + w%K, where
 *     g = i / (D/4), w = (i % (D/4)) * elem_bytes, K = min(16, D*elem_bytes/4) is the
 *     chunk size, c = w / K and C = D*elem_bytes/(4K).  (K = 16 for every head_dim the
 *     library supports; when the quarter is at most 16 bytes, e.g. D = 64 with 1-byte
 *     elements, this is plain token-major.)  The pages fix
 *     only that the cache is held in fixed-size blocks [CAP "Why the KV cache sets
 *     long-context capacity"].
 *   - query head hq reads kv head hq / g, g = Hq / Hkv (contiguous groups);
 *     the pages name only the group ratio g [FLOPS "Arithmetic intensity"].
 *   - positions attended: [lo, L) with lo = max(0, L - W) for a window W > 0,
 *     else 0; an empty range yields a zero output.
 *   - softmax scale 1/sqrt(head_dim).
 *
 * Precision: all attention arithmetic in double; the only float operation is
 * the quantiser's f32 division, which is the step being specified.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_CACHE_E4M3 0
#define ORACLE_CACHE_BF16 1
#define ORACLE_CACHE_E5M2 3
#define ORACLE_CACHE_INT8 4

/* ---------------------------------------------------------------- bf16 --- */

/* A bf16 value is the upper half of an IEEE binary32. */
float oracle_bf16_to_f32(uint16_t h) {
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* ---------------------------------------------------------------- e4m3 --- */

/*
 * Value of an OCP E4M3 code [CAP "What FP8 KV changes" / E4M3 vs E5M2: three
 * mantissa bits, largest normal 448].  Fields: sign s = bit 7, exponent
 * E = bits 6..3 (bias 7), mantissa M = bits 2..0.
 *   E = 15, M = 7   -> NaN (the only non-finite codes; there is no infinity)
 *   E = 0           -> subnormal, M * 2^-9
 *   otherwise       -> (1 + M/8) * 2^(E-7)
 */
double oracle_e4m3_decode(uint8_t c) {
    int s = (c >> 7) & 1;
    int E = (c >> 3) & 0xF;
    int M = c & 0x7;
    double mag;
    if (E == 15 && M == 7) return s ? -NAN : NAN;
    if (E == 0)
        mag = ldexp((double)M, -9);
    else
        mag = ldexp(1.0 + (double)M / 8.0, E - 7);
    return s ? -mag : mag;
}

/*
 * Nearest E4M3 code to y, ties to even mantissa, saturating at 448.
 * y is an f32 value carried in a double, so every step below is exact in
 * double except the explicit rint() (round-half-even under the default
 * rounding mode).
 */
uint8_t oracle_e4m3_encode(double y) {
    uint8_t sign = signbit(y) ? 0x80 : 0x00;
    double a = fabs(y);
    if (isnan(y)) return (uint8_t)(sign | 0x7F);
    if (a >= 448.0) return (uint8_t)(sign | 0x7E);   /* saturate, +-inf too */
    if (a < ldexp(1.0, -6)) {
        /* subnormal spacing 2^-9; m == 8 is the smallest normal, code 0x08 */
        double m = rint(a * 512.0);
        return (uint8_t)(sign | (uint8_t)m);
    }
    int e;
    (void)frexp(a, &e);      /* a = f * 2^e, f in [0.5, 1) */
    e -= 1;                  /* now a = f' * 2^e, f' in [1, 2) */
    double m = rint((ldexp(a, -e) - 1.0) * 8.0);
    if (m == 8.0) {          /* mantissa carried into the exponent */
        m = 0.0;
        e += 1;
    }
    /* a < 448 = 1.75 * 2^8 keeps (e, m) at or below (8, 6): never the NaN code */
    return (uint8_t)(sign | (uint8_t)((e + 7) << 3) | (uint8_t)m);
}

/*
 * Quantise one bf16 element with a per-tensor scale: divide in IEEE f32, then
 * cast once to e4m3 [CAP "Scales and calibration": each K or V tensor is
 * divided by its scale before the cast].
 */
uint8_t oracle_quantize(uint16_t x_bf16, float scale) {
    float x = oracle_bf16_to_f32(x_bf16);
    float y = x / scale;                 /* binary32 division, round-to-nearest-even */
    return oracle_e4m3_encode((double)y);
}

/* ------------------------------------------------------ other codecs --- */

/*
 * The two other one-byte codecs the pages name for the KV cache: E5M2 (two mantissa
 * bits, largest finite 57344 [FLOPS "Workarounds"; CAP "What FP8 KV changes" / E4M3 vs
 * E5M2]) and INT8 (a near-identical story with no separate measurement [FLOPS "notes"]).
 * The pages give neither codec's rounding; the readings mirror the E4M3 ones:
 *   E5M2 (OCP): sign bit 7, exponent bits 6..2 (bias 15), mantissa bits 1..0;
 *     E = 31 is infinity (M = 0) or NaN; E = 0 is subnormal, M * 2^-16.  Encoding rounds
 *     to nearest with ties to the even code, saturates magnitudes >= 57344 (and
 *     infinities) to +-57344, keeps the sign of zero, and maps NaN to 0x7F | sign.
 *   INT8: symmetric; the code is the f32 quotient rounded to the nearest integer (ties to
 *     even) and clamped to [-127, 127], stored as a two's-complement byte; NaN -> 0.
 */
double oracle_e5m2_decode(uint8_t c) {
    int sign = c >> 7, E = (c >> 2) & 0x1F, M = c & 3;
    double mag;
    if (E == 31)
        mag = M == 0 ? INFINITY : NAN;
    else if (E == 0)
        mag = ldexp((double)M, -16);
    else
        mag = ldexp(1.0 + (double)M / 4.0, E - 15);
    return sign ? -mag : mag;
}

uint8_t oracle_e5m2_encode(double y) {
    uint8_t sgn = signbit(y) ? 0x80 : 0x00;
    if (isnan(y)) return (uint8_t)(0x7F | sgn);
    double a = fabs(y);
    if (a >= 57344.0) return (uint8_t)(sgn | 0x7B);          /* saturate */
    if (a < ldexp(1.0, -14)) {                                /* subnormal range */
        double m = rint(ldexp(a, 16));                        /* m = 4 is the smallest normal */
        return (uint8_t)(sgn | (uint8_t)m);
    }
    int e = (int)floor(log2(a));
    if (ldexp(1.0, e) > a) e -= 1;                            /* guard log2 rounding */
    if (ldexp(1.0, e + 1) <= a) e += 1;
    double mq = rint((ldexp(a, -e) - 1.0) * 4.0);
    if (mq == 4.0) {
        mq = 0.0;
        e += 1;
    }
    return (uint8_t)(sgn | ((e + 15) << 2) | (int)mq);
}

double oracle_int8_decode(uint8_t c) { return (double)(int8_t)c; }

uint8_t oracle_int8_encode(double y) {
    if (isnan(y)) return 0;
    double r = rint(y);                                       /* ties to even */
    if (r > 127.0) r = 127.0;
    if (r < -127.0) r = -127.0;
    return (uint8_t)(int8_t)r;
}

/* The f32 quotient of a bf16 element and the scale, cast once to the codec. */
static uint8_t quantize_codec(uint16_t x_bf16, float scale, int codec) {
    float y = oracle_bf16_to_f32(x_bf16) / scale;
    if (codec == ORACLE_CACHE_E5M2) return oracle_e5m2_encode((double)y);
    if (codec == ORACLE_CACHE_INT8) return oracle_int8_encode((double)y);
    return oracle_e4m3_encode((double)y);
}

void oracle_e5m2_decode_n(const uint8_t* c, double* out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_e5m2_decode(c[i]);
}
void oracle_e5m2_encode_n(const double* y, uint8_t* out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_e5m2_encode(y[i]);
}
void oracle_int8_encode_n(const double* y, uint8_t* out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_int8_encode(y[i]);
}

/* Array helpers so callers can sweep whole domains in one call. */
void oracle_e4m3_decode_n(const uint8_t* c, double* out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_e4m3_decode(c[i]);
}
void oracle_e4m3_encode_n(const double* y, uint8_t* out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_e4m3_encode(y[i]);
}
void oracle_quantize_n(const uint16_t* x, float scale, uint8_t* out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_quantize(x[i], scale);
}
void oracle_div_f32_n(const float* x, float scale, float* out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = x[i] / scale;
}

/* ------------------------------------------------------- paged layout --- */

/* Element offset of (block, kv_head, slot, dim) in a key cache whose elements take
 * `eb` bytes (1 for e4m3, 2 for bf16); see the layout note at the top. */
static int64_t key_index(int64_t blk, int h, int off, int i, int Hkv, int bs, int D, int eb) {
    int q = D / 4;                     /* dims per quarter (D is a multiple of 4) */
    int g = i / q;                     /* quarter */
    int w = (i % q) * eb;              /* byte within the quarter's part of the row */
    int K = q * eb < 16 ? q * eb : 16; /* chunk bytes: 16, or the whole quarter if smaller */
    int C = q * eb / K;                /* chunks per quarter */
    int c = w / K;
    int64_t byte_in_tile = ((int64_t)((off / 4) * C + c) * 4 + off % 4) * (4 * K) + g * K + w % K;
    return (blk * Hkv + h) * (int64_t)bs * D + byte_in_tile / eb;
}
/* Offset of (block, kv_head, slot, dim) in a value cache (channel-major tile). */
static int64_t value_index(int64_t blk, int h, int off, int i, int Hkv, int bs, int D) {
    return ((blk * Hkv + h) * (int64_t)D + i) * (int64_t)bs + off;
}

/* --------------------------------------------------------- cache write --- */

/*
 * Quantise-on-write [CAP "Scales and calibration"] and scatter by slot into
 * paged blocks [CAP "Why the KV cache sets long-context capacity"].
 *   key, value    bf16 [T][Hkv][D]
 *   key_cache     [NB][Hkv] chunked key tiles, value_cache [NB][Hkv][D][bs] (layout
 *                 note at the top; bs = 16), elements of
 *                 cache_dtype (u8 e4m3 codes, or bf16 kept as-is: the native-
 *                 dtype variant used for skipped sliding-window layers,
 *                 [FLOPS "Workarounds"]; scales are not applied to it)
 *   slot_mapping  int64 [T]: slot = block * bs + offset.  A slot outside
 *                 [0, NB*bs) writes nothing.  Untouched bytes keep their value.
 */
void oracle_cache_write(const uint16_t* key, const uint16_t* value,
                        void* key_cache, void* value_cache, int cache_dtype,
                        const int64_t* slot_mapping, int T, int Hkv, int D,
                        int bs, int NB, float k_scale, float v_scale) {
    for (int t = 0; t < T; ++t) {
        int64_t slot = slot_mapping[t];
        if (slot < 0 || slot >= (int64_t)NB * bs) continue;
        int64_t blk = slot / bs;
        int off = (int)(slot % bs);
        for (int h = 0; h < Hkv; ++h) {
            for (int i = 0; i < D; ++i) {
                uint16_t xk = key[((int64_t)t * Hkv + h) * D + i];
                uint16_t xv = value[((int64_t)t * Hkv + h) * D + i];
                int64_t ki = key_index(blk, h, off, i, Hkv, bs, D,
                                       cache_dtype == ORACLE_CACHE_BF16 ? 2 : 1);
                int64_t vi = value_index(blk, h, off, i, Hkv, bs, D);
                if (cache_dtype == ORACLE_CACHE_E4M3) {
                    ((uint8_t*)key_cache)[ki] = oracle_quantize(xk, k_scale);
                    ((uint8_t*)value_cache)[vi] = oracle_quantize(xv, v_scale);
                } else {
                    ((uint16_t*)key_cache)[ki] = xk;
                    ((uint16_t*)value_cache)[vi] = xv;
                }
            }
        }
    }
}

/*
 * Per-attention-head scales [CAP "Scales and calibration"]: the same write with one
 * scale pair per kv head -- head h's key elements are divided by k_scales[h] and its
 * value elements by v_scales[h] before the cast (k_scales, v_scales float [Hkv]).
 */
void oracle_cache_write_per_head(const uint16_t* key, const uint16_t* value,
                                 void* key_cache, void* value_cache, int cache_dtype,
                                 const int64_t* slot_mapping, int T, int Hkv, int D,
                                 int bs, int NB, const float* k_scales, const float* v_scales) {
    for (int t = 0; t < T; ++t) {
        int64_t slot = slot_mapping[t];
        if (slot < 0 || slot >= (int64_t)NB * bs) continue;
        int64_t blk = slot / bs;
        int off = (int)(slot % bs);
        for (int h = 0; h < Hkv; ++h) {
            for (int i = 0; i < D; ++i) {
                uint16_t xk = key[((int64_t)t * Hkv + h) * D + i];
                uint16_t xv = value[((int64_t)t * Hkv + h) * D + i];
                int64_t ki = key_index(blk, h, off, i, Hkv, bs, D,
                                       cache_dtype == ORACLE_CACHE_BF16 ? 2 : 1);
                int64_t vi = value_index(blk, h, off, i, Hkv, bs, D);
                if (cache_dtype == ORACLE_CACHE_E4M3) {
                    ((uint8_t*)key_cache)[ki] = oracle_quantize(xk, k_scales[h]);
                    ((uint8_t*)value_cache)[vi] = oracle_quantize(xv, v_scales[h]);
                } else {
                    ((uint16_t*)key_cache)[ki] = xk;
                    ((uint16_t*)value_cache)[vi] = xv;
                }
            }
        }
    }
}

/*
 * The cache write with a one-byte codec (ORACLE_CACHE_E4M3, _E5M2 or _INT8): the same
 * slots and tile layout as oracle_cache_write, each element cast by quantize_codec.
 */
void oracle_cache_write_codec(const uint16_t* key, const uint16_t* value,
                              void* key_cache, void* value_cache, int codec,
                              const int64_t* slot_mapping, int T, int Hkv, int D,
                              int bs, int NB, float k_scale, float v_scale) {
    for (int t = 0; t < T; ++t) {
        int64_t slot = slot_mapping[t];
        if (slot < 0 || slot >= (int64_t)NB * bs) continue;
        int64_t blk = slot / bs;
        int in_blk = (int)(slot % bs);
        for (int h = 0; h < Hkv; ++h)
            for (int i = 0; i < D; ++i) {
                int64_t src = ((int64_t)t * Hkv + h) * D + i;
                ((uint8_t*)key_cache)[key_index(blk, h, in_blk, i, Hkv, bs, D, 1)] =
                    quantize_codec(key[src], k_scale, codec);
                ((uint8_t*)value_cache)[value_index(blk, h, in_blk, i, Hkv, bs, D)] =
                    quantize_codec(value[src], v_scale, codec);
            }
    }
}

/* Dequantised cache element: the code's value times scale, or the bf16 value. */
static double cache_value(const void* cache, int cache_dtype, int64_t idx, double scale) {
    if (cache_dtype == ORACLE_CACHE_E5M2)
        return oracle_e5m2_decode(((const uint8_t*)cache)[idx]) * scale;
    if (cache_dtype == ORACLE_CACHE_INT8)
        return oracle_int8_decode(((const uint8_t*)cache)[idx]) * scale;
    if (cache_dtype == ORACLE_CACHE_E4M3)
        return oracle_e4m3_decode(((const uint8_t*)cache)[idx]) * scale;
    return (double)oracle_bf16_to_f32(((const uint16_t*)cache)[idx]);
}

/* ---------------------------------------------------- decode attention --- */

/*
 * Softmax attention of one query vector over L_eff key/value rows, fp64:
 *   s_j = (q . K_j) / sqrt(D);  w_j = exp(s_j - max s);  out = sum w_j V_j / sum w_j
 * K and V are given already dequantised, row-major [n][D].  n = 0 -> zeros.
 * This is the unpaged definition the paged walk below must agree with.
 */
void oracle_attention_rows(double* out, const double* q, const double* K,
                           const double* V, int64_t n, int D) {
    for (int i = 0; i < D; ++i) out[i] = 0.0;
    if (n <= 0) return;
    double* s = (double*)malloc(sizeof(double) * (size_t)n);
    double m = -INFINITY;
    for (int64_t j = 0; j < n; ++j) {
        double dot = 0.0;
        for (int i = 0; i < D; ++i) dot += q[i] * K[j * D + i];
        s[j] = dot / sqrt((double)D);
        if (s[j] > m) m = s[j];
    }
    double Z = 0.0;
    for (int64_t j = 0; j < n; ++j) {
        s[j] = exp(s[j] - m);
        Z += s[j];
    }
    for (int64_t j = 0; j < n; ++j)
        for (int i = 0; i < D; ++i) out[i] += s[j] * V[j * D + i];
    for (int i = 0; i < D; ++i) out[i] /= Z;
    free(s);
}

/*
 * Decode attention for one (sequence b, query head hq) over the paged cache:
 * GQA with group ratio g = Hq/Hkv [FLOPS "Arithmetic intensity"], K and V
 * dequantised inside the attention [CAP "Attention backend interactions"],
 * optional sliding window [CAP "Accuracy risks to test for"].
 *   q             bf16 [B][Hq][D]
 *   block_tables  int32 [B][max_blocks]; logical block n of sequence b lives
 *                 in physical block block_tables[b][n]
 *   context_lens  int32 [B]
 *   out           double [D]
 */
void oracle_paged_decode_head(double* out, const uint16_t* q,
                              const void* key_cache, const void* value_cache,
                              int cache_dtype, const int32_t* block_tables,
                              int max_blocks, const int32_t* context_lens,
                              int Hq, int Hkv, int D, int bs,
                              double k_scale, double v_scale, int window,
                              int b, int hq) {
    int g = Hq / Hkv;
    int h = hq / g;
    int64_t L = context_lens[b];
    int64_t lo = (window > 0 && L > window) ? L - window : 0;
    int64_t n = L > lo ? L - lo : 0;
    int eb = cache_dtype == ORACLE_CACHE_BF16 ? 2 : 1;
    double* qv = (double*)malloc(sizeof(double) * (size_t)D);
    double* K = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1) * D);
    double* V = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1) * D);
    for (int i = 0; i < D; ++i)
        qv[i] = (double)oracle_bf16_to_f32(q[((int64_t)b * Hq + hq) * D + i]);
    for (int64_t j = lo; j < L; ++j) {
        int64_t pb = block_tables[(int64_t)b * max_blocks + j / bs];
        int off = (int)(j % bs);
        for (int i = 0; i < D; ++i) {
            K[(j - lo) * D + i] = cache_value(key_cache, cache_dtype,
                                              key_index(pb, h, off, i, Hkv, bs, D, eb), k_scale);
            V[(j - lo) * D + i] = cache_value(value_cache, cache_dtype,
                                              value_index(pb, h, off, i, Hkv, bs, D), v_scale);
        }
    }
    oracle_attention_rows(out, qv, K, V, n, D);
    free(qv);
    free(K);
    free(V);
}

/* All (b, hq) pairs: out double [B][Hq][D]. */
void oracle_paged_decode(double* out, const uint16_t* q, const void* key_cache,
                         const void* value_cache, int cache_dtype,
                         const int32_t* block_tables, int max_blocks,
                         const int32_t* context_lens, int B, int Hq, int Hkv,
                         int D, int bs, double k_scale, double v_scale, int window) {
    for (int b = 0; b < B; ++b)
        for (int hq = 0; hq < Hq; ++hq)
            oracle_paged_decode_head(out + ((int64_t)b * Hq + hq) * D, q, key_cache,
                                     value_cache, cache_dtype, block_tables, max_blocks,
                                     context_lens, Hq, Hkv, D, bs, k_scale, v_scale,
                                     window, b, hq);
}

/* Selected (b, hq) pairs, pairs int32 [n][2]: out double [n][D]. */
void oracle_paged_decode_pairs(double* out, const int32_t* pairs, int npairs,
                               const uint16_t* q, const void* key_cache,
                               const void* value_cache, int cache_dtype,
                               const int32_t* block_tables, int max_blocks,
                               const int32_t* context_lens, int Hq, int Hkv, int D,
                               int bs, double k_scale, double v_scale, int window) {
    for (int p = 0; p < npairs; ++p)
        oracle_paged_decode_head(out + (int64_t)p * D, q, key_cache, value_cache,
                                 cache_dtype, block_tables, max_blocks, context_lens,
                                 Hq, Hkv, D, bs, k_scale, v_scale, window,
                                 pairs[2 * p], pairs[2 * p + 1]);
}

/*
 * Per-attention-head scales [CAP "Scales and calibration"]: selected (b, hq) pairs, each
 * query head dequantising with the scales of its kv head h = hq / g (k_scales, v_scales
 * double [Hkv]).  out double [n][D].
 */
void oracle_paged_decode_pairs_per_head(double* out, const int32_t* pairs, int npairs,
                                        const uint16_t* q, const void* key_cache,
                                        const void* value_cache, int cache_dtype,
                                        const int32_t* block_tables, int max_blocks,
                                        const int32_t* context_lens, int Hq, int Hkv, int D,
                                        int bs, const double* k_scales, const double* v_scales,
                                        int window) {
    int g = Hq / Hkv;
    for (int p = 0; p < npairs; ++p) {
        int kv = pairs[2 * p + 1] / g;
        oracle_paged_decode_head(out + (int64_t)p * D, q, key_cache, value_cache,
                                 cache_dtype, block_tables, max_blocks, context_lens,
                                 Hq, Hkv, D, bs, k_scales[kv], v_scales[kv], window,
                                 pairs[2 * p], pairs[2 * p + 1]);
    }
}

/* ---------------------------------------------------- prefill attention --- */

/*
 * Prefill / chunked prefill over the paged cache: the query tokens of a prompt chunk
 * attend to the cached context, the chunk itself included, with K and V dequantised
 * inside the attention [CAP "Attention backend interactions"]; this is the pass whose
 * contraction runs over the whole context [VLLM "ACCURACY AT LONG CONTEXT"].
 * Sequence b's chunk is the query rows [qsl[b], qsl[b+1]); its n_b = qsl[b+1] - qsl[b]
 * tokens occupy the last n_b positions of the context, so row qsl[b] + j sits at position
 * p = L_b - n_b + j (L_b = context_lens[b], which counts the chunk).  Position p attends
 * causally to positions [lo, p] with lo = max(0, p + 1 - W) for a window W > 0, else 0:
 * exactly a decode over a context of length p + 1.  A row with p < 0 attends to nothing
 * and gets a zero output.
 *   q      bf16 [Tq][Hq][D]
 *   pairs  int32 [n][2]: (query row, query head) to compute;  out double [n][D]
 */
void oracle_hadamard_f64(double* x, int d);

/* rotate != 0: the rotated-cache form (page "KV Cache Quantization: What FP8 and q8_0 Cost
 * in Accuracy", paragraph on the llama.cpp rotation): each query row is rotated (fp64)
 * before the attention and each output row rotated back, as oracle_paged_decode_rotated_pairs
 * does for one decode token. */
static void prefill_pairs_core(double* out, const int32_t* pairs, int npairs,
                               const uint16_t* q, const int32_t* qsl, int B,
                               const void* key_cache, const void* value_cache,
                               int cache_dtype, const int32_t* block_tables, int max_blocks,
                               const int32_t* context_lens, int Hq, int Hkv, int D, int bs,
                               double k_scale, double v_scale, int window, int rotate) {
    int group = Hq / Hkv;
    int eb = cache_dtype == ORACLE_CACHE_BF16 ? 2 : 1;
    for (int p = 0; p < npairs; ++p) {
        int64_t row = pairs[2 * p];
        int hq = pairs[2 * p + 1];
        int kvh = hq / group;
        int b = 0;                               /* the sequence that owns this row */
        while (b + 1 < B && qsl[b + 1] <= row) ++b;
        int64_t chunk = qsl[b + 1] - qsl[b];
        int64_t pos = (int64_t)context_lens[b] - chunk + (row - qsl[b]);
        int64_t end = pos + 1;                   /* attended positions: [start, end) */
        int64_t start = (window > 0 && end > window) ? end - window : 0;
        int64_t n = end > start ? end - start : 0;
        double* qv = (double*)malloc(sizeof(double) * (size_t)D);
        double* K = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1) * D);
        double* V = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1) * D);
        for (int i = 0; i < D; ++i)
            qv[i] = (double)oracle_bf16_to_f32(q[(row * Hq + hq) * D + i]);
        if (rotate) oracle_hadamard_f64(qv, D);
        for (int64_t j = start; j < end; ++j) {
            int64_t phys = block_tables[(int64_t)b * max_blocks + j / bs];
            int slot = (int)(j % bs);
            for (int i = 0; i < D; ++i) {
                K[(j - start) * D + i] = cache_value(key_cache, cache_dtype,
                                                     key_index(phys, kvh, slot, i, Hkv, bs, D, eb),
                                                     k_scale);
                V[(j - start) * D + i] = cache_value(value_cache, cache_dtype,
                                                     value_index(phys, kvh, slot, i, Hkv, bs, D),
                                                     v_scale);
            }
        }
        oracle_attention_rows(out + (int64_t)p * D, qv, K, V, n, D);
        if (rotate) oracle_hadamard_f64(out + (int64_t)p * D, D);   /* back to the original coordinates */
        free(qv);
        free(K);
        free(V);
    }
}

void oracle_paged_prefill_pairs(double* out, const int32_t* pairs, int npairs,
                                const uint16_t* q, const int32_t* qsl, int B,
                                const void* key_cache, const void* value_cache,
                                int cache_dtype, const int32_t* block_tables, int max_blocks,
                                const int32_t* context_lens, int Hq, int Hkv, int D, int bs,
                                double k_scale, double v_scale, int window) {
    prefill_pairs_core(out, pairs, npairs, q, qsl, B, key_cache, value_cache, cache_dtype,
                       block_tables, max_blocks, context_lens, Hq, Hkv, D, bs, k_scale, v_scale,
                       window, 0);
}

/* Prefill over a rotated cache (fp8kv-style rotated rows, per-tensor scales). */
void oracle_paged_prefill_rotated_pairs(double* out, const int32_t* pairs, int npairs,
                                        const uint16_t* q, const int32_t* qsl, int B,
                                        const void* key_cache, const void* value_cache,
                                        int cache_dtype, const int32_t* block_tables,
                                        int max_blocks, const int32_t* context_lens, int Hq,
                                        int Hkv, int D, int bs, double k_scale, double v_scale,
                                        int window) {
    prefill_pairs_core(out, pairs, npairs, q, qsl, B, key_cache, value_cache, cache_dtype,
                       block_tables, max_blocks, context_lens, Hq, Hkv, D, bs, k_scale, v_scale,
                       window, 1);
}

/* --------------------------------------------------- Hadamard rotation --- */

/*
 * Normalized Hadamard rotation of one d-vector (d a power of two), applied to Q, K and V
 * before caching so that outliers spread across coordinates while dot products stay the
 * same; attention runs in the rotated space and its output is rotated back [ACC,
 * paragraph on the llama.cpp rotation merged 2026-04-01].  The Sylvester Hadamard matrix
 * is symmetric and, divided by sqrt(d), orthonormal, so the same transform rotates back.
 *
 * f32 form (the one the quantised codes are defined by, so that a code decision is taken
 * in f32 on both sides): the fast Walsh-Hadamard butterflies in the order
 * h = 1, 2, 4, ..., d/2 -- each pair (x[i], x[i+h]) of a 2h-block becomes
 * (x[i] + x[i+h], x[i] - x[i+h]), one f32 rounding each -- then every element times the
 * f32 constant (float)(1/sqrt(d)).
 */
void oracle_hadamard_f32(float* x, int d) {
    for (int h = 1; h < d; h *= 2)
        for (int i = 0; i < d; i += 2 * h)
            for (int j = i; j < i + h; ++j) {
                float a = x[j], b = x[j + h];
                x[j] = a + b;
                x[j + h] = a - b;
            }
    float c = (float)(1.0 / sqrt((double)d));
    for (int i = 0; i < d; ++i) x[i] = x[i] * c;
}

/* fp64 form, for the attention oracle: the same butterflies and 1/sqrt(d) in double. */
void oracle_hadamard_f64(double* x, int d) {
    for (int h = 1; h < d; h *= 2)
        for (int i = 0; i < d; i += 2 * h)
            for (int j = i; j < i + h; ++j) {
                double a = x[j], b = x[j + h];
                x[j] = a + b;
                x[j + h] = -b + a;             /* (the same value as a - b) */
            }
    double c = 1.0 / sqrt((double)d);
    for (int i = 0; i < d; ++i) x[i] *= c;
}

/* An f32 value divided by the scale in f32 and cast once to e4m3 (the quantiser of
 * oracle_quantize, for an input that is already f32). */
static uint8_t quantize_f32(float y, float scale) {
    float q = y / scale;
    return oracle_e4m3_encode((double)q);
}

/* bf16 nearest to an f32 (round to nearest, ties to even; NaN kept quiet). */
static uint16_t f32_to_bf16(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x0040u);
    uint32_t r = u + 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(r >> 16);
}

/*
 * Rotated cache write: each K and V row (d elements of one token and kv head) is widened
 * to f32, rotated by oracle_hadamard_f32, then quantised exactly as oracle_cache_write
 * quantises (e4m3 cache) or rounded to bf16 (bf16 cache).  k_scales / v_scales: one scale
 * per kv head (the per-attention-head granularity of "FP8 KV Cache Quantization: Capacity
 * Gains and Accuracy Risk", "Scales and calibration"), or null for k_scale / v_scale.
 */
static void cache_write_rotated_core(const uint16_t* key, const uint16_t* value,
                                     void* key_cache, void* value_cache, int cache_dtype,
                                     const int64_t* slot_mapping, int T, int Hkv, int D, int bs,
                                     int NB, float k_scale, float v_scale, const float* k_scales,
                                     const float* v_scales) {
    float* rk = (float*)malloc(sizeof(float) * (size_t)D);
    float* rv = (float*)malloc(sizeof(float) * (size_t)D);
    for (int t = 0; t < T; ++t) {
        int64_t slot = slot_mapping[t];
        if (slot < 0 || slot >= (int64_t)NB * bs) continue;
        int64_t blk = slot / bs;
        int in_block = (int)(slot % bs);
        for (int h = 0; h < Hkv; ++h) {
            for (int i = 0; i < D; ++i) {
                rk[i] = oracle_bf16_to_f32(key[((int64_t)t * Hkv + h) * D + i]);
                rv[i] = oracle_bf16_to_f32(value[((int64_t)t * Hkv + h) * D + i]);
            }
            oracle_hadamard_f32(rk, D);
            oracle_hadamard_f32(rv, D);
            for (int i = 0; i < D; ++i) {
                int64_t ki = key_index(blk, h, in_block, i, Hkv, bs, D,
                                       cache_dtype == ORACLE_CACHE_BF16 ? 2 : 1);
                int64_t vi = value_index(blk, h, in_block, i, Hkv, bs, D);
                if (cache_dtype == ORACLE_CACHE_E4M3) {
                    ((uint8_t*)key_cache)[ki] = quantize_f32(rk[i], k_scales ? k_scales[h] : k_scale);
                    ((uint8_t*)value_cache)[vi] = quantize_f32(rv[i], v_scales ? v_scales[h] : v_scale);
                } else {
                    ((uint16_t*)key_cache)[ki] = f32_to_bf16(rk[i]);
                    ((uint16_t*)value_cache)[vi] = f32_to_bf16(rv[i]);
                }
            }
        }
    }
    free(rk);
    free(rv);
}

void oracle_cache_write_rotated(const uint16_t* key, const uint16_t* value,
                                void* key_cache, void* value_cache, int cache_dtype,
                                const int64_t* slot_mapping, int T, int Hkv, int D, int bs,
                                int NB, float k_scale, float v_scale) {
    cache_write_rotated_core(key, value, key_cache, value_cache, cache_dtype, slot_mapping, T,
                             Hkv, D, bs, NB, k_scale, v_scale, NULL, NULL);
}

void oracle_cache_write_rotated_per_head(const uint16_t* key, const uint16_t* value,
                                         void* key_cache, void* value_cache, int cache_dtype,
                                         const int64_t* slot_mapping, int T, int Hkv, int D,
                                         int bs, int NB, const float* k_scales,
                                         const float* v_scales) {
    cache_write_rotated_core(key, value, key_cache, value_cache, cache_dtype, slot_mapping, T,
                             Hkv, D, bs, NB, 1.0f, 1.0f, k_scales, v_scales);
}

/*
 * Decode over a rotated cache: the query row is rotated (fp64), attention runs over the
 * dequantised rotated rows exactly as oracle_paged_decode_head, and the output is rotated
 * back (fp64).  Selected (b, hq) pairs, out double [n][D].
 */
void oracle_paged_decode_rotated_pairs(double* out, const int32_t* pairs, int npairs,
                                       const uint16_t* q, const void* key_cache,
                                       const void* value_cache, int cache_dtype,
                                       const int32_t* block_tables, int max_blocks,
                                       const int32_t* context_lens, int Hq, int Hkv, int D,
                                       int bs, double k_scale, double v_scale, int window) {
    int g = Hq / Hkv;
    int eb = cache_dtype == ORACLE_CACHE_BF16 ? 2 : 1;
    double* qr = (double*)malloc(sizeof(double) * (size_t)D);
    for (int p = 0; p < npairs; ++p) {
        int b = pairs[2 * p], hq = pairs[2 * p + 1];
        int kvh = hq / g;
        int64_t L = context_lens[b];
        int64_t lo = 0;                          /* window: the last W positions */
        if (window > 0 && L > window) lo = L - window;
        int64_t n = L > lo ? L - lo : 0;
        double* K = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1) * D);
        double* V = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1) * D);
        for (int i = 0; i < D; ++i)
            qr[i] = (double)oracle_bf16_to_f32(q[((int64_t)b * Hq + hq) * D + i]);
        oracle_hadamard_f64(qr, D);
        for (int64_t j = lo; j < L; ++j) {
            int64_t pb = block_tables[(int64_t)b * max_blocks + j / bs];
            int in_block = (int)(j % bs);
            for (int i = 0; i < D; ++i) {
                K[(j - lo) * D + i] = cache_value(key_cache, cache_dtype,
                                                  key_index(pb, kvh, in_block, i, Hkv, bs, D, eb),
                                                  k_scale);
                V[(j - lo) * D + i] = cache_value(value_cache, cache_dtype,
                                                  value_index(pb, kvh, in_block, i, Hkv, bs, D),
                                                  v_scale);
            }
        }
        double* o = out + (int64_t)p * D;
        oracle_attention_rows(o, qr, K, V, n, D);
        oracle_hadamard_f64(o, D);              /* back to the original coordinates */
        free(K);
        free(V);
    }
    free(qr);
}

/*
 * Decode over a rotated cache with one (k, v) scale pair per kv head: each pair decoded as
 * oracle_paged_decode_rotated_pairs decodes it, with its kv head's two scales.
 */
void oracle_paged_decode_rotated_pairs_per_head(double* out, const int32_t* pairs, int npairs,
                                                const uint16_t* q, const void* key_cache,
                                                const void* value_cache, int cache_dtype,
                                                const int32_t* block_tables, int max_blocks,
                                                const int32_t* context_lens, int Hq, int Hkv,
                                                int D, int bs, const double* k_scales,
                                                const double* v_scales, int window) {
    int group = Hq / Hkv;
    for (int p = 0; p < npairs; ++p) {
        int kvh = pairs[2 * p + 1] / group;
        oracle_paged_decode_rotated_pairs(out + (int64_t)p * D, pairs + 2 * p, 1, q, key_cache,
                                          value_cache, cache_dtype, block_tables, max_blocks,
                                          context_lens, Hq, Hkv, D, bs, k_scales[kvh],
                                          v_scales[kvh], window);
    }
}
