// paged_prefill.hip -- prefill / chunked-prefill attention over the paged fp8 (or bf16) KV
// cache.
//
// What is computed (header fp8kv.h has the exact definition): the chunk of n_b new query
// tokens of sequence b sits at the last n_b positions of its context; the token at
// position p attends causally to the cached positions [lo(p), p] (lo = p + 1 - W under a
// sliding window W), K and V dequantised inside the kernel (page "FP8 KV Cache
// Quantization: Capacity Gains and Accuracy Risk", "Attention backend interactions"),
// query head hq reading kv head hq / g (page "ctx-fp8-kv-cache-long-context-accuracy",
// "Arithmetic intensity").  Prefill is the pass whose contraction runs over the whole
// context, so it keeps the two-level accumulation of page "The State of FP8 KV-Cache and
// Attention Quantization in vLLM", "ACCURACY AT LONG CONTEXT": the matrix-core
// accumulator sums at most kFlushSteps key steps, then its partial sums move into plain
// fp32 registers.
//
// Work mapping.  A query "column" is one (chunk token, query head of the group) pair; the
// columns of a (sequence, kv head) are numbered token-major, head fastest, so the g heads
// of one token -- which read the same keys -- sit side by side.  A workgroup of 4 waves
// owns 128 consecutive columns of one (sequence, kv head); each wave owns 32 and walks
// the keys its columns need, 32 tokens (two cache blocks) per step, straight from the
// paged cache (no LDS staging: a step's K and V bytes are read once per wave, and the
// waves and workgroups of one kv head share them through the L2).  Both products run on
// v_mfma_f32_32x32x16_bf16:
//   S = K.Q^T : A = 32 key rows x 16 channels, B = 16 channels x 32 columns.  The result
//               lands with lane l holding column l%32 and 16 key rows, so the softmax
//               max and sum of a column stay inside the lane pair (l, l^32).  Key row r
//               reads token tau(r) = r with bits 2 and 3 swapped: that makes the 8
//               probabilities a lane feeds to P.V tokens 8h..8h+7 of one block (h = l/32).
//               Each lane reads half of its key row's channels, as the key tile's
//               16-byte chunks of quarters 2h and 2h+1; the query operand follows the
//               same channel order.
//   O += P.V  : A = 32 columns x 16 tokens (the lane's own probabilities, as a high and a
//               low bf16 term: two products), B = 16 tokens x 32 channels: lane l reads
//               the 8 (or 16, bf16)
//               contiguous bytes of channel l%32's row in the channel-major value tile
//               that hold tokens 8h..8h+7 -- no transpose.
// One-byte codes (E4M3, E5M2, INT8) become bf16 exactly.  Scores are kept in base-2
// units (k_scale log2(e)/sqrt(d) folded into one multiply); v_scale multiplies the final
// normalisation.  The running maximum of a column is only moved when a score exceeds it
// by 2^8, so probabilities stay below 256 and the accumulators are rarely rescaled.
#include <type_traits>

#include "codec.h"
#include "internal.h"

namespace fp8kv {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef const __attribute__((address_space(4))) int32_t* ConstI32Ptr;

constexpr int kWaves = 4;
constexpr int kCols = 32;                  // query columns per wave
constexpr int kStep = 32;                  // key tokens per wave step (two cache blocks)
constexpr int kFlushSteps = 8;             // key steps summed in the matrix-core accumulator
constexpr float kRescaleLog2 = 8.0f;

__device__ inline bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ inline f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// First channel of the 8 channels a lane of half h feeds to contraction slice kk of the
// S product (see the key layout in internal.h: the lane reads quarters 2h and 2h+1).
template <int D, int ES>
__device__ constexpr int key_slice_channel(int h, int kk) {
    if constexpr (ES == 1)      // a 16-byte chunk holds 16 channels: two slices
        return (2 * h + (kk % 4) / 2) * (D / 4) + 16 * (kk / 4) + 8 * (kk % 2);
    else                        // a 16-byte chunk holds 8 channels: one slice
        return (2 * h + kk % 2) * (D / 4) + 8 * (kk / 2);
}

// Key row r of a step reads token tau(r): bits 2 and 3 of r swapped.
__device__ inline int key_token(int r) { return (r & 0x13) | ((r & 4) << 1) | ((r & 8) >> 1); }

__device__ inline void store_out(void* out, int out_f32, int64_t idx, float v) {
    if (out_f32)
        static_cast<float*>(out)[idx] = v;
    else
        static_cast<__bf16*>(out)[idx] = (__bf16)v;   // round to nearest even
}

// Compensated add (Knuth's TwoSum) of x into (hi, lo).
__device__ inline void comp_add(float& hi, float& lo, float x) {
    const float s = hi + x;
    const float bp = s - hi;
    const float ap = s - bp;
    lo += (hi - ap) + (x - bp);
    hi = s;
}

// C: the cache codec (kCodecBF16, or a one-byte codec: E4M3, E5M2, INT8).
template <int D, int C>
__global__ __launch_bounds__(64 * kWaves) void prefill_kernel(PrefillParams p) {
    constexpr bool FP8 = C != kCodecBF16;  // one-byte codes
    constexpr int ES = FP8 ? 1 : 2;
    constexpr int NK = D / 16;             // contraction slices of S (16 channels each)
    constexpr int NT = D / 32;             // 32-channel output tiles of O
    constexpr int TILE = kBlockSize * D * ES;   // bytes of one (block, kv head) tile
    constexpr int NV = TILE / 64 / 16;     // 16-byte pieces per lane of one staged tile
    // a staged step: key tiles of its two blocks, then their value tiles
    __shared__ __attribute__((aligned(16))) uint8_t sm_kv[2][4 * TILE];
    __shared__ float sm_f[kWaves][kCols];

    const int lane = threadIdx.x & 63;
    // wave-uniform (kept in a scalar register: block ids then come from scalar loads, whose
    // waits do not drain the vector loads in flight)
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int col = lane & 31;             // this lane's query column (S layout)
    const int half = lane >> 5;            // contraction half
    const int h = blockIdx.y;              // kv head
    const int b = blockIdx.z;
    const int G = p.num_q_heads / p.num_kv_heads;

    const int q0 = ((ConstI32Ptr)p.query_start_loc)[b];
    const int nq = ((ConstI32Ptr)p.query_start_loc)[b + 1] - q0;       // chunk tokens
    const int tile = (int)gridDim.x - 1 - (int)blockIdx.x;             // heaviest tiles first
    const int64_t ncols = (int64_t)(nq > 0 ? nq : 0) * G;
    const int64_t cw0 = (int64_t)tile * (kWaves * kCols);             // first column of the workgroup
    if (cw0 >= ncols) return;                                         // (whole workgroup)
    const int64_t c0 = cw0 + wave * kCols;                            // first column of the wave
    const bool wactive = c0 < ncols;

    int L = ((ConstI32Ptr)p.context_lens)[b];
    if (L > p.max_context_len) L = p.max_context_len;
    if (L > p.max_blocks_per_seq * kBlockSize) L = p.max_blocks_per_seq * kBlockSize;
    if (L < 0) L = 0;
    const int W = p.sliding_window;
    auto lo_of = [&](int pos) { return (W > 0 && pos + 1 > W) ? pos + 1 - W : 0; };

    // this lane's column
    const int64_t cg = c0 + col;
    const bool cvalid = cg < ncols;
    const int tok = cvalid ? (int)(cg / G) : 0;
    const int hq = h * G + (cvalid ? (int)(cg % G) : 0);
    const int pos = L - nq + tok;          // < 0: the column attends to nothing
    const int clo = lo_of(pos);

    // key ranges: the workgroup stages [lo of its first position, its last position]; a
    // wave computes only the steps its own columns can see
    const int64_t cwlast = (cw0 + kWaves * kCols <= ncols ? cw0 + kWaves * kCols : ncols) - 1;
    const int pwmin = L - nq + (int)(cw0 / G);
    const int kend = L - nq + (int)(cwlast / G) + 1;                  // exclusive, <= L
    const int kfirst = pwmin >= 0 ? (lo_of(pwmin) / kStep) * kStep : 0;
    const int nsteps = kend > kfirst ? (kend - kfirst + kStep - 1) / kStep : 0;
    const int64_t clast = wactive ? (c0 + kCols <= ncols ? c0 + kCols : ncols) - 1 : c0;
    const int pmin = L - nq + (int)(c0 / G);
    const int pmax = L - nq + (int)(clast / G);
    const int lomax = lo_of(pmax);
    const int lomin = lo_of(pmin);

    // query operand of S: slice kk = q[hq][key_slice_channel(half, kk) .. +8)
    bf16x8 qb[NK];
    {
        const uint16_t* qrow = p.query + ((int64_t)(q0 + tok) * p.num_q_heads + hq) * D;
#pragma unroll
        for (int kk = 0; kk < NK; ++kk) {
            u32x4 v = {0u, 0u, 0u, 0u};
            if (cvalid && pos >= 0)
                v = *reinterpret_cast<const u32x4*>(qrow + key_slice_channel<D, ES>(half, kk));
            qb[kk] = as_bf16x8(v);
        }
    }

    const float kscale = p.k_scales != nullptr
                             ? ((const __attribute__((address_space(4))) float*)p.k_scales)[h]
                             : 1.0f;
    const float sscale = p.score_scale * kscale;
    const ConstI32Ptr bt = (ConstI32Ptr)(p.block_tables + (int64_t)b * p.max_blocks_per_seq);

    // block c of the step at kb: valid id, or -1 (past the table, outside [0, num_blocks),
    // or starting at or after kend)
    auto block_of = [&](int kb, int c) {
        const int n = kb / kBlockSize + c;
        const int id = n < p.max_blocks_per_seq ? bt[n] : -1;
        return (id >= 0 && id < p.num_blocks && kb + c * kBlockSize < kend) ? id : -1;
    };

    // ---- staging: wave w moves piece w of a step (key block 0, key block 1, value block 0,
    // value block 1).  The loads are always issued (a missing block or a step past the end
    // reads block 0 of the cache, in bounds) so that no branch sits between a load and
    // its use; missing blocks become zeros and value slots at or past kend are zeroed when
    // the piece is written to LDS, where the wait for the data happens anyway.
    const int part_c = wave & 1;
    const bool part_v = wave >= 2;
    const uint8_t* part_src = static_cast<const uint8_t*>(part_v ? p.value_cache : p.key_cache);
    auto stage_load = [&](int st, u32x4 (&r)[NV]) {
        const int kb = kfirst + (st < nsteps ? st : 0) * kStep;
        const int id = block_of(kb, part_c);
        const uint8_t* src = part_src + ((int64_t)(id >= 0 ? id : 0) * p.num_kv_heads + h) * TILE +
                             lane * (NV * 16);
#pragma unroll
        for (int i = 0; i < NV; ++i)
            r[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + 16 * i));
    };
    auto stage_store = [&](int buf, int st, const u32x4 (&r)[NV]) {
        const int kb = kfirst + st * kStep;
        const bool ok = block_of(kb, part_c) >= 0;
        // value slots kept: a 16-byte piece holds 16 slots (fp8) or 8 slots (bf16) of one row
        const int nvalid = part_v ? kend - (kb + part_c * kBlockSize) : kBlockSize;
        uint8_t* dst = &sm_kv[buf][wave * TILE + lane * (NV * 16)];
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            u32x4 v = r[i];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                uint32_t m = ok ? 0xFFFFFFFFu : 0u;
#pragma unroll
                for (int k = 0; k < 4 / ES; ++k) {
                    const int slot = ((lane * NV + i) * (16 / ES) + e * (4 / ES) + k) % kBlockSize;
                    if (slot >= nvalid) m &= ~((ES == 1 ? 0xFFu : 0xFFFFu) << (8 * ES * k));
                }
                v[e] &= m;
            }
            *reinterpret_cast<u32x4*>(dst + 16 * i) = v;
        }
    };

    f32x16 oacc[NT], osum[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        oacc[t] = f32x16{};
        osum[t] = f32x16{};
    }
    float mref = -INFINITY;                // running reference maximum of this column
    float l_hi = 0.0f, l_lo = 0.0f;        // sum of this lane's half of the probabilities
    int flush = 0;

    // rescale the O rows (columns 8j + 4*half + i) by the per-column factors in sm_f
    auto rescale_rows = [&](float f) {
        if (half == 0) sm_f[wave][col] = f;
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        float fr[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) fr[r] = sm_f[wave][(r / 4) * 8 + 4 * half + (r % 4)];
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                oacc[t][r] *= fr[r];
                osum[t][r] *= fr[r];
            }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
    };

    const int kt = key_token(col);         // token (within the step) of this lane's key row
    // one step of the wave from staged buffer `buf`
    // whether step st holds any key this wave's columns attend to
    auto visible = [&](int st) {
        const int kb = kfirst + st * kStep;
        return st < nsteps && wactive && kb <= pmax && kb + kStep > lomin;
    };
    // S = K.Q^T of the step staged in buffer `buf`
    auto s_product = [&](int buf) {
        const uint8_t* sk = sm_kv[buf];
        // ---- S = K.Q^T, as two independent accumulator chains (even and odd slices) up to
        // head_dim 128
        f32x16 s;
        {
            f32x16 s0 = f32x16{}, s1 = f32x16{};
            const uint8_t* ktile = sk + (kt / kBlockSize) * TILE;
            const int slot = kt % kBlockSize;
            if constexpr (ES == 1) {
#pragma unroll
                for (int kk = 0; kk < NK; kk += 2) {
                    const u32x4 v = *reinterpret_cast<const u32x4*>(
                        ktile + key_chunk_offset<D, 1>(slot, key_slice_channel<D, 1>(half, kk)));
                    s0 = mfma32(codes8_to_bf16x8<C>(v[0], v[1]), qb[kk], s0);
                    if constexpr (D <= 128)
                        s1 = mfma32(codes8_to_bf16x8<C>(v[2], v[3]), qb[kk + 1], s1);
                    else    // (head_dim 256: one chain, to stay within the registers)
                        s0 = mfma32(codes8_to_bf16x8<C>(v[2], v[3]), qb[kk + 1], s0);
                }
            } else {
#pragma unroll
                for (int kk = 0; kk < NK; kk += 2) {
                    const u32x4 v0 = *reinterpret_cast<const u32x4*>(
                        ktile + key_chunk_offset<D, 2>(slot, key_slice_channel<D, 2>(half, kk)));
                    const u32x4 v1 = *reinterpret_cast<const u32x4*>(
                        ktile + key_chunk_offset<D, 2>(slot, key_slice_channel<D, 2>(half, kk + 1)));
                    s0 = mfma32(as_bf16x8(v0), qb[kk], s0);
                    if constexpr (D <= 128)
                        s1 = mfma32(as_bf16x8(v1), qb[kk + 1], s1);
                    else
                        s0 = mfma32(as_bf16x8(v1), qb[kk + 1], s0);
                }
            }
            if constexpr (D <= 128)
                s = s0 + s1;
            else
                s = s0;
        }
        return s;
    };
    // softmax update and O += P.V of step st, whose scores are s, staged in buffer `buf`
    auto finish = [&](int st, f32x16 s, int buf) {
        const int kb = kfirst + st * kStep;
        const bool bok0 = block_of(kb, 0) >= 0, bok1 = block_of(kb, 1) >= 0;
        const uint8_t* sk = sm_kv[buf];

        // ---- raw scores masked outside [clo, pos] and outside valid blocks; the base-2
        // scale (> 0) is applied to the maximum and inside the exponent's FMA
        const bool edge = kb + kStep > pmin + 1 || kb < lomax || !bok0 || !bok1;
        float mx = -INFINITY;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float v = s[r];
            if (edge) {
                const int tr = key_token((r / 4) * 8 + 4 * half + (r % 4));
                const int kp = kb + tr;
                const bool ok = kp >= clo && kp <= pos && (tr < kBlockSize ? bok0 : bok1);
                v = ok ? v : -INFINITY;
            }
            s[r] = v;
            mx = fmaxf(mx, v);
        }
        mx = fmaxf(mx, __shfl_xor(mx, 32)) * sscale;
        // lazy reference move: only when a score exceeds it by 2^8 (or on the first keys)
        const bool move = mx > mref + kRescaleLog2;
        if (__ballot(move) != 0) {
            const float f = move ? (mref == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(mref - mx)) : 1.0f;
            if (move) {
                mref = mx;
                l_hi *= f;
                l_lo *= f;
            }
            rescale_rows(f);
        }
        const float mu = mref == -INFINITY ? 0.0f : mref;

        // ---- probabilities as the sum of two bf16 terms (about 16 significant bits: one
        // bf16 term alone moves a weighted average by up to 2^-9 of the value spread)
        // (the high term is pf truncated to bf16, so pf - hi is exact; the low term is
        // that remainder rounded to bf16)
        bf16x8 pa[2], pb[2];
        float psum = 0.0f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const float pf = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], sscale, -mu));
            const float hf = __uint_as_float(__float_as_uint(pf) & 0xFFFF0000u);
            pa[r / 8][r % 8] = __builtin_bit_cast(__bf16, (uint16_t)(__float_as_uint(pf) >> 16));
            pb[r / 8][r % 8] = (__bf16)(pf - hf);
            psum += pf;
        }
        comp_add(l_hi, l_lo, psum);

        // ---- O += P.V: chunk c = block c of the step, lane reads tokens 8*half .. +7
        // (value slots past the context were zeroed when staged)
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            const uint8_t* vtile = sk + (2 + c) * TILE;
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                const int ch = 32 * t + col;
                bf16x8 vb;
                if constexpr (ES == 1) {
                    const u32x2 v = *reinterpret_cast<const u32x2*>(vtile + ch * kBlockSize + 8 * half);
                    vb = codes8_to_bf16x8<C>(v[0], v[1]);
                } else {
                    vb = as_bf16x8(*reinterpret_cast<const u32x4*>(vtile + (ch * kBlockSize + 8 * half) * 2));
                }
                oacc[t] = mfma32(pa[c], vb, oacc[t]);
                oacc[t] = mfma32(pb[c], vb, oacc[t]);
            }
        }

        // ---- second level: move the matrix-core partial sums into fp32 registers
        if (++flush == kFlushSteps) {
            flush = 0;
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                osum[t] += oacc[t];
                oacc[t] = f32x16{};
            }
        }
    };
    auto compute = [&](int st, int buf) {
        if (visible(st)) finish(st, s_product(buf), buf);
    };

    if constexpr (D <= 128) {
        // ---- the pipeline: step s+2 is loaded into registers while step s is computed
        // from one LDS buffer and step s+1 is written into the other; one barrier per step
        u32x4 ra[NV], rb[NV];
        stage_load(0, ra);
        stage_load(1, rb);
        stage_store(0, 0, ra);
        __syncthreads();
        for (int st = 0; st < nsteps; st += 2) {
            stage_load(st + 2, ra);
            compute(st, 0);
            stage_store(1, st + 1, rb);
            __syncthreads();
            if (st + 1 >= nsteps) break;
            stage_load(st + 3, rb);
            compute(st + 1, 1);
            stage_store(0, st + 2, ra);
            __syncthreads();
        }
    } else {
        // ---- head_dim 256 (twice the accumulators): one register set, step s+1 loaded
        // while step s is computed
        u32x4 ra[NV];
        stage_load(0, ra);
        for (int st = 0; st < nsteps; ++st) {
            stage_store(st & 1, st, ra);
            __syncthreads();
            stage_load(st + 1, ra);
            compute(st, st & 1);
        }
    }
    if (!wactive) return;
#pragma unroll
    for (int t = 0; t < NT; ++t) osum[t] += oacc[t];

    // ---- normalise: the column's probability sum over both halves, then v_scale / l
    float l_tot = l_hi + l_lo;
    l_tot += __shfl_xor(l_tot, 32);
    const float vscale = p.v_scales != nullptr
                             ? ((const __attribute__((address_space(4))) float*)p.v_scales)[h]
                             : p.v_scale;
    const float inv = l_tot > 0.0f ? vscale / l_tot : 0.0f;   // no attended key: zero row
    if (half == 0) sm_f[wave][col] = inv;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int orow = (r / 4) * 8 + 4 * half + (r % 4);    // the column this row holds
        const int64_t oc = c0 + orow;
        if (oc >= ncols) continue;
        const float f = sm_f[wave][orow];
        const int otok = (int)(oc / G);
        const int ohq = h * G + (int)(oc % G);
        const int64_t base = ((int64_t)(q0 + otok) * p.num_q_heads + ohq) * D;
#pragma unroll
        for (int t = 0; t < NT; ++t) store_out(p.out, p.out_f32, base + 32 * t + col, osum[t][r] * f);
    }
}

template <int D>
hipError_t launch_d(const PrefillParams& p, Codec codec, hipStream_t s) {
    const int G = p.num_q_heads / p.num_kv_heads;
    const int64_t tiles = ((int64_t)p.max_query_len * G + kWaves * kCols - 1) / (kWaves * kCols);
    if (tiles <= 0 || p.num_seqs <= 0) return hipSuccess;
    if (tiles > 0x7FFFFFFF || p.num_seqs > 65535 || p.num_kv_heads > 65535) return hipErrorInvalidValue;
    const void* fn;
    switch (codec) {
        case kCodecE4M3: fn = reinterpret_cast<const void*>(&prefill_kernel<D, kCodecE4M3>); break;
        case kCodecBF16: fn = reinterpret_cast<const void*>(&prefill_kernel<D, kCodecBF16>); break;
        case kCodecE5M2: fn = reinterpret_cast<const void*>(&prefill_kernel<D, kCodecE5M2>); break;
        case kCodecINT8: fn = reinterpret_cast<const void*>(&prefill_kernel<D, kCodecINT8>); break;
        default: return hipErrorInvalidValue;
    }
    return launch_kernel(fn, dim3((unsigned)tiles, p.num_kv_heads, p.num_seqs), dim3(64 * kWaves),
                         0, s, p);
}

}  // namespace

hipError_t launch_prefill(const PrefillParams& p, Codec codec, int head_dim, hipStream_t s) {
    switch (head_dim) {
        case 64: return launch_d<64>(p, codec, s);
        case 128: return launch_d<128>(p, codec, s);
        case 256: return launch_d<256>(p, codec, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace fp8kv
