// paged_decode.hip -- GQA decode attention that reads the paged fp8 (or bf16) KV cache.
//
// What is computed (header fp8kv.h has the exact definition): for each sequence and
// query head, softmax(q.K^T/sqrt(d)).V over the positions [lo, L) of the sequence's
// context, K and V dequantised inside the kernel (page "FP8 KV Cache Quantization:
// Capacity Gains and Accuracy Risk", "Attention backend interactions"), grouped-query
// heads sharing one kv head (page "ctx-fp8-kv-cache-long-context-accuracy",
// "Arithmetic intensity").  The context is cut into fixed-size splits whose fp32
// partials (m, l, acc) are merged by log-sum-exp in a second pass.
//
// Two-level accumulation (page "The State of FP8 KV-Cache and Attention Quantization in
// vLLM", "ACCURACY AT LONG CONTEXT": long contractions need partial sums moved out of
// the matrix-core accumulator into real fp32 registers).  Here the matrix-core
// accumulator only ever sums a bounded chunk of tokens (kFlushSteps wave steps); each
// chunk is then added into a running fp32 pair (hi, lo) with an error-free TwoSum, and
// the split partials are merged with the same compensated sum.  The rounding error of
// the result therefore does not grow with the context length.
//
// Work mapping (pass 1).  A workgroup of 4 waves owns one (split, kv head, sequence).
// Each wave step covers 4 consecutive cache blocks = 64 tokens, and both products run on
// the gfx950 matrix cores as v_mfma_f32_16x16x32_bf16 with the query group padded to 16
// columns:
//   S = K.q^T : A = 16 key rows x 32 channels, B = 32 channels x 16 heads.  Lane l
//               (n = l%16, grp = l/16) feeds key row n = (block n/4, token 4s + n%4), so
//               the 16x16 result lands with lane l holding scores of block grp, tokens
//               4s..4s+3, head n; over s = 0..3 a lane owns all 16 tokens of one block.
//               The 32-channel contraction slot of lane group grp is channels
//               [grp*D/4 + 8kk, +8); key tiles are stored so that the 16-byte pieces
//               one load instruction needs from a tile are 256 contiguous bytes.
//   O += P.V  : A = 16 heads x 32 tokens (the lane's own probabilities), B = 32 tokens x
//               16 channels.  The contraction slot of lane group grp is (block grp,
//               tokens 8u..8u+7), exactly the 8 value bytes that one channel row of a
//               channel-major value tile holds there, so each lane loads one 16-byte row
//               per 16-channel output tile and no LDS transpose is needed.
// One-byte codes (E4M3, and the E5M2 / INT8 variants) become bf16 exactly with the native
// gfx950 conversions (INT8 through f32); k_scale/sqrt(d)*log2(e) scales the fp32 scores and v_scale is applied at
// the final normalisation, since the hardware's scaled conversions only take powers of 2.
//
// Memory pipeline: the KV stream is read once, so it uses nontemporal 16-byte loads.  The
// next step's key rows are requested as soon as the current S product has consumed the
// key registers, and the next value rows as soon as P.V has consumed the value
// registers, so every wave keeps a step of loads in flight while it computes, without a
// second register buffer.  Block ids come from wave-uniform loads one step ahead.
#include <climits>
#include <type_traits>

#include "codec.h"
#include "hadamard.h"
#include "internal.h"

namespace fp8kv {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kFlushSteps = 4;         // wave steps summed in the matrix-core accumulator
constexpr float kRescaleLog2 = 8.0f;   // reference max moves only when a score exceeds it by 2^8
#ifndef FP8KV_CLAIM_TAIL
#define FP8KV_CLAIM_TAIL 2
#endif
constexpr int kClaimTail = FP8KV_CLAIM_TAIL;   // pool entries per workgroup claimed at the end

__device__ inline f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ inline uint4 load16(const void* p) { return *reinterpret_cast<const uint4*>(p); }

// Streaming 16-byte load (the KV cache is read once per step).
__device__ inline uint4 load16_stream(const void* p) {
    const u32x4 t = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    return make_uint4(t[0], t[1], t[2], t[3]);
}

// Knuth's TwoSum: s + e == a + b exactly (round-to-nearest, no reassociation).
__device__ inline void two_sum(float a, float b, float& s, float& e) {
    s = a + b;
    const float bp = s - a;
    const float ap = s - bp;
    e = (a - ap) + (b - bp);
}

// Add x into the compensated pair (hi, lo).
__device__ inline void comp_add(float& hi, float& lo, float x) {
    float s, e;
    two_sum(hi, x, s, e);
    hi = s;
    lo += e;
}

// Mask keeping tokens [lo, hi) of dword k of a 16-token row (element size 1 or 2 bytes).
template <int ES>
__device__ inline uint32_t token_mask_dword(int lo, int hi, int k) {
    uint32_t m = 0;
    constexpr int PER = 4 / ES;  // tokens per dword
#pragma unroll
    for (int e = 0; e < PER; ++e) {
        const int tok = k * PER + e;
        if (tok >= lo && tok < hi) m |= (ES == 1 ? 0xFFu : 0xFFFFu) << (8 * ES * e);
    }
    return m;
}

__device__ inline void store_out(void* out, int out_f32, int64_t idx, float v) {
    if (out_f32)
        static_cast<float*>(out)[idx] = v;
    else
        static_cast<__bf16*>(out)[idx] = (__bf16)v;   // round to nearest even
}

// Device-scope (relaxed atomic) store of one float.  On this chip it writes through the
// L2 of the issuing XCD to the device coherence point, so the partials need no L2
// write-back before another XCD reads them (an agent-scope release fence would write back
// the whole L2, which costs microseconds per workgroup).
__device__ inline void store_device(float* ptr, float v) {
    __hip_atomic_store(ptr, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Value of lane l ^ 1 (a DPP quad permutation: no LDS round trip).
__device__ inline float pair_swap(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false));
}

// Splits one lane of the fused merge reads (the lane pair of a channel quad covers twice
// as many), and partials it holds at once.
constexpr int kMergeLaneSplits = 32;
constexpr int kMergeLaneBatch = 16;

// Log-sum-exp merge of the `ns` split partials of the G query heads of (sequence b, kv
// head h), by one workgroup, into `out` (x v_scale / Lambda).
// Lanes 2q and 2q + 1 own channel quad q and read the even and the odd splits.  Every
// (m, l) pair of a lane and its first kMergeLaneBatch partials are requested at once (one
// round trip for up to 2 * kMergeLaneBatch splits); the pair agrees on the maximum, each
// lane forms the weights, normaliser and weighted sums of its splits, and the pair
// combines through lane swaps -- no LDS and no barrier.  The sums are plain fp32: over at
// most 2 * kMergeLaneSplits terms their relative rounding error stays below 2^-18, far
// under the bf16 rounding of the output (the merge kernel, which takes up to kMaxSplits
// partials, compensates its sums).
//
// Q passes over the quads with at most 2 * S splits (Q = 2, S = 16: group ratio 8 at
// head_dim 128; Q = 4, S = 8: group ratio 8 at head_dim 256): each lane takes all Q of its
// quads at once -- every load is issued before the first wait, unconditionally (absent
// splits read the last split and weigh 0) so the compiler can count them -- one round trip
// instead of Q.
// Two output values of head hh of the group (channels ch, ch + 1): to `out`, or -- for the
// rotated cache -- to the group's f32 rows in LDS, rotated back before they are stored.
template <bool ROT, int D>
__device__ inline void emit2(const DecodeParams& p, float* rot, int64_t hq0, int hh, int ch, float a, float b) {
    if constexpr (ROT) {
        rot[hh * D + ch] = a;
        rot[hh * D + ch + 1] = b;
    } else {
        const int64_t o = (hq0 + hh) * D + ch;
        store_out(p.out, p.out_f32, o, a);
        store_out(p.out, p.out_f32, o + 1, b);
    }
}

template <int D, int Q, int S, bool ROT>
__device__ void merge_quads(const DecodeParams& p, int64_t hq0, int NQ, int ns, float vsc, float* rot) {
    const int par = threadIdx.x & 1;
    float2 mv[Q][S];
    float4 xv[Q][S];
#pragma unroll
    for (int j = 0; j < Q; ++j) {
        const int q = min((int)(threadIdx.x >> 1) + j * 32 * kDecodeWaves, NQ - 1);
        const int hh = q / (D / 4), c4 = q % (D / 4);
        const int64_t row = (hq0 + hh) * p.splits;
        const float4* xp = reinterpret_cast<const float4*>(p.ws_acc + row * D + 4 * c4);
        const float2* mp = reinterpret_cast<const float2*>(p.ws_ml) + row;
#pragma unroll
        for (int u = 0; u < S; ++u) {
            const int sp = min(2 * u + par, ns - 1);
            mv[j][u] = mp[sp];
            xv[j][u] = xp[sp * (D / 4)];
        }
    }
#pragma unroll
    for (int j = 0; j < Q; ++j) {
        float M = -INFINITY;
#pragma unroll
        for (int u = 0; u < S; ++u) {
            if (2 * u + par >= ns) mv[j][u] = make_float2(-INFINITY, 0.0f);   // absent: weight 0
            M = fmaxf(M, mv[j][u].x);
        }
        M = fmaxf(M, pair_swap(M));
        const float Mu = (M == -INFINITY) ? 0.0f : M;
        float lam = 0.0f;
        float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int u = 0; u < S; ++u) {
            const float ws = __builtin_amdgcn_exp2f(mv[j][u].x - Mu);
            lam = fmaf(ws, mv[j][u].y, lam);
            a.x = fmaf(ws, xv[j][u].x, a.x);
            a.y = fmaf(ws, xv[j][u].y, a.y);
            a.z = fmaf(ws, xv[j][u].z, a.z);
            a.w = fmaf(ws, xv[j][u].w, a.w);
        }
        lam += pair_swap(lam);
        const float scale = lam > 0.0f ? vsc / lam : 0.0f;
        const float r0 = a.x + pair_swap(a.x), r1 = a.y + pair_swap(a.y);
        const float r2 = a.z + pair_swap(a.z), r3 = a.w + pair_swap(a.w);
        const int q = (int)(threadIdx.x >> 1) + j * 32 * kDecodeWaves;
        if (q < NQ) {
            const int hh = q / (D / 4), c4 = q % (D / 4);
            emit2<ROT, D>(p, rot, hq0, hh, 4 * c4 + 2 * par, scale * (par ? r2 : r0), scale * (par ? r3 : r1));
        }
    }
}

template <int D, bool ROT>
__device__ void merge_group(const DecodeParams& p, int b, int h, int G, int ns, float* rot) {
    const float vsc = head_scale(p.v_scales, h, p.v_scale);
    const int par = threadIdx.x & 1;
    const int NQ = G * D / 4;                                  // channel quads of the group
    const int64_t hq0 = (int64_t)b * p.num_q_heads + (int64_t)h * G;
    if (NQ > 32 * kDecodeWaves && NQ <= 64 * kDecodeWaves && ns <= 2 * kMergeLaneBatch) {
        merge_quads<D, 2, kMergeLaneBatch, ROT>(p, hq0, NQ, ns, vsc, rot);
        return;
    }
    if constexpr (D == 256) {   // one wave per SIMD: room for 4 x 8 partials per lane
        if (NQ > 64 * kDecodeWaves && NQ <= 128 * kDecodeWaves && ns <= kMergeLaneBatch) {
            merge_quads<D, 4, kMergeLaneBatch / 2, ROT>(p, hq0, NQ, ns, vsc, rot);
            return;
        }
    }
    for (int q = threadIdx.x >> 1; q < NQ; q += 32 * kDecodeWaves) {   // lane pairs of the workgroup
        const int hh = q / (D / 4), c4 = q % (D / 4);
        const int64_t row = (hq0 + hh) * p.splits;
        // one base pointer per array: the loads below differ by constant offsets
        const float4* xp = reinterpret_cast<const float4*>(p.ws_acc + (row + par) * D + 4 * c4);
        const float2* mp = reinterpret_cast<const float2*>(p.ws_ml) + row + par;
        float2 mv[kMergeLaneSplits];
        float4 xv[kMergeLaneBatch];
        auto load_x = [&](int u0) {
#pragma unroll
            for (int u = 0; u < kMergeLaneBatch; ++u) {
                xv[u] = make_float4(0.f, 0.f, 0.f, 0.f);
                if (2 * (u0 + u) + par < ns) xv[u] = xp[(u0 + u) * (D / 2)];
            }
        };
#pragma unroll
        for (int u = 0; u < kMergeLaneSplits; ++u) {
            mv[u] = make_float2(-INFINITY, 0.0f);
            if (2 * u + par < ns) mv[u] = mp[2 * u];
        }
        load_x(0);
        float M = -INFINITY;
#pragma unroll
        for (int u = 0; u < kMergeLaneSplits; ++u) M = fmaxf(M, mv[u].x);
        M = fmaxf(M, pair_swap(M));
        const float Mu = (M == -INFINITY) ? 0.0f : M;
        float lam = 0.0f;
        float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
        auto accumulate = [&](int u0) {
#pragma unroll
            for (int u = 0; u < kMergeLaneBatch; ++u) {
                const float ws = __builtin_amdgcn_exp2f(mv[u0 + u].x - Mu);   // 0 if absent
                lam = fmaf(ws, mv[u0 + u].y, lam);
                a.x = fmaf(ws, xv[u].x, a.x);
                a.y = fmaf(ws, xv[u].y, a.y);
                a.z = fmaf(ws, xv[u].z, a.z);
                a.w = fmaf(ws, xv[u].w, a.w);
            }
        };
        accumulate(0);
        if (ns > 2 * kMergeLaneBatch) {
            load_x(kMergeLaneBatch);
            accumulate(kMergeLaneBatch);
        }
        lam += pair_swap(lam);
        const float scale = lam > 0.0f ? vsc / lam : 0.0f;
        const float r0 = a.x + pair_swap(a.x), r1 = a.y + pair_swap(a.y);
        const float r2 = a.z + pair_swap(a.z), r3 = a.w + pair_swap(a.w);
        emit2<ROT, D>(p, rot, hq0, hh, 4 * c4 + 2 * par, scale * (par ? r2 : r0), scale * (par ? r3 : r1));
    }
}

// The rotated cache: the G merged f32 rows of the group, held in LDS, rotated back (D/8
// lanes per row, the butterflies of hadamard_row) and stored to `out`.  Every thread of the
// workgroup calls this (it starts with a barrier).
template <int D>
__device__ void rotate_rows_out(const DecodeParams& p, const float* rot, int G, int64_t out_row0) {
    __syncthreads();
    constexpr int CH = D / 8;
    for (int base = 0; base < G * CH; base += 64 * kDecodeWaves) {
        const int li = base + (int)threadIdx.x;           // (row, chunk) of this lane
        const int lc = li < G * CH ? li : G * CH - 1;    // clamped: every lane shuffles
        const int row = lc / CH, c = lc % CH;
        float v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = rot[row * D + c * 8 + j];
        hadamard_row<D>(v, c, p.rot_scale);
        if (li < G * CH)
#pragma unroll
            for (int j = 0; j < 8; ++j) store_out(p.out, p.out_f32, out_row0 + (int64_t)row * D + c * 8 + j, v[j]);
    }
}

// Two waves per SIMD (<= 256 registers per lane) wherever the tile fits; head_dim 256 and
// 2-byte caches need more and run one wave per SIMD.
// The variant with a second (low) query term -- the rotated query, carried as two bf16
// terms -- runs one wave per SIMD.
#ifndef FP8KV_DECODE_WPE
#define FP8KV_DECODE_WPE 0
#endif
template <int D, int C, bool QLO>
constexpr int partial_waves_per_eu() {
    if (FP8KV_DECODE_WPE > 0) return FP8KV_DECODE_WPE;
    return QLO ? 1 : ((D <= 128 && C != kCodecBF16) || D == 64 ? 2 : 1);
}

// C: the cache codec (kCodecBF16, or a one-byte codec: E4M3, E5M2, INT8).  ROT: a
// Hadamard-rotated cache; the kernel rotates the query into its two bf16 terms (so QLO),
// rotates the step token before quantising it, and rotates a merged output back.
template <int D, int C, bool QLO, bool ROT = false>
__global__ __launch_bounds__(64 * kDecodeWaves)
__attribute__((amdgpu_waves_per_eu(partial_waves_per_eu<D, C, QLO>(), 8)))
void decode_partial_kernel(DecodeParams p) {
    static_assert(!ROT || QLO, "the rotated query is carried as two bf16 terms");
    constexpr bool FP8 = C != kCodecBF16;         // one-byte codes
    constexpr int ES = FP8 ? 1 : 2;               // bytes per cache element
    constexpr int DG = D / 4;                     // channels per lane group in S = K.q^T
    constexpr int KK = D / 32;                    // MFMA k-steps for S
    constexpr int NT = D / 16;                    // 16-channel output tiles of O
    constexpr int K16 = DG * ES / 16;             // 16-byte key loads per lane per row
    constexpr int V16 = ES;                       // 16-byte value loads per lane per tile
    constexpr int TILE_BYTES = kBlockSize * D * ES;

    extern __shared__ float lds[];
    // Read every argument now, in one batch of scalar loads: left to itself the compiler
    // loads each field just before its first use, which puts several round trips to memory
    // in series before the first KV load.
    asm volatile("" :: "s"(p.out), "s"(p.query), "s"(p.key_cache), "s"(p.value_cache),
                 "s"(p.block_tables), "s"(p.context_lens), "s"(p.ws_ml), "s"(p.ws_acc));
    asm volatile("" :: "s"(p.k_new), "s"(p.v_new), "s"(p.counters), "s"(p.use_claims),
                 "s"(p.max_blocks_per_seq), "s"(p.max_context_len), "s"(p.num_q_heads),
                 "s"(p.num_kv_heads), "s"(p.num_blocks), "s"(p.sliding_window));
    asm volatile("" :: "s"(p.score_scale), "s"(p.v_scale), "s"(p.splits), "s"(p.blocks_per_split),
                 "s"(p.write_final), "s"(p.k_scale_q), "s"(p.v_scale_q), "s"(p.merge_in_kernel),
                 "s"(p.k_scales), "s"(p.v_scales), "s"(p.err),
                 "s"(p.out_f32));
    const int split = kHeadsFastest ? blockIdx.y : blockIdx.x;
    const int h = kHeadsFastest ? blockIdx.x : blockIdx.y;
    const int b = blockIdx.z;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n = lane & 15;
    const int grp = lane >> 4;
    const int G = p.num_q_heads / p.num_kv_heads;

    // The block ids of this wave's first pool step (4*split + wave) do not depend on the
    // context length when there is no sliding window (the window then starts at block 0):
    // request them together with the length, so that the first KV loads wait for one round
    // trip to memory instead of two.  They are used only if that step is the wave's first.
    typedef const __attribute__((address_space(4))) int32_t* ConstI32Ptr;
    const int st_early = kDecodeWaves * split + wave;
    int id_early[4];
    {
        const ConstI32Ptr row = (ConstI32Ptr)(p.block_tables + (int64_t)b * p.max_blocks_per_seq);
#pragma unroll
        for (int x = 0; x < 4; ++x) {
            const int i = 4 * st_early + x;
            id_early[x] = (p.sliding_window <= 0 && i < p.max_blocks_per_seq) ? row[i] : -1;
        }
    }
    // (a scalar load, like the block ids)
    const int len_in = ((ConstI32Ptr)p.context_lens)[b];
    const SeqWindow w = seq_window(len_in, p.max_context_len, p.max_blocks_per_seq, p.sliding_window);
    if (p.err != nullptr && split == 0 && h == 0 && threadIdx.x == 0 &&
        (len_in < 0 || len_in != w.L))
        report_error(p.err, kErrContextLen);
    const int ns = (w.nblk + p.blocks_per_split - 1) / p.blocks_per_split;   // workgroups taking part
    const int64_t out_row0 = ((int64_t)b * p.num_q_heads + (int64_t)h * G) * D;
    if (split >= ns) {
        // an empty context: the first split writes the zero output when no merge kernel will
        if ((p.write_final || (p.counters != nullptr && p.merge_in_kernel)) && split == 0)
            for (int i = threadIdx.x; i < G * D; i += 64 * kDecodeWaves) store_out(p.out, p.out_f32, out_row0 + i, 0.0f);
        return;
    }

    // Query group as the B operand of S = K.q^T: lane (n, grp) holds head n, channels
    // [grp*DG + 8kk, +8) for kk = 0..KK-1; heads >= G are zero columns.
    bf16x8 qop[KK];
    bf16x8 qlo[QLO ? KK : 1];                     // the query's low bf16 term (QLO only)
    if constexpr (ROT) {
        // the lane's quarter of head n's row in f32, rotated in place with the butterflies of
        // hadamard_row (h = 1, 2, ..., D/2: inside the lane for h < DG, then with the lanes
        // of groups grp ^ 1 and grp ^ 2), times (float)(1/sqrt(D)), then split into a high
        // and a low bf16 term
        const int64_t qoff = out_row0 + (int64_t)(n < G ? n : 0) * D + grp * DG;
        float x[DG];
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
            uint4 u = load16(p.query + qoff + 8 * kk);
            if (n >= G) u = make_uint4(0, 0, 0, 0);
            float f[8];
            bf16x8_to_f32(u, f);
#pragma unroll
            for (int e = 0; e < 8; ++e) x[8 * kk + e] = f[e];
        }
#pragma unroll
        for (int hh = 1; hh < DG; hh *= 2)
#pragma unroll
            for (int j = 0; j < DG; ++j)
                if ((j & hh) == 0) {
                    const float a = x[j], c = x[j + hh];
                    x[j] = a + c;
                    x[j + hh] = a - c;
                }
#pragma unroll
        for (int m = 1; m <= 2; m *= 2) {             // h = m * DG: lane groups grp and grp ^ m
            const bool upper = (grp & m) != 0;
#pragma unroll
            for (int j = 0; j < DG; ++j) {
                const float other = __shfl_xor(x[j], 16 * m);
                x[j] = upper ? other - x[j] : x[j] + other;
            }
        }
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
            uint32_t hi[4], lo[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float a = x[8 * kk + 2 * j] * p.rot_scale, c = x[8 * kk + 2 * j + 1] * p.rot_scale;
                hi[j] = pack_bf16x2(a, c);
                lo[j] = pack_bf16x2(a - __uint_as_float(hi[j] << 16), c - __uint_as_float(hi[j] & 0xFFFF0000u));
            }
            qop[kk] = __builtin_bit_cast(bf16x8, make_uint4(hi[0], hi[1], hi[2], hi[3]));
            qlo[kk] = __builtin_bit_cast(bf16x8, make_uint4(lo[0], lo[1], lo[2], lo[3]));
        }
    } else {
        // heads n >= G read head 0's row (in bounds) and are zeroed: no branch around the loads
        const int64_t qoff = out_row0 + (int64_t)(n < G ? n : 0) * D + grp * DG;
        const uint16_t* qrow = p.query + qoff;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
            uint4 u = load16(qrow + 8 * kk);
            if (n >= G) u = make_uint4(0, 0, 0, 0);
            qop[kk] = __builtin_bit_cast(bf16x8, u);
        }
        if constexpr (QLO) {
#pragma unroll
            for (int kk = 0; kk < KK; ++kk) {
                uint4 u = load16(p.query_lo + qoff + 8 * kk);
                if (n >= G) u = make_uint4(0, 0, 0, 0);
                qlo[kk] = __builtin_bit_cast(bf16x8, u);
            }
        }
    }

    const char* kcache = static_cast<const char*>(p.key_cache);
    const char* vcache = static_cast<const char*>(p.value_cache);
    // The block table is read-only while the kernel runs: reading it through the constant
    // address space lets the wave-uniform id reads below be scalar loads, which do not queue
    // behind the vector KV loads in flight.
    const ConstI32Ptr bt = (ConstI32Ptr)(p.block_tables + (int64_t)b * p.max_blocks_per_seq + w.blk0);
    const float sscale = p.score_scale * head_scale(p.k_scales, h, 1.0f);
    const int nblk = w.nblk;                      // blocks of the window
    const int nsteps = (nblk + 3) >> 2;           // wave steps (4 blocks) of the window

    // Physical ids of the 4 blocks of wave step `stp` (-1 past the window or out of range);
    // the addresses are wave-uniform.  Lanes pick their key block (n/4) and their
    // score/value block (grp).
    auto pick_ids = [&](const int* id, int& kid, int& vid) {
        const int kq = n >> 2;
        kid = kq == 0 ? id[0] : kq == 1 ? id[1] : kq == 2 ? id[2] : id[3];
        vid = grp == 0 ? id[0] : grp == 1 ? id[1] : grp == 2 ? id[2] : id[3];
        if ((unsigned)kid >= (unsigned)p.num_blocks) kid = -1;
        if ((unsigned)vid >= (unsigned)p.num_blocks) vid = -1;
    };
    // Any id of an attended block outside [0, num_blocks) (a wave-uniform flag, reported once
    // at the end; the block reads as empty).
    bool bad_id = false;
    auto note_ids = [&](const int* id, int stp) {
#pragma unroll
        for (int x = 0; x < 4; ++x)
            bad_id |= 4 * stp + x < nblk && (unsigned)id[x] >= (unsigned)p.num_blocks;
    };
    auto step_ids = [&](int stp, int& kid, int& vid) {
        int id[4];
#pragma unroll
        for (int x = 0; x < 4; ++x) id[x] = (4 * stp + x < nblk) ? bt[4 * stp + x] : -1;
        note_ids(id, stp);
        pick_ids(id, kid, vid);
    };
    // Loads are unconditional (branch-free, so the compiler can count them in flight): a
    // missing block (-1) reads block 0, which exists whenever any block can be valid, and
    // its scores are masked and its values zeroed below.  One step of loads is in flight
    // while the previous step is processed.
    struct Buf {
        uint4 k[4][K16];
        uint4 v[NT][V16];
        int kid, vid;
    };
    auto issue_k = [&](Buf& bf, int kid) {
        // lane (n, grp) reads slot 4s + n%4, channels [grp*DG, +DG) of block n/4: chunk x of
        // that row sits at key_chunk_offset(4s + n%4, grp*DG + 16x/ES)
        const char* kt = kcache + ((int64_t)max(kid, 0) * p.num_kv_heads + h) * TILE_BYTES
                         + key_chunk_offset<D, ES>(n & 3, grp * DG);
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int x = 0; x < K16; ++x) bf.k[s][x] = load16_stream(kt + (s * K16 + x) * 256);
    };
    auto issue_v = [&](Buf& bf, int vid) {
        const char* vt = vcache + ((int64_t)max(vid, 0) * p.num_kv_heads + h) * TILE_BYTES
                         + (int64_t)n * kBlockSize * ES;
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int x = 0; x < V16; ++x) bf.v[t][x] = load16_stream(vt + (int64_t)(16 * t) * kBlockSize * ES + 16 * x);
    };

    float m_use = -INFINITY;     // reference max of base-2 scores for head n
    float l_chunk = 0.0f;        // this lane's softmax sum over the current chunk
    float l_hi = 0.0f, l_lo = 0.0f;
    f32x4 acc[NT];               // matrix-core accumulator of the current chunk
    f32x4 run_hi[NT], run_lo[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
        run_hi[t] = acc[t];
        run_lo[t] = acc[t];
    }
    auto flush = [&]() {
#pragma unroll
        for (int t = 0; t < NT; ++t) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                float hs = run_hi[t][r], ls = run_lo[t][r];
                comp_add(hs, ls, acc[t][r]);
                run_hi[t][r] = hs;
                run_lo[t][r] = ls;
            }
            acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        comp_add(l_hi, l_lo, l_chunk);
        l_chunk = 0.0f;
    };

    int chunk_steps = 0;
    // One wave step over the 4 blocks of step `stp` held in `bf`; refills `bf` with step
    // `nstp` as soon as each half of the buffer has been consumed.  `steady` (a compile-time
    // tag) marks steps with a successor: their prefetch is unconditional, which keeps the
    // loads in straight-line code so the compiler can wait for exactly the loads each use
    // needs; the wave's last step (no successor) prefetches nothing.
    auto process = [&](Buf& bf, int stp, int nstp, auto steady) {
        constexpr bool kSteady = decltype(steady)::value;
        constexpr bool more = kSteady;
        int nkid = -1, nvid = -1;
        if (more) step_ids(nstp, nkid, nvid);

            // ---- S = K.q^T on the matrix cores
            f32x4 sc[4];
    #pragma unroll
            for (int s = 0; s < 4; ++s) {
                f32x4 c = {0.f, 0.f, 0.f, 0.f};
    #pragma unroll
                for (int kk = 0; kk < KK; ++kk) {
                    bf16x8 a;
                    if constexpr (FP8) {
                        const uint4 u = bf.k[s][kk >> 1];
                        a = (kk & 1) ? codes8_to_bf16x8<C>(u.z, u.w) : codes8_to_bf16x8<C>(u.x, u.y);
                    } else {
                        a = __builtin_bit_cast(bf16x8, bf.k[s][kk]);
                    }
                    c = mfma16x16x32(a, qop[kk], c);
                    if constexpr (QLO) c = mfma16x16x32(a, qlo[kk], c);
                }
                sc[s] = c;
            }
            if (more) issue_k(bf, nkid);   // key registers are free again
            // Keep the value-side work below the softmax: without this the scheduler hoists
            // the value conversions above the q.K products, and every step then waits for
            // its value loads before it can start.
            __builtin_amdgcn_sched_barrier(0);

            // ---- mask and scale: lane holds block grp of the step, tokens 4s+r, head n
            const bool vval = bf.vid >= 0;
            const int pos0 = (w.blk0 + 4 * stp + grp) * kBlockSize;
            const int tlo = vval ? max(0, w.lo - pos0) : kBlockSize;   // missing block: no tokens
            const int thi = vval ? min(kBlockSize, w.L - pos0) : 0;
            float sv[16];
            float mloc = -INFINITY;
    #pragma unroll
            for (int s = 0; s < 4; ++s)
    #pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int tok = 4 * s + r;
                    const bool ok = tok >= tlo && tok < thi;
                    const float x = ok ? sc[s][r] * sscale : -INFINITY;
                    sv[4 * s + r] = x;
                    mloc = fmaxf(mloc, x);
                }
            float mt = fmaxf(mloc, __shfl_xor(mloc, 16));
            mt = fmaxf(mt, __shfl_xor(mt, 32));
            // move the reference max only when a score exceeds it by more than 2^kRescaleLog2
            // (or on the first valid scores): p = 2^(s - m_use) then stays below 2^8
            const float m_new = (mt > m_use + kRescaleLog2 || m_use == -INFINITY) ? mt : m_use;
            if (__any(m_new != m_use)) {
                const float alpha = (m_use == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(m_use - m_new);
                float ar[4];
    #pragma unroll
                for (int r = 0; r < 4; ++r) ar[r] = __shfl(alpha, 4 * grp + r);
    #pragma unroll
                for (int t = 0; t < NT; ++t)
    #pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        acc[t][r] *= ar[r];
                        run_hi[t][r] *= ar[r];
                        run_lo[t][r] *= ar[r];
                    }
                l_chunk *= alpha;
                l_hi *= alpha;
                l_lo *= alpha;
                m_use = m_new;
            }
            const float m_ref = (m_use == -INFINITY) ? 0.0f : m_use;
            float pv[16];
            float psum = 0.0f;
    #pragma unroll
            for (int k = 0; k < 16; ++k) {
                pv[k] = __builtin_amdgcn_exp2f(sv[k] - m_ref);   // exp2(-inf) = 0
                psum += pv[k];
            }
            l_chunk += psum;

            __builtin_amdgcn_sched_barrier(0);
            // values of tokens outside [lo, L) (partial or missing blocks) are zeroed so that a
            // poisoned (NaN) slot never reaches the accumulator through p = 0
            if (tlo > 0 || thi < kBlockSize) {
    #pragma unroll
                for (int t = 0; t < NT; ++t)
    #pragma unroll
                    for (int x = 0; x < V16; ++x) {
                        bf.v[t][x].x &= token_mask_dword<ES>(tlo, thi, 4 * x + 0);
                        bf.v[t][x].y &= token_mask_dword<ES>(tlo, thi, 4 * x + 1);
                        bf.v[t][x].z &= token_mask_dword<ES>(tlo, thi, 4 * x + 2);
                        bf.v[t][x].w &= token_mask_dword<ES>(tlo, thi, 4 * x + 3);
                    }
            }

            // ---- O += P.V on the matrix cores.  p is carried as a bf16 pair hi + lo (about 16
            // significant bits): a single bf16 would cost up to 2^-9 * sum p|V| of error, which
            // short windows do not average away.  V is exact in bf16.
            bf16x8 phi[2], plo[2];
    #pragma unroll
            for (int u = 0; u < 2; ++u) {
    #pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float x = pv[8 * u + e];
                    const __bf16 hi = (__bf16)x;
                    phi[u][e] = hi;
                    plo[u][e] = (__bf16)(x - (float)hi);
                }
            }
    #pragma unroll
            for (int t = 0; t < NT; ++t) {
    #pragma unroll
                for (int u = 0; u < 2; ++u) {
                    bf16x8 vb8;
                    if constexpr (FP8) {
                        const uint4 v = bf.v[t][0];
                        vb8 = u ? codes8_to_bf16x8<C>(v.z, v.w) : codes8_to_bf16x8<C>(v.x, v.y);
                    } else {
                        vb8 = __builtin_bit_cast(bf16x8, bf.v[t][u]);
                    }
                    acc[t] = mfma16x16x32(phi[u], vb8, acc[t]);
                    acc[t] = mfma16x16x32(plo[u], vb8, acc[t]);
                }
            }
        if (more) issue_v(bf, nvid);   // value registers are free again
        bf.kid = nkid;
        bf.vid = nvid;
        if (++chunk_steps == kFlushSteps) {
            flush();
            chunk_steps = 0;
        }
    };

    // ---- which wave steps this wave processes
    // Slot `wave` of this (sequence, kv head) owns the window steps 4k + wave, k = 0, 1, ...
    // (its pool).  Workgroup `split` (of the ns taking part) takes pool entries split and
    // split + ns; after those it claims entries from the slot's counter when the caller
    // provides one -- whichever wave is free takes the next step, which evens out speed
    // differences between compute units and XCDs -- and otherwise continues statically with
    // split + 2ns, split + 3ns, ...  With a step token to write, the window's last step
    // (which holds position L-1) leaves the pools: the writer wave writes the token and
    // then processes that step first, so its own loads of the block come after its stores.
    const bool writing = p.k_new != nullptr;
    const int np = writing ? nsteps - 1 : nsteps;            // steps in the pools
    const bool writer = writing && split == 0 && wave == (nsteps - 1) % kDecodeWaves;
    auto pool_step = [&](int k) {
        const int st = kDecodeWaves * k + wave;
        return st < np ? st : -1;
    };
    unsigned int* const rec = p.counters == nullptr ? nullptr
        : p.counters + ((int64_t)b * p.num_kv_heads + h) * kCounterRecordWords;
    unsigned int* claim = rec != nullptr && p.use_claims ? rec + (1 + wave) * kCounterLineWords : nullptr;

    // Fused decode step: lanes [0, D/8) write 8 key channels of the token each, lanes
    // [32, 32 + D/8) 8 value channels.  Load and store sit in one branch: a token load left
    // pending across branches makes the compiler wait for every load in flight (the query
    // rows included) before the first KV loads of every wave.
    auto store_step_token = [&]() {
        const int tok_blk = ((ConstI32Ptr)p.block_tables)[(int64_t)b * p.max_blocks_per_seq + (w.L - 1) / kBlockSize];
        const uint4 tok = load16((lane >= 32 ? p.v_new : p.k_new) + ((int64_t)b * p.num_kv_heads + h) * D +
                                 min(lane & 31, D / 8 - 1) * 8);
        const int c = lane & 31;
        if ((unsigned)tok_blk >= (unsigned)p.num_blocks && lane == 0) report_error(p.err, kErrBlockId);
        // the rotated cache: each row (lanes [0, D/8) keys, [32, 32 + D/8) values) rotated in
        // f32 by every lane of the wave (the shuffles stay inside each half), exactly as the
        // rotated cache write does
        float rv[8];
        if constexpr (ROT) {
            bf16x8_to_f32(tok, rv);
            hadamard_row<D>(rv, c, p.rot_scale);
        }
        if ((unsigned)tok_blk < (unsigned)p.num_blocks && c < D / 8) {
            const bool val = lane >= 32;
            const int off = (w.L - 1) % kBlockSize;
            char* tile = static_cast<char*>(const_cast<void*>(val ? p.value_cache : p.key_cache))
                         + ((int64_t)tok_blk * p.num_kv_heads + h) * TILE_BYTES;
            if constexpr (ROT) {
                if constexpr (FP8) {
                    // IEEE f32 division by the head's scale, then the cast
                    const float sc = val ? head_scale(p.v_scales, h, p.v_scale_q)
                                         : head_scale(p.k_scales, h, p.k_scale_q);
                    uint32_t cw[4];
#pragma unroll
                    for (int j = 0; j < 4; ++j) cw[j] = pack2<C>(rv[2 * j] / sc, rv[2 * j + 1] / sc);
                    const uint2 q8 = make_uint2(cw[0] | (cw[1] << 16), cw[2] | (cw[3] << 16));
                    if (!val) {
                        *reinterpret_cast<uint2*>(tile + key_chunk_offset<D, 1>(off, c * 8)) = q8;
                    } else {
#pragma unroll
                        for (int i = 0; i < 8; ++i)
                            tile[(c * 8 + i) * kBlockSize + off] = (char)(((i < 4 ? q8.x : q8.y) >> (8 * (i & 3))) & 0xFF);
                    }
                } else {
                    if (!val) {
                        *reinterpret_cast<uint4*>(tile + key_chunk_offset<D, 2>(off, c * 8)) =
                            make_uint4(pack_bf16x2(rv[0], rv[1]), pack_bf16x2(rv[2], rv[3]),
                                       pack_bf16x2(rv[4], rv[5]), pack_bf16x2(rv[6], rv[7]));
                    } else {
                        uint16_t* vt16 = reinterpret_cast<uint16_t*>(tile);
#pragma unroll
                        for (int i = 0; i < 8; ++i)
                            vt16[(c * 8 + i) * kBlockSize + off] = __builtin_bit_cast(uint16_t, (__bf16)rv[i]);
                    }
                }
            } else if constexpr (FP8) {
                const uint2 q8 = quantize8<C>(tok, val ? head_scale(p.v_scales, h, p.v_scale_q)
                                                    : head_scale(p.k_scales, h, p.k_scale_q));
                if (!val) {
                    *reinterpret_cast<uint2*>(tile + key_chunk_offset<D, 1>(off, c * 8)) = q8;
                } else {
#pragma unroll
                    for (int i = 0; i < 8; ++i)
                        tile[(c * 8 + i) * kBlockSize + off] = (char)(((i < 4 ? q8.x : q8.y) >> (8 * (i & 3))) & 0xFF);
                }
            } else {
                if (!val) {
                    *reinterpret_cast<uint4*>(tile + key_chunk_offset<D, 2>(off, c * 8)) = tok;
                } else {
                    const uint32_t wd[4] = {tok.x, tok.y, tok.z, tok.w};
                    uint16_t* vt16 = reinterpret_cast<uint16_t*>(tile);
#pragma unroll
                    for (int i = 0; i < 8; ++i)
                        vt16[(c * 8 + i) * kBlockSize + off] = (uint16_t)(wd[i >> 1] >> (16 * (i & 1)));
                }
            }
        }
        // Only this wave reads the block, with loads it issues after these stores, and a
        // wave's memory operations are performed in issue order: wavefront-scope ordering
        // suffices (no wait for the stores, nor for the loads already in flight).
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        __builtin_amdgcn_wave_barrier();
    };
    // Pool entries e < e_static of this wave are static (split + e*ns).  With claim
    // counters, the last entries of the slot -- about two per workgroup, enough to absorb
    // the differences in speed that show up by the end -- are claimed instead: entry
    // e >= e_static is e_static*ns + (a claim on the slot's counter).  Claims are only used
    // at the end because each one is a device-scope atomic whose completion the step loads
    // issued before it also wait for.  A claim is requested at the end of an iteration,
    // after that step's loads, and read at the end of the next one.
    const bool dyn = claim != nullptr;
    const int slot_entries = np > wave ? (np - wave + kDecodeWaves - 1) / kDecodeWaves : 0;
    const int e_static = dyn ? max(3, slot_entries / ns - kClaimTail) : INT_MAX;
    int cur = writer ? nsteps - 1 : pool_step(split);
    int e_nxt = writer ? 0 : 1;                   // pool entry that `nxt` is
    int nxt = cur >= 0 ? pool_step(split + e_nxt * ns) : -1;
    if (cur >= 0) {
        if (writer) store_step_token();
        Buf buf;
        if (cur == st_early && p.sliding_window <= 0) {
            int id[4];
#pragma unroll
            for (int x = 0; x < 4; ++x) id[x] = (4 * cur + x < nblk) ? id_early[x] : -1;
            note_ids(id, cur);
            pick_ids(id, buf.kid, buf.vid);
        } else {
            step_ids(cur, buf.kid, buf.vid);
        }
        issue_k(buf, buf.kid);
        issue_v(buf, buf.vid);
        // Consume the query operands here, once: afterwards the compiler knows they have
        // arrived, and the loop waits only for the key or value loads each use needs
        // (without this it waits for every load in flight at the top of each step).
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) asm volatile("" ::"v"(qop[kk]));
        if constexpr (QLO) {
#pragma unroll
            for (int kk = 0; kk < KK; ++kk) asm volatile("" ::"v"(qlo[kk]));
        }
        unsigned int c_pend = 0;                  // claim for entry e_nxt + 1, when claimed
        while (nxt >= 0) {
            process(buf, cur, nxt, std::true_type{});
            // (keeps the read of the claim, and the wait for it, here)
            asm volatile("" : "+v"(c_pend));
            const int e = e_nxt + 1;
            const int k = e >= e_static ? e_static * ns + (int)__builtin_amdgcn_readfirstlane(c_pend)
                                        : split + e * ns;
            cur = nxt;
            nxt = pool_step(k);
            e_nxt = e;
            // request entry e + 1 (a wrapping increment with no reachable wrap: unlike an add,
            // the compiler does not turn it into a wave-wide form that waits for the result)
            c_pend = 0;
            if (e + 1 >= e_static && nxt >= 0 && lane == 0)
                c_pend = __builtin_amdgcn_atomic_inc32(claim, 0xFFFFFFFFu, __ATOMIC_RELAXED, "agent");
        }
        process(buf, cur, -1, std::false_type{});
    }
    flush();
    if (bad_id && lane == 0) report_error(p.err, kErrBlockId);

    // ---- combine the waves of this workgroup in LDS
    float l_tot = l_hi + l_lo;
    l_tot += __shfl_xor(l_tot, 16);
    l_tot += __shfl_xor(l_tot, 32);
    float* sm_m = lds;                           // [waves][16]
    float* sm_l = lds + kDecodeWaves * 16;       // [waves][16]
    // [waves][16][D]: every MFMA row (heads >= G are padding) is written, with no condition
    // per element -- a guard per write becomes a branch per write
    float* sm_a = lds + 2 * kDecodeWaves * 16;
    if (grp == 0) {
        sm_m[wave * 16 + n] = m_use;
        sm_l[wave * 16 + n] = l_tot;
    }
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r)
            sm_a[(wave * 16 + 4 * grp + r) * D + 16 * t + n] = run_hi[t][r] + run_lo[t][r];
    __syncthreads();

    // per head, once: the waves' weights w_v = 2^(m_v - M), the normaliser and the output
    // scale (threads 0..G-1)
    float* sm_w = lds + 2 * kDecodeWaves * 16 + kDecodeWaves * 16 * D;  // [waves][16]
    float* sm_s = sm_w + kDecodeWaves * 16;                              // [16] v_scale / Lambda
    float* sm_M = sm_s + 16;                                             // [16] M
    float* sm_L = sm_M + 16;                                             // [16] Lambda
    float* sm_rot = sm_L + 16;                                           // [16][D] rotated cache only
    if (threadIdx.x < G) {
        const int hd = threadIdx.x;
        float M = -INFINITY;
#pragma unroll
        for (int v = 0; v < kDecodeWaves; ++v) M = fmaxf(M, sm_m[v * 16 + hd]);
        const float Mu = (M == -INFINITY) ? 0.0f : M;
        float lam = 0.0f, lam_c = 0.0f;
#pragma unroll
        for (int v = 0; v < kDecodeWaves; ++v) {
            const float wv = __builtin_amdgcn_exp2f(sm_m[v * 16 + hd] - Mu);
            sm_w[v * 16 + hd] = wv;
            comp_add(lam, lam_c, wv * sm_l[v * 16 + hd]);
        }
        lam += lam_c;
        sm_s[hd] = lam > 0.0f ? head_scale(p.v_scales, h, p.v_scale) / lam : 0.0f;
        sm_M[hd] = M;
        sm_L[hd] = lam;
    }
    __syncthreads();

    for (int idx = threadIdx.x; idx < G * D; idx += 64 * kDecodeWaves) {
        const int head = idx / D;
        const int i = idx - head * D;
        float a = 0.0f, a_c = 0.0f;
#pragma unroll
        for (int v = 0; v < kDecodeWaves; ++v) comp_add(a, a_c, sm_w[v * 16 + head] * sm_a[(v * 16 + head) * D + i]);
        a += a_c;
        if (p.write_final) {
            if constexpr (ROT) sm_rot[head * D + i] = sm_s[head] * a;
            else store_out(p.out, p.out_f32, out_row0 + (int64_t)head * D + i, sm_s[head] * a);
        } else {
            const int64_t row = ((int64_t)b * p.num_q_heads + (int64_t)h * G + head) * p.splits + split;
            store_device(p.ws_acc + row * D + i, a);
            if (i == 0) {
                store_device(p.ws_ml + row * 2 + 0, sm_M[head]);
                store_device(p.ws_ml + row * 2 + 1, sm_L[head]);
            }
        }
    }
    if constexpr (ROT) {
        if (p.write_final) rotate_rows_out<D>(p, sm_rot, G, out_row0);   // (uniform branch)
    }

    // Arrival: the last workgroup of this (sequence, kv head) to finish resets the group's
    // counters for the next call and, when asked, merges the partials of all its splits.
    // No workgroup ever waits for another.
    // Ordering of the merge: the partials are device-scope stores, and every thread waits
    // until its own have completed (reached the device coherence point) before the barrier
    // after which thread 0 counts in with a device-scope atomic.  The workgroup that
    // completes the count invalidates its caches (agent-scope acquire) before any of its
    // threads reads a partial.  This is the ordering an agent-scope release/acquire pair
    // gives, without the release's L2 write-back, which only data stored through the L2
    // without device scope would need.
    if (!p.write_final && p.counters != nullptr) {
        __shared__ int s_last;
        if (p.merge_in_kernel) __builtin_amdgcn_s_waitcnt(0);   // this thread's partial stores done
        __syncthreads();                                         // ... and every thread's
        if (threadIdx.x == 0) {
            const unsigned int old = __hip_atomic_fetch_add(rec, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            const bool last = old + 1 == (unsigned int)ns;
            if (last) {
                // every wave of the group has made its last claim
                __hip_atomic_store(rec, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                if (p.use_claims)
                    for (int v = 0; v < kDecodeWaves; ++v)
                        __hip_atomic_store(rec + (1 + v) * kCounterLineWords, 0u, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
                // drop stale copies of the partials from this CU's L1 and this XCD's L2;
                // the barrier below orders the other threads' loads after it
                if (p.merge_in_kernel) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
            }
            s_last = (int)last;
        }
        __syncthreads();
        if (s_last && p.merge_in_kernel) {
            merge_group<D, ROT>(p, b, h, G, ns, sm_rot);
            if constexpr (ROT) rotate_rows_out<D>(p, sm_rot, G, out_row0);
        }
    }
}

// Pass 2: log-sum-exp merge of one (sequence, query head, 64-channel chunk) over its
// splits, with compensated sums so the merge error does not grow with the split count.
// 256 threads = 16 split lanes x 16 channel quads; each thread reads float4 partials.  The
// first kMergeBatch partials of every thread and their (m, l) are requested together,
// before the block-wide max, so a merge over up to 16 * kMergeBatch splits costs one
// round trip to memory.
constexpr int kMergeBatch = 4;

__global__ __launch_bounds__(256) void decode_merge_kernel(DecodeParams p, int D) {
    __shared__ float s_red[2][4];
    __shared__ float4 s_part[16][16][2];         // [split lane][channel quad][hi, lo]
    const int hq = blockIdx.x;
    const int b = blockIdx.y;
    const int chunk = blockIdx.z;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wv = tid >> 6;
    const int q = tid & 15;                      // channel quad: channels chunk*64 + 4q .. +3
    const int sl = tid >> 4;                     // split lane: splits sl, sl + 16, ...
    const SeqWindow w = seq_window(p.context_lens[b], p.max_context_len, p.max_blocks_per_seq,
                                   p.sliding_window);
    const int ns = (w.nblk + p.blocks_per_split - 1) / p.blocks_per_split;
    const int64_t row0 = ((int64_t)b * p.num_q_heads + hq) * p.splits;
    const float2* ml = reinterpret_cast<const float2*>(p.ws_ml) + row0;
    const float* accp = p.ws_acc + row0 * D + chunk * 64 + 4 * q;

    float4 x[kMergeBatch];
    float2 mv[kMergeBatch];
#pragma unroll
    for (int u = 0; u < kMergeBatch; ++u) {
        const int s = sl + 16 * u;
        x[u] = make_float4(0.f, 0.f, 0.f, 0.f);
        mv[u] = make_float2(-INFINITY, 0.0f);
        if (s < ns) {
            x[u] = *reinterpret_cast<const float4*>(accp + (int64_t)s * D);
            mv[u] = ml[s];
        }
    }

    // max of the split maxima
    float M = -INFINITY;
#pragma unroll
    for (int u = 0; u < kMergeBatch; ++u) M = fmaxf(M, mv[u].x);
    for (int s = sl + 16 * kMergeBatch; s < ns; s += 16) M = fmaxf(M, ml[s].x);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
    if (lane == 0) s_red[0][wv] = M;
    __syncthreads();
    M = fmaxf(fmaxf(s_red[0][0], s_red[0][1]), fmaxf(s_red[0][2], s_red[0][3]));
    const float Mu = (M == -INFINITY) ? 0.0f : M;

    // weighted sums: acc over this thread's splits; Lambda = sum_s w_s l_s counted once per
    // split (by the q == 0 thread of its split lane)
    float4 hi = make_float4(0.f, 0.f, 0.f, 0.f), lo = hi;
    float lh = 0.0f, ll = 0.0f;
    auto add = [&](float4 v, float2 m) {
        const float ws = __builtin_amdgcn_exp2f(m.x - Mu);   // 0 for an empty slot (m = -inf)
        comp_add(hi.x, lo.x, ws * v.x);
        comp_add(hi.y, lo.y, ws * v.y);
        comp_add(hi.z, lo.z, ws * v.z);
        comp_add(hi.w, lo.w, ws * v.w);
        if (q == 0) comp_add(lh, ll, ws * m.y);
    };
#pragma unroll
    for (int u = 0; u < kMergeBatch; ++u) add(x[u], mv[u]);
    for (int s = sl + 16 * kMergeBatch; s < ns; s += 16)
        add(*reinterpret_cast<const float4*>(accp + (int64_t)s * D), ml[s]);

    float lam = lh + ll;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) lam += __shfl_xor(lam, o);
    if (lane == 0) s_red[1][wv] = lam;
    s_part[sl][q][0] = hi;
    s_part[sl][q][1] = lo;
    __syncthreads();
    lam = (s_red[1][0] + s_red[1][1]) + (s_red[1][2] + s_red[1][3]);
    const int h = hq / (p.num_q_heads / p.num_kv_heads);
    const float scale = lam > 0.0f ? head_scale(p.v_scales, h, p.v_scale) / lam : 0.0f;
    if (tid < 64) {
        const int qq = tid >> 2, comp = tid & 3;
        float sh = 0.0f, sc = 0.0f;
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            const float4 a = s_part[k][qq][0];
            const float4 c = s_part[k][qq][1];
            const float av = comp == 0 ? a.x : comp == 1 ? a.y : comp == 2 ? a.z : a.w;
            const float cv = comp == 0 ? c.x : comp == 1 ? c.y : comp == 2 ? c.z : c.w;
            comp_add(sh, sc, av);
            sc += cv;
        }
        const int ch = chunk * 64 + 4 * qq + comp;
        store_out(p.out, p.out_f32, ((int64_t)b * p.num_q_heads + hq) * D + ch, scale * (sh + sc));
    }
}

// Largest dynamic LDS a partial-kernel launch may request (head_dim 256 keeps all 16 MFMA
// rows of 4 waves: about 65 KB; the rotated variant adds 16 KB of output rows).  Launches
// above 64 KB also need the device to allow it (gfx950 has 160 KB per workgroup).
constexpr size_t kMaxPartialLds = 160 * 1024;

// Dynamic LDS of the partial kernel: per-wave (m, l), every wave's accumulators over all 16
// MFMA rows, and the per-head wave weights, scale, max and normaliser; the rotated variant
// adds the 16 output rows it rotates back.
template <int D, bool ROT = false>
size_t partial_lds_bytes(int G) {
    (void)G;
    return sizeof(float) * (2 * kDecodeWaves * 16 + (size_t)kDecodeWaves * 16 * D + kDecodeWaves * 16 + 48 +
                            (ROT ? 16 * D : 0));
}

// Kernels whose dynamic LDS can exceed 64 KiB (g = 16 at head_dim 256) get their limit
// raised once, to the largest size any group ratio needs.
template <int D, int C, bool QLO, bool ROT = false>
hipError_t allow_lds(size_t need) {
    if (need <= 65536) return hipSuccess;
    // raise this kernel's limit once, to what the device allows (up to kMaxPartialLds)
    // (the kernel's static LDS counts against the same per-workgroup maximum)
    static const int allowed = [] {
        const void* fn = reinterpret_cast<const void*>(&decode_partial_kernel<D, C, QLO, ROT>);
        int dev = 0, lim = 65536;
        hipFuncAttributes fa{};
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&lim, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess ||
            hipFuncGetAttributes(&fa, fn) != hipSuccess)
            return 65536;
        lim -= (int)fa.sharedSizeBytes;
        if ((size_t)lim > kMaxPartialLds) lim = (int)kMaxPartialLds;
        if (hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, lim) != hipSuccess)
            return 65536;
        return lim;
    }();
    return need <= (size_t)allowed ? hipSuccess : hipErrorInvalidValue;
}

template <int D, int C, bool QLO, bool ROT = false>
hipError_t launch_partial_dc(const DecodeParams& p, size_t lds, dim3 grid, dim3 block, hipStream_t s) {
    const hipError_t e = allow_lds<D, C, QLO, ROT>(lds);
    if (e != hipSuccess) return e;
    return launch_kernel(reinterpret_cast<const void*>(&decode_partial_kernel<D, C, QLO, ROT>), grid, block,
                         lds, s, p);
}

template <int D>
hipError_t launch_rotated_d(const DecodeParams& p, Codec codec, hipStream_t s) {
    const int G = p.num_q_heads / p.num_kv_heads;
    const size_t lds = partial_lds_bytes<D, true>(G);
    const dim3 grid = kHeadsFastest ? dim3(p.num_kv_heads, p.splits, p.num_seqs)
                                    : dim3(p.splits, p.num_kv_heads, p.num_seqs);
    const dim3 block(64 * kDecodeWaves);
    switch (codec) {
        case kCodecE4M3: return launch_partial_dc<D, kCodecE4M3, true, true>(p, lds, grid, block, s);
        case kCodecBF16: return launch_partial_dc<D, kCodecBF16, true, true>(p, lds, grid, block, s);
        default: return hipErrorInvalidValue;
    }
}

template <int D, int C>
hipError_t launch_partial_c(const DecodeParams& p, size_t lds, dim3 grid, dim3 block, hipStream_t s) {
    return p.query_lo != nullptr ? launch_partial_dc<D, C, true>(p, lds, grid, block, s)
                                 : launch_partial_dc<D, C, false>(p, lds, grid, block, s);
}

template <int D>
hipError_t launch_partial_d(const DecodeParams& p, Codec codec, hipStream_t s) {
    const int G = p.num_q_heads / p.num_kv_heads;
    const size_t lds = partial_lds_bytes<D>(G);
    const dim3 grid = kHeadsFastest ? dim3(p.num_kv_heads, p.splits, p.num_seqs)
                                    : dim3(p.splits, p.num_kv_heads, p.num_seqs);
    const dim3 block(64 * kDecodeWaves);
    switch (codec) {
        case kCodecE4M3: return launch_partial_c<D, kCodecE4M3>(p, lds, grid, block, s);
        case kCodecBF16: return launch_partial_c<D, kCodecBF16>(p, lds, grid, block, s);
        case kCodecE5M2: return launch_partial_c<D, kCodecE5M2>(p, lds, grid, block, s);
        case kCodecINT8: return launch_partial_c<D, kCodecINT8>(p, lds, grid, block, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_decode_partial(const DecodeParams& p, Codec codec, int head_dim, hipStream_t s) {
    switch (head_dim) {
        case 64: return launch_partial_d<64>(p, codec, s);
        case 128: return launch_partial_d<128>(p, codec, s);
        case 256: return launch_partial_d<256>(p, codec, s);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_decode_partial_rotated(const DecodeParams& p, Codec codec, int head_dim, hipStream_t s) {
    switch (head_dim) {
        case 64: return launch_rotated_d<64>(p, codec, s);
        case 128: return launch_rotated_d<128>(p, codec, s);
        case 256: return launch_rotated_d<256>(p, codec, s);
        default: return hipErrorInvalidValue;
    }
}

bool fused_merge_fits(int group, int head_dim, int splits) {
    // every lane reads at most kMergeLaneSplits splits, in at most two passes over the
    // quads; at head_dim 256, four passes (one round trip) when a lane reads at most 8
    const int pairs = 64 * kDecodeWaves / 2;
    const int quads = group * head_dim / 4;
    return (splits <= 2 * kMergeLaneSplits && quads <= 2 * pairs) ||
           (head_dim == 256 && splits <= kMergeLaneBatch && quads <= 4 * pairs);
}

hipError_t launch_decode_merge(const DecodeParams& p, int head_dim, hipStream_t s) {
    if (head_dim != 64 && head_dim != 128 && head_dim != 256) return hipErrorInvalidValue;
    const dim3 grid(p.num_q_heads, p.num_seqs, head_dim / 64);
    int d = head_dim;
    void* args[] = {const_cast<DecodeParams*>(&p), &d};
    return hipLaunchKernel(reinterpret_cast<const void*>(&decode_merge_kernel), grid, dim3(256), args,
                           0, s);
}

}  // namespace fp8kv
