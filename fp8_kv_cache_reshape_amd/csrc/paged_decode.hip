// paged_decode.hip -- GQA decode attention that reads the paged fp8 (or bf16) KV cache.
//
// What is computed (header fp8kv.h has the exact definition): for each sequence and
// query head, softmax(q.K^T/sqrt(d)).V over the positions [lo, L) of the sequence's
// context, K and V dequantised inside the kernel (page "FP8 KV Cache Quantization:
// Capacity Gains and Accuracy Risk", "Attention backend interactions"), grouped-query
// heads sharing one kv head (page "ctx-fp8-kv-cache-long-context-accuracy",
// "Arithmetic intensity").  The context is cut into fixed-size splits whose fp32
// partials (m, l, acc) are merged by log-sum-exp in a second pass: partial sums stay in
// real fp32 registers at both levels, the two-level accumulation the pages credit with
// keeping 100K+ contractions accurate (page "The State of FP8 KV-Cache and Attention
// Quantization in vLLM", "ACCURACY AT LONG CONTEXT").
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
//               [grp*D/4 + 8kk, +8): every lane reads D/4 contiguous key bytes per row.
//   O += P.V  : A = 16 heads x 32 tokens (the lane's own probabilities, rounded to
//               bf16), B = 32 tokens x 16 channels.  The contraction slot of lane group
//               grp is (block grp, tokens 8u..8u+7), exactly the 8 value bytes that one
//               channel row of a channel-major value tile holds there, so each lane loads
//               one 16-byte row per 16-channel output tile and no LDS transpose is needed.
// fp8 codes become bf16 exactly (E4M3 is a subset of bf16) with the native gfx950
// conversion; k_scale/sqrt(d)*log2(e) scales the fp32 scores and v_scale is applied at
// the final normalisation, since the hardware's scaled conversions only take powers of 2.
#include "internal.h"

namespace fp8kv {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ inline bf16x8 bits_as_bf16x8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
    uint4 u = make_uint4(a, b, c, d);
    return __builtin_bit_cast(bf16x8, u);
}

// 8 E4M3 codes (bytes of lo then hi, in memory order) -> 8 bf16, exactly.
__device__ inline bf16x8 e4m3x8_to_bf16x8(uint32_t lo, uint32_t hi) {
    const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false);
    const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true);
    const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false);
    const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true);
    bf16x8 r = {a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
    return r;
}

__device__ inline f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ inline uint4 load16(const void* p) { return *reinterpret_cast<const uint4*>(p); }

// Byte mask keeping tokens [lo, hi) of a 16-token row (element size 1 or 2 bytes);
// returns the mask for the dword holding tokens [4k/es .. ) i.e. dword index k.
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

template <int D, bool FP8>
__global__ __launch_bounds__(64 * kDecodeWaves) void decode_partial_kernel(DecodeParams p) {
    constexpr int ES = FP8 ? 1 : 2;               // bytes per cache element
    constexpr int DG = D / 4;                     // channels per lane group in S = K.q^T
    constexpr int KK = D / 32;                    // MFMA k-steps for S
    constexpr int NT = D / 16;                    // 16-channel output tiles of O
    constexpr int K16 = DG * ES / 16;             // 16-byte key loads per lane per row
    constexpr int V16 = ES;                       // 16-byte value loads per lane per tile
    constexpr int TILE_BYTES = kBlockSize * D * ES;

    extern __shared__ float lds[];
    const int split = blockIdx.x;
    const int h = blockIdx.y;
    const int b = blockIdx.z;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int n = lane & 15;
    const int grp = lane >> 4;
    const int G = p.num_q_heads / p.num_kv_heads;

    const SeqWindow w = seq_window(p.context_lens[b], p.max_context_len, p.max_blocks_per_seq,
                                   p.sliding_window);
    const int sb = split * p.blocks_per_split;
    const int se = min(w.nblk, sb + p.blocks_per_split);
    const int64_t out_row0 = ((int64_t)b * p.num_q_heads + (int64_t)h * G) * D;
    if (sb >= se) {
        if (p.write_final && split == 0)
            for (int i = threadIdx.x; i < G * D; i += blockDim.x) store_out(p.out, p.out_f32, out_row0 + i, 0.0f);
        return;
    }

    // Query group as the B operand of S = K.q^T: lane (n, grp) holds head n, channels
    // [grp*DG + 8kk, +8) for kk = 0..KK-1; heads >= G are zero columns.
    bf16x8 qop[KK];
    {
        const uint16_t* qrow = p.query + out_row0 + (int64_t)n * D + grp * DG;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
            uint4 u = make_uint4(0, 0, 0, 0);
            if (n < G) u = load16(qrow + 8 * kk);
            qop[kk] = __builtin_bit_cast(bf16x8, u);
        }
    }

    const char* kcache = static_cast<const char*>(p.key_cache);
    const char* vcache = static_cast<const char*>(p.value_cache);
    const int32_t* bt = p.block_tables + (int64_t)b * p.max_blocks_per_seq + w.blk0 + sb;
    const float sscale = p.score_scale;

    float m_run = -INFINITY;     // running max of base-2 scores for head n
    float l_run = 0.0f;          // this lane's share of the running softmax sum
    f32x4 acc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int nsteps = (se - sb + 3) >> 2;
    for (int st = wave; st < nsteps; st += kDecodeWaves) {
        const int j0 = st * 4;
        const int kb = j0 + (n >> 2);            // block of the key rows this lane loads
        const int vb = j0 + grp;                 // block of this lane's scores and values
        int kphys = (sb + kb < se) ? bt[kb] : -1;
        int vphys = (sb + vb < se) ? bt[vb] : -1;
        const bool kval = (unsigned)kphys < (unsigned)p.num_blocks;
        const bool vval = (unsigned)vphys < (unsigned)p.num_blocks;

        // ---- loads: key rows (4 rows x DG channels) and value rows (NT channel rows)
        uint4 kr[4][K16];
        uint4 vr[NT][V16];
        {
            const char* kt = kcache + ((int64_t)(kval ? kphys : 0) * p.num_kv_heads + h) * TILE_BYTES
                             + (int64_t)((n & 3) * D + grp * DG) * ES;
#pragma unroll
            for (int s = 0; s < 4; ++s)
#pragma unroll
                for (int x = 0; x < K16; ++x)
                    kr[s][x] = kval ? load16(kt + (int64_t)(4 * s) * D * ES + 16 * x) : make_uint4(0, 0, 0, 0);
            const char* vt = vcache + ((int64_t)(vval ? vphys : 0) * p.num_kv_heads + h) * TILE_BYTES
                             + (int64_t)n * kBlockSize * ES;
#pragma unroll
            for (int t = 0; t < NT; ++t)
#pragma unroll
                for (int x = 0; x < V16; ++x)
                    vr[t][x] = vval ? load16(vt + (int64_t)(16 * t) * kBlockSize * ES + 16 * x) : make_uint4(0, 0, 0, 0);
        }

        // ---- S = K.q^T on the matrix cores
        f32x4 sc[4];
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < KK; ++kk) {
                bf16x8 a;
                if constexpr (FP8) {
                    const uint4 u = kr[s][kk >> 1];
                    a = (kk & 1) ? e4m3x8_to_bf16x8(u.z, u.w) : e4m3x8_to_bf16x8(u.x, u.y);
                } else {
                    a = __builtin_bit_cast(bf16x8, kr[s][kk]);
                }
                c = mfma16x16x32(a, qop[kk], c);
            }
            sc[s] = c;
        }

        // ---- mask and scale: lane holds block vb, tokens 4s+r, head n
        const int pos0 = (w.blk0 + sb + vb) * kBlockSize;
        const int tlo = max(0, w.lo - pos0);
        const int thi = min(kBlockSize, w.L - pos0);
        float sv[16];
        float mloc = -INFINITY;
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int tok = 4 * s + r;
                const bool ok = vval && tok >= tlo && tok < thi;
                const float x = ok ? sc[s][r] * sscale : -INFINITY;
                sv[4 * s + r] = x;
                mloc = fmaxf(mloc, x);
            }
        float mt = fmaxf(mloc, __shfl_xor(mloc, 16));
        mt = fmaxf(mt, __shfl_xor(mt, 32));
        const float m_new = fmaxf(m_run, mt);
        const float m_use = (m_new == -INFINITY) ? 0.0f : m_new;
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);   // exp2(-inf) = 0
        float pv[16];
        float psum = 0.0f;
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            pv[k] = __builtin_amdgcn_exp2f(sv[k] - m_use);
            psum += pv[k];
        }
        l_run = l_run * alpha + psum;
        m_run = m_new;

        // rescale the accumulators of heads 4grp..4grp+3 when any running max moved
        if (__any(alpha != 1.0f)) {
            float ar[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) ar[r] = __shfl(alpha, 4 * grp + r);
#pragma unroll
            for (int t = 0; t < NT; ++t)
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[t][r] *= ar[r];
        }

        // values of tokens outside [lo, L) in a partial block are zeroed so that a
        // poisoned (NaN) slot never reaches the accumulator through p = 0
        if (vval && (tlo > 0 || thi < kBlockSize)) {
#pragma unroll
            for (int t = 0; t < NT; ++t)
#pragma unroll
                for (int x = 0; x < V16; ++x) {
                    vr[t][x].x &= token_mask_dword<ES>(tlo, thi, 4 * x + 0);
                    vr[t][x].y &= token_mask_dword<ES>(tlo, thi, 4 * x + 1);
                    vr[t][x].z &= token_mask_dword<ES>(tlo, thi, 4 * x + 2);
                    vr[t][x].w &= token_mask_dword<ES>(tlo, thi, 4 * x + 3);
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
                    const uint4 v = vr[t][0];
                    vb8 = u ? e4m3x8_to_bf16x8(v.z, v.w) : e4m3x8_to_bf16x8(v.x, v.y);
                } else {
                    vb8 = __builtin_bit_cast(bf16x8, vr[t][u]);
                }
                acc[t] = mfma16x16x32(phi[u], vb8, acc[t]);
                acc[t] = mfma16x16x32(plo[u], vb8, acc[t]);
            }
        }
    }

    // ---- combine the waves of this workgroup in LDS
    float l_tot = l_run + __shfl_xor(l_run, 16);
    l_tot += __shfl_xor(l_tot, 32);
    float* sm_m = lds;                           // [waves][16]
    float* sm_l = lds + kDecodeWaves * 16;       // [waves][16]
    float* sm_a = lds + 2 * kDecodeWaves * 16;   // [waves][G][D]
    if (grp == 0) {
        sm_m[wave * 16 + n] = m_run;
        sm_l[wave * 16 + n] = l_tot;
    }
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int head = 4 * grp + r;
            if (head < G) sm_a[(wave * G + head) * D + 16 * t + n] = acc[t][r];
        }
    __syncthreads();

    for (int idx = threadIdx.x; idx < G * D; idx += blockDim.x) {
        const int head = idx / D;
        const int i = idx - head * D;
        float M = -INFINITY;
#pragma unroll
        for (int v = 0; v < kDecodeWaves; ++v) M = fmaxf(M, sm_m[v * 16 + head]);
        const float Mu = (M == -INFINITY) ? 0.0f : M;
        float lam = 0.0f, a = 0.0f;
#pragma unroll
        for (int v = 0; v < kDecodeWaves; ++v) {
            const float wv = __builtin_amdgcn_exp2f(sm_m[v * 16 + head] - Mu);
            lam += wv * sm_l[v * 16 + head];
            a += wv * sm_a[(v * G + head) * D + i];
        }
        if (p.write_final) {
            store_out(p.out, p.out_f32, out_row0 + (int64_t)head * D + i,
                      lam > 0.0f ? p.v_scale * a / lam : 0.0f);
        } else {
            const int64_t row = ((int64_t)b * p.num_q_heads + (int64_t)h * G + head) * p.splits + split;
            p.ws_acc[row * D + i] = a;
            if (i == 0) {
                p.ws_ml[row * 2 + 0] = M;
                p.ws_ml[row * 2 + 1] = lam;
            }
        }
    }
}

// Pass 2: log-sum-exp merge of one (sequence, query head) over its splits.
template <int D>
__global__ __launch_bounds__(256) void decode_merge_kernel(DecodeParams p) {
    constexpr int NSUB = 256 / D;                // threads per channel
    __shared__ float s_w[kMaxSplits];            // per-split weight exp2(m_s - M) / Lambda
    __shared__ float s_part[256];
    const int hq = blockIdx.x;
    const int b = blockIdx.y;
    const int tid = threadIdx.x;
    const SeqWindow w = seq_window(p.context_lens[b], p.max_context_len, p.max_blocks_per_seq,
                                   p.sliding_window);
    const int ns = (w.nblk + p.blocks_per_split - 1) / p.blocks_per_split;
    const int64_t row0 = ((int64_t)b * p.num_q_heads + hq) * p.splits;
    const int64_t out_idx = ((int64_t)b * p.num_q_heads + hq) * D;

    if (tid < 64) {
        float M = -INFINITY;
        for (int s = tid; s < ns; s += 64) M = fmaxf(M, p.ws_ml[(row0 + s) * 2]);
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
        const float Mu = (M == -INFINITY) ? 0.0f : M;
        float lam = 0.0f;
        for (int s = tid; s < ns; s += 64) {
            const float wv = __builtin_amdgcn_exp2f(p.ws_ml[(row0 + s) * 2] - Mu);
            s_w[s] = wv;
            lam += wv * p.ws_ml[(row0 + s) * 2 + 1];
        }
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) lam += __shfl_xor(lam, o);
        const float inv = lam > 0.0f ? p.v_scale / lam : 0.0f;
        for (int s = tid; s < ns; s += 64) s_w[s] *= inv;
    }
    __syncthreads();

    const int i = tid % D;
    const int sub = tid / D;
    float a = 0.0f;
    for (int s = sub; s < ns; s += NSUB) a += s_w[s] * p.ws_acc[(row0 + s) * D + i];
    if (NSUB > 1) {
        s_part[tid] = a;
        __syncthreads();
        if (sub == 0) {
            for (int k = 1; k < NSUB; ++k) a += s_part[k * D + i];
        }
    }
    if (sub == 0) store_out(p.out, p.out_f32, out_idx + i, a);
}

// Dynamic LDS of the partial kernel: per-wave (m, l) and the group's accumulators.
template <int D>
size_t partial_lds_bytes(int G) {
    return sizeof(float) * (2 * kDecodeWaves * 16 + (size_t)kDecodeWaves * G * D);
}

// Kernels whose dynamic LDS can exceed 64 KiB (g = 16 at head_dim 256) get their limit
// raised once, to the largest size any group ratio needs.
template <int D, bool FP8>
hipError_t allow_lds() {
    static const hipError_t e = [] {
        const size_t need = partial_lds_bytes<D>(kMaxGroup);
        if (need <= 65536) return hipSuccess;
        return hipFuncSetAttribute(reinterpret_cast<const void*>(&decode_partial_kernel<D, FP8>),
                                   hipFuncAttributeMaxDynamicSharedMemorySize, (int)need);
    }();
    return e;
}

template <int D>
hipError_t launch_partial_d(const DecodeParams& p, bool fp8, hipStream_t s) {
    const int G = p.num_q_heads / p.num_kv_heads;
    const size_t lds = partial_lds_bytes<D>(G);
    const dim3 grid(p.splits, p.num_kv_heads, p.num_seqs);
    const dim3 block(64 * kDecodeWaves);
    hipError_t e = fp8 ? allow_lds<D, true>() : allow_lds<D, false>();
    if (e != hipSuccess) return e;
    const void* fn = fp8 ? reinterpret_cast<const void*>(&decode_partial_kernel<D, true>)
                         : reinterpret_cast<const void*>(&decode_partial_kernel<D, false>);
    return launch_kernel(fn, grid, block, lds, s, p);
}

template <int D>
hipError_t launch_merge_d(const DecodeParams& p, hipStream_t s) {
    return launch_kernel(reinterpret_cast<const void*>(&decode_merge_kernel<D>),
                         dim3(p.num_q_heads, p.num_seqs), dim3(256), 0, s, p);
}

}  // namespace

hipError_t launch_decode_partial(const DecodeParams& p, bool fp8, int head_dim, hipStream_t s) {
    switch (head_dim) {
        case 64: return launch_partial_d<64>(p, fp8, s);
        case 128: return launch_partial_d<128>(p, fp8, s);
        case 256: return launch_partial_d<256>(p, fp8, s);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_decode_merge(const DecodeParams& p, int head_dim, hipStream_t s) {
    switch (head_dim) {
        case 64: return launch_merge_d<64>(p, s);
        case 128: return launch_merge_d<128>(p, s);
        case 256: return launch_merge_d<256>(p, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace fp8kv
