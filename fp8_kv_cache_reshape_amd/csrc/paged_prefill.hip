// paged_prefill.hip -- prefill / chunked-prefill attention over the paged KV cache.
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
// accumulator sums at most kFlushKeys keys, then its partial sums move into plain
// fp32 registers.
//
// Work mapping.  A query "column" is one (chunk token, query head of the group) pair; the
// columns of a (sequence, kv head) are numbered token-major, head fastest, so the g heads
// of one token -- which read the same keys -- sit side by side.  A workgroup of 8 waves
// owns consecutive columns of one (sequence, kv head): two 16-column tiles per wave at
// d <= 128 (256 per workgroup), whose products share every key and value operand read, and
// one at d = 256 (128 per workgroup), whose accumulators would not fit twice.  It walks the
// keys its columns need one step at a time (Stage: 32 to 128 keys).  The grid is ordered
// longest first over every (sequence, kv head).
//
// Staging.  Each step's K and V tiles are loaded once per workgroup (spread over the waves),
// widened on the way -- keys to bf16, values to fp16 (bf16 for the bf16 cache); one-byte
// codes are exact in both -- and written into a double-buffered LDS tile; the loads run
// two steps ahead in registers.  The matrix cores then read their operands straight from
// LDS, so no wave converts codes itself.  The LDS
// tiles have their own order, chosen so that every operand read instruction covers
// contiguous 256-byte runs (no bank conflicts): keys [group][slice][slot][8 channels],
// values of a block pair [16-channel tile][group][channel][block][4 slots].  With two
// column tiles the query operands sit in LDS too, in each wave's own region.
//
// Both products run on 16x16x32 matrix-core tiles (per 16-column tile; 16 columns keep
// the layout in which the scores feed P.V straight from registers):
//   S = K.Q^T per block : A = 16 key slots x 32 channels, B = 32 channels x 16 columns.
//               Lane l (column l%16, group g = l/16) gets slots 4g..4g+3 of the block; the
//               32-channel slice kk of group g is channels [g*d/4 + 8kk, +8) -- one 16-byte
//               chunk of the key tile.
//   O += P.V  : A = 16 columns x 32 keys, B = 32 keys x 16 channels, per pair of blocks.
//               Group g's contraction slot is slots 4g..4g+3 of both blocks of the pair:
//               8 of the probabilities the lane holds, and one 16-byte LDS read.
// S runs in bf16 (q is bf16).  With a one-byte cache P.V runs in fp16: each probability is
// rounded once to fp16 (relative error <= 2^-12, eight times below a bf16 rounding), after
// a 2^7 scaling that keeps small probabilities out of the fp16 subnormal range (the
// normaliser carries the same factor).  With the bf16 cache, whose values are not fp16
// values, probabilities enter P.V as a high (truncated) and a low bf16 term.  Scores are kept in
// base-2 units (k_scale log2(e)/sqrt(d) is applied inside the exponent's FMA); v_scale
// multiplies the final normalisation.  The running maximum of a column only moves when a
// score exceeds it by 2^8, so the accumulators are rarely rescaled.
#include <type_traits>

#include "codec.h"
#include "internal.h"

namespace fp8kv {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef const __attribute__((address_space(4))) int32_t* ConstI32Ptr;

constexpr int kWaves = 8;
constexpr int kCols = 16;                  // query columns per wave
constexpr int kFlushKeys = 256;            // keys summed in the matrix-core accumulator
constexpr float kRescaleLog2 = 8.0f;
constexpr int kPShift = 7;                 // fp16 probabilities are scaled by 2^7 (<= 2^15)

__device__ inline f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ inline f32x4 mfma16(f16x8 a, f16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ inline void store_out(void* out, int out_f32, int64_t idx, float v) {
    if (out_f32)
        static_cast<float*>(out)[idx] = v;
    else
        static_cast<__bf16*>(out)[idx] = (__bf16)v;   // round to nearest even
}

// Maximum over the four lanes l, l^16, l^32, l^48 (the four contraction groups of a
// column), with the VALU row swaps of gfx950: after a swap the two results hold the values
// of lane l and its partner, in some order, so their maximum is the pair's.
__device__ inline float max_over_groups(float m) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(m), __float_as_uint(m), false, false);
    m = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// Compensated add (Knuth's TwoSum) of x into (hi, lo).
__device__ inline void comp_add(float& hi, float& lo, float x) {
    const float s = hi + x;
    const float bp = s - hi;
    const float ap = s - bp;
    lo += (hi - ap) + (x - bp);
    hi = s;
}

// LDS byte offset of key element (slot, channel) of a staged block: [group g = ch/(D/4)]
// [slice kk = (ch % (D/4))/8][slot ^ swz(g, kk)][channel % 8], bf16.  The XOR keeps each
// 16-slot row a permutation, so the operand reads stay conflict-free; swz (bit 2: bit 1
// of g ^ bit 0 of kk, bit 3: bit 0 ^ bit 1 of kk) gives the lanes of one staging store --
// the same slot in different (group, slice) rows -- different banks, 8 and 16 lanes at a
// time, at head_dim 128 and 256.
template <int D>
__device__ constexpr int lds_key(int slot, int ch) {
    const int g = ch / (D / 4);
    const int kk = (ch % (D / 4)) / 8;
    const int swz = 4 * (((g >> 1) ^ kk) & 1) + 8 * ((kk ^ (kk >> 1)) & 1);
    return ((g * (D / 32) + kk) * kBlockSize + (slot ^ swz)) * 16 + (ch % 8) * 2;
}

// LDS byte offset of value element (channel, slot) of block cb (0 or 1) of a staged block
// pair: [tile t = ch/16][group = slot/4][channel % 16][cb][slot % 4], bf16 -- the 4 slots
// of a group in both blocks of the pair are one 16-byte operand read.
__device__ constexpr int lds_value(int ch, int slot, int cb) {
    return ((((ch / 16) * 4 + slot / 4) * 16 + ch % 16) * 2 + cb) * 8 + (slot % 4) * 2;
}

// Staging geometry.  A step covers NB cache blocks: 128 keys (8 blocks) for one-byte caches
// at d <= 128 and for d = 64, whose double-buffered widened tiles (2 x 2 x NB) fill 128 KB
// of the 160 KB LDS, so each step's fixed work (block ids, masks, barrier) is spread over
// twice the matrix-core products; 64 keys for the bf16 cache at d = 128 and 32 at d = 256,
// where the larger step would not fit the registers of two waves per SIMD.  Its 2*NB cache
// tiles (keys of blocks 0..NB-1, then their values) are moved by the 8 waves: each wave
// WAVE_SRC contiguous source bytes, in PIECES pieces of PIECE_SRC bytes that each lie in one
// tile, each lane PER bytes of a piece.
#ifndef FP8KV_PREFILL_TILES
#define FP8KV_PREFILL_TILES 2
#endif
// Column tiles per wave: two 16-column tiles at d <= 128, whose products share every key and
// value operand read from LDS; one at d = 256, whose accumulators would not fit twice in the
// registers of two waves per SIMD.
__host__ __device__ constexpr int col_tiles(int d) { return d <= 128 && FP8KV_PREFILL_TILES >= 2 ? 2 : 1; }

template <int D, int C, bool QLO = false>
struct Stage {
    static constexpr int CT = col_tiles(D);
    static constexpr bool WIDE = D == 64 || (D == 128 && C != kCodecBF16);
    // blocks per step (a two-byte cache stages twice the bytes and needs the low P term, so
    // its steps are half as long at two column tiles)
    // (with the low query term the query operands take twice the LDS, so head_dim 128 steps
    // are 32 keys)
    static constexpr int NB = CT == 2 ? (QLO && D == 128 ? 2 : (D == 64 ? 8 : 4) / (C == kCodecBF16 ? 2 : 1))
                                      : (D <= 128 ? 4 : 2) * (WIDE ? 2 : 1);
    static constexpr int STEP = NB * kBlockSize;              // keys per step
    static constexpr int ES = C == kCodecBF16 ? 2 : 1;       // source bytes per element
    static constexpr int TILE_SRC = kBlockSize * D * ES;     // bytes of a cache tile
    static constexpr int TILE_LDS = kBlockSize * D * 2;      // bytes of its bf16 copy
    static constexpr int WAVE_SRC = 2 * NB * TILE_SRC / kWaves;
    static constexpr int PIECE_SRC = WAVE_SRC < TILE_SRC ? WAVE_SRC : TILE_SRC;
    static constexpr int PIECES = WAVE_SRC / PIECE_SRC;
    static constexpr int PER = PIECE_SRC / 64;               // source bytes per lane and piece
    static constexpr int NW = PER / 4;                       // dwords per lane and piece
    static constexpr int FLUSH = kFlushKeys / STEP;          // steps per accumulator flush
    static_assert(TILE_SRC % PIECE_SRC == 0 && WAVE_SRC % PIECE_SRC == 0, "a piece stays in one tile");
    static_assert(PER % 16 == 0 && FLUSH >= 1, "staging geometry");
};

// QLO: the rotated prefill, whose query enters S as two bf16 terms (query, query_lo).
template <int D, int C, bool QLO = false>
__global__ __launch_bounds__(64 * kWaves)
__attribute__((amdgpu_waves_per_eu(2, 2)))
void prefill_kernel(PrefillParams p) {
    using S = Stage<D, C, QLO>;
    constexpr int CT = S::CT;
    constexpr int WCOLS = kCols * CT;      // query columns per wave
    constexpr int NB = S::NB;
    constexpr int STEP = S::STEP;
    constexpr int NK = D / 32;             // 32-channel contraction slices of S
    constexpr int NT = D / 16;             // 16-channel output tiles of O
    constexpr int TL = S::TILE_LDS;
    constexpr uint32_t kAllBlocks = (1u << NB) - 1;
    // P.V operands: fp16 for the one-byte codecs (their codes are exact fp16 values), bf16
    // for the bf16 cache
    constexpr bool kF16 = C != kCodecBF16;
    using pv_t = std::conditional_t<kF16, f16x8, bf16x8>;
    // a staged step: key tiles of blocks 0..NB-1 in bf16, then their value tiles (pv_t)
    __shared__ __attribute__((aligned(16))) uint8_t sm_kv[2][2 * NB * TL];
    // with two column tiles the query operands live in LDS (each wave's own region, 16-byte
    // pieces [tile][slice][lane]), read again for every step: registers are what bounds
    // this kernel
    constexpr bool kQLds = CT == 2;
    static_assert(!QLO || kQLds, "the low query term lives in LDS");
    constexpr int kQTerms = QLO ? 2 : 1;
    __shared__ __attribute__((aligned(16))) uint8_t sm_q[kQLds ? kWaves * kQTerms * CT * NK * 64 * 16 : 16];

    const int lane = threadIdx.x & 63;
    // wave-uniform (a scalar register, so that the staging addresses stay scalar)
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int col = lane & 15;             // this lane's query column
    const int grp = lane >> 4;             // contraction group
    // grid x = (column tile, sequence, kv head), tile slowest: workgroups start in index order,
    // so the heaviest tiles of every sequence and head go first (longest first over the grid)
    const int hb = (int)blockIdx.x % (p.num_seqs * p.num_kv_heads);
    const int h = hb % p.num_kv_heads;     // kv head
    const int b = hb / p.num_kv_heads;
    const int G = p.num_q_heads / p.num_kv_heads;

    const int q0 = ((ConstI32Ptr)p.query_start_loc)[b];
    const int nq = ((ConstI32Ptr)p.query_start_loc)[b + 1] - q0;       // chunk tokens
    const int tile = (int)gridDim.x / (p.num_seqs * p.num_kv_heads) - 1 -
                     (int)blockIdx.x / (p.num_seqs * p.num_kv_heads);  // heaviest tiles first
    const int64_t ncols = (int64_t)(nq > 0 ? nq : 0) * G;
    const int64_t cw0 = (int64_t)tile * (kWaves * WCOLS);            // first column of the workgroup
    if (p.err != nullptr && tile == 0 && h == 0 && threadIdx.x == 0) {
        const int len_in = ((ConstI32Ptr)p.context_lens)[b];
        if (nq < 0 || nq > p.max_query_len) report_error(p.err, kErrQueryLen);
        if (len_in < 0 || len_in > p.max_context_len || len_in > p.max_blocks_per_seq * kBlockSize)
            report_error(p.err, kErrContextLen);
    }
    if (cw0 >= ncols) return;                                         // (whole workgroup)
    const int64_t c0 = cw0 + wave * WCOLS;                            // first column of the wave
    const bool wactive = c0 < ncols;

    int L = ((ConstI32Ptr)p.context_lens)[b];
    if (L > p.max_context_len) L = p.max_context_len;
    if (L > p.max_blocks_per_seq * kBlockSize) L = p.max_blocks_per_seq * kBlockSize;
    if (L < 0) L = 0;
    const int W = p.sliding_window;
    auto lo_of = [&](int pos) { return (W > 0 && pos + 1 > W) ? pos + 1 - W : 0; };

    // this lane's column in tile j: c0 + 16 j + col
    bool cvalid[CT];
    int tok[CT], hq[CT], pos[CT], clo[CT];
#pragma unroll
    for (int j = 0; j < CT; ++j) {
        const int64_t cg = c0 + kCols * j + col;
        cvalid[j] = cg < ncols && q0 + (int)(cg / G) < p.num_rows;
        tok[j] = cvalid[j] ? (int)(cg / G) : 0;
        hq[j] = h * G + (cvalid[j] ? (int)(cg % G) : 0);
        pos[j] = L - nq + tok[j];          // < 0: the column attends to nothing
        clo[j] = lo_of(pos[j]);
    }

    // key ranges: the workgroup stages [lo of its first position, its last position]; a
    // wave computes only the steps its own columns can see
    const int64_t cwlast = (cw0 + kWaves * WCOLS <= ncols ? cw0 + kWaves * WCOLS : ncols) - 1;
    const int pwmin = L - nq + (int)(cw0 / G);
    const int kend = L - nq + (int)(cwlast / G) + 1;                  // exclusive, <= L
    const int kfirst = pwmin >= 0 ? (lo_of(pwmin) / STEP) * STEP : 0;
    const int nsteps = kend > kfirst ? (kend - kfirst + STEP - 1) / STEP : 0;
    const int64_t clast = wactive ? (c0 + WCOLS <= ncols ? c0 + WCOLS : ncols) - 1 : c0;
    const int pmin = L - nq + (int)(c0 / G);
    const int pmax = L - nq + (int)(clast / G);
    const int lomax = lo_of(pmax);
    const int lomin = lo_of(pmin);

    // query operand of S for tile j: slice kk = q[hq][grp*D/4 + 8kk .. +8), in registers
    // (one tile) or in this wave's LDS region (two tiles; only this wave reads it back, and a
    // wave's LDS accesses take effect in order, so no barrier is needed)
    bf16x8 qb[kQLds ? 1 : CT][NK];
    uint8_t* const sq = sm_q + (kQLds ? wave * (kQTerms * CT * NK * 64 * 16) : 0);
#pragma unroll
    for (int j = 0; j < CT; ++j) {
        const int64_t qoff = ((int64_t)(q0 + tok[j]) * p.num_q_heads + hq[j]) * D + grp * (D / 4);
#pragma unroll
        for (int kk = 0; kk < NK; ++kk) {
            u32x4 v = {0u, 0u, 0u, 0u};
            if (cvalid[j] && pos[j] >= 0) v = *reinterpret_cast<const u32x4*>(p.query + qoff + 8 * kk);
            if constexpr (kQLds)
                *reinterpret_cast<u32x4*>(sq + ((j * NK + kk) * 64 + lane) * 16) = v;
            else
                qb[kQLds ? 0 : j][kk] = __builtin_bit_cast(bf16x8, v);
            if constexpr (QLO) {   // the low term, in the second half of the region
                u32x4 u = {0u, 0u, 0u, 0u};
                if (cvalid[j] && pos[j] >= 0) u = *reinterpret_cast<const u32x4*>(p.query_lo + qoff + 8 * kk);
                *reinterpret_cast<u32x4*>(sq + (((CT + j) * NK + kk) * 64 + lane) * 16) = u;
            }
        }
    }
    auto read_q = [&](int j, int kk) {
        return kQLds ? __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(sq + ((j * NK + kk) * 64 + lane) * 16))
                     : qb[kQLds ? 0 : j][kk];
    };
    auto read_qlo = [&](int j, int kk) {
        return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(sq + (((CT + j) * NK + kk) * 64 + lane) * 16));
    };

    const float kscale = p.k_scales != nullptr
                             ? ((const __attribute__((address_space(4))) float*)p.k_scales)[h]
                             : 1.0f;
    const float sscale = p.score_scale * kscale;
    const ConstI32Ptr bt = (ConstI32Ptr)(p.block_tables + (int64_t)b * p.max_blocks_per_seq);

    f32x4 oacc[CT][NT], osum[CT][NT];
    float mref[CT];                        // running reference maximum of this lane's columns
    float l_hi[CT], l_lo[CT];              // sum of this lane's share of their probabilities
#pragma unroll
    for (int j = 0; j < CT; ++j) {
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            oacc[j][t] = f32x4{};
            osum[j][t] = f32x4{};
        }
        mref[j] = -INFINITY;
        l_hi[j] = 0.0f;
        l_lo[j] = 0.0f;
    }

    if (nsteps > 0) {   // (then L >= 1, so the table and the cache hold at least one block)
    // ---- block ids.  The NB ids of a step are read one step before the step is staged,
    // ahead of a barrier, so the loads never stall the matrix-core work.  When the step's NB
    // table entries all lie inside the row (every step but at most the row's last) they are
    // one NB-dword scalar load; otherwise each index is clamped to the row.  ok_mask turns
    // them into a bit per block, without branches: a valid id (inside [0, num_blocks)) whose
    // first key lies before kend (such a block is inside the row, as kend <= L).
    typedef int ids_t __attribute__((ext_vector_type(NB)));
    typedef const __attribute__((address_space(4))) ids_t* ConstIdsPtr;
    const int nrow = p.max_blocks_per_seq;
    auto load_ids = [&](int st) {
        const int n0 = (kfirst + (st < nsteps ? st : 0) * STEP) / kBlockSize;
        ids_t ids;
        if (n0 + NB <= nrow) {
            // NB consecutive dwords of the row (dword-aligned: one scalar load)
            ids = *(ConstIdsPtr)(bt + n0);
        } else {
#pragma unroll
            for (int c = 0; c < NB; ++c) ids[c] = bt[n0 + c < nrow ? n0 + c : nrow - 1];
        }
        return ids;
    };
    auto ok_mask = [&](int st, ids_t ids) {
        const int kb = kfirst + st * STEP;
        uint32_t m = 0;
#pragma unroll
        for (int c = 0; c < NB; ++c)
            m |= ((uint32_t)((unsigned)ids[c] < (unsigned)p.num_blocks) &
                  (uint32_t)(kb + c * kBlockSize < kend)) << c;
        return m;
    };

    // ---- staging: wave w moves source bytes [w*WAVE_SRC, +WAVE_SRC) of the step's tiles, in
    // PIECES pieces that each lie in one tile.  The loads are always issued (a missing block
    // reads block 0, in bounds) so that no branch sits between a load and its use; missing
    // blocks become zeros and value slots at or past kend are zeroed when a piece is widened
    // and written to LDS.
    typedef uint32_t piece_t __attribute__((ext_vector_type(S::NW)));
    struct stage_t { piece_t pc[S::PIECES]; };
    // geometry of piece i of this wave (wave-uniform except the lane's byte offset)
    auto piece_part = [&](int i) { return (wave * S::WAVE_SRC + i * S::PIECE_SRC) / S::TILE_SRC; };
    auto piece_off = [&](int i) {        // byte offset of this lane's bytes in the piece's tile
        return (wave * S::WAVE_SRC + i * S::PIECE_SRC) % S::TILE_SRC + lane * S::PER;
    };
    auto stage_load = [&](ids_t ids, uint32_t okm, stage_t& r) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < S::PIECES; ++i) {
            const int part = piece_part(i);
            const int part_c = part % NB;
            int id = ids[0];
#pragma unroll
            for (int c = 1; c < NB; ++c) id = part_c == c ? ids[c] : id;
            id = (okm >> part_c) & 1u ? id : 0;
            const uint8_t* src = static_cast<const uint8_t*>(part >= NB ? p.value_cache : p.key_cache) +
                                 ((int64_t)id * p.num_kv_heads + h) * S::TILE_SRC + piece_off(i);
            r.pc[i] = __builtin_nontemporal_load(reinterpret_cast<const piece_t*>(src));
        }
    };
    auto stage_store = [&](int buf, int st, uint32_t okmask, const stage_t& r0) __attribute__((always_inline)) {
        const int kb = kfirst + st * STEP;
#pragma unroll
        for (int i = 0; i < S::PIECES; ++i) {
        const int part = piece_part(i);
        const int part_c = part % NB;
        const bool part_v = part >= NB;
        const int src_off = piece_off(i);
        // a missing block stages zeros (a wave-uniform test: no per-lane masking in the
        // common case)
        piece_t r = r0.pc[i];
        if (!((okmask >> part_c) & 1u)) r = piece_t{};
        // value slots at or past kend are zeroed below, only in a block that reaches kend
        const int nvalid = kend - (kb + part_c * kBlockSize);
        const bool tail = nvalid < kBlockSize;
        // keys: tile part; values: the pair region of blocks 2*(c/2), 2*(c/2)+1
        uint8_t* dst = sm_kv[buf] + (part_v ? NB + 2 * (part_c / 2) : part) * TL;
        constexpr int EPL = S::PER / S::ES;                       // elements per lane
        constexpr int DW8 = 2 * S::ES;                            // source dwords per 8 elements
#pragma unroll
        for (int j = 0; j < EPL / 8; ++j) {
            const int e0 = src_off / S::ES + 8 * j;               // element index in the tile
            u32x4 v;
            if constexpr (C == kCodecBF16) {
                v = u32x4{r[4 * j], r[4 * j + 1], r[4 * j + 2], r[4 * j + 3]};
            } else if (!part_v) {
                v = __builtin_bit_cast(u32x4, codes8_to_bf16x8<C>(r[DW8 * j], r[DW8 * j + 1]));
            } else {
                v = __builtin_bit_cast(u32x4, codes8_to_f16x8<C>(r[DW8 * j], r[DW8 * j + 1]));
            }
            if (!part_v) {
                // element e0 of the source key tile: invert the chunk layout to (slot, channel)
                const int o = e0 * S::ES;                         // source byte offset
                constexpr int C1 = D * S::ES / 64;                // chunks per quarter of a slot
                const int slot = 4 * ((o / 256) / C1) + (o / 64) % 4;
                const int ch = ((o % 64) / 16) * (D / 4) + (16 * ((o / 256) % C1) + o % 16) / S::ES;
                *reinterpret_cast<u32x4*>(dst + lds_key<D>(slot, ch)) = v;
            } else {
                // value tile: channel-major rows of 16 slots; zero the slots at or past kend
                const int slot0 = e0 % kBlockSize;
                if (tail && slot0 + 8 > nvalid) {
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        const uint32_t lo = slot0 + 2 * k < nvalid ? 0x0000FFFFu : 0u;
                        const uint32_t hi = slot0 + 2 * k + 1 < nvalid ? 0xFFFF0000u : 0u;
                        v[k] &= lo | hi;
                    }
                }
                // slots slot0 .. slot0+7 of channel e0 / 16: two 4-slot groups
                const int ch = e0 / kBlockSize;
                *reinterpret_cast<u32x2*>(dst + lds_value(ch, slot0, part_c % 2)) = u32x2{v[0], v[1]};
                *reinterpret_cast<u32x2*>(dst + lds_value(ch, slot0 + 4, part_c % 2)) = u32x2{v[2], v[3]};
            }
        }
        }
    };

    int flush = 0;
    // multiply the O rows of tile j (its columns 4*grp + i) by their columns' factors
    auto rescale_rows = [&](int j, float f) __attribute__((always_inline)) {
        float fr[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) fr[i] = __shfl(f, 4 * grp + i);
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                oacc[j][t][i] *= fr[i];
                osum[j][t][i] *= fr[i];
            }
    };

    auto compute = [&](int st, int buf, uint32_t okmask) __attribute__((always_inline)) {
        const int kb = kfirst + st * STEP;
        // whether the step holds any key this wave's columns attend to (one uniform test)
        if (!((st < nsteps) & wactive & (kb <= pmax) & (kb + STEP > lomin))) return;
        const uint8_t* sk = sm_kv[buf];

        // ---- value operands of P.V (lane: slots 4*grp .. +3 of both blocks of a pair, channel
        // 16t + col).  They do not depend on the scores: with one column tile, when they fit in
        // 64 registers, they are read first, so their LDS latency hides behind S and the
        // softmax; otherwise each is read just before its products.
        auto read_v = [&](int t, int r) {
            return *reinterpret_cast<const pv_t*>(sk + (NB + 2 * r) * TL + lds_value(16 * t + col, 4 * grp, 0));
        };
        constexpr bool kEarlyV = CT == 1 && D <= 128 && NT * (NB / 2) <= 16;
        pv_t vb[kEarlyV ? NT : 1][NB / 2];
        if constexpr (kEarlyV) {
#pragma unroll
            for (int t = 0; t < NT; ++t)
#pragma unroll
                for (int r = 0; r < NB / 2; ++r) vb[t][r] = read_v(t, r);
        }

        // ---- S = K.Q^T for each block and column tile: lane holds slots 4*grp + i of its
        // column; each key operand read feeds the products of every tile
        f32x4 s[CT][NB];
        auto read_k = [&](int c, int kk) {
            return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(
                sk + c * TL + lds_key<D>(col, grp * (D / 4) + 8 * kk)));
        };
        if constexpr (CT == 2) {
            // contraction slice outermost: the query operands of slice kk are read once per
            // step, and the 2 NB accumulators are independent
#pragma unroll
            for (int c = 0; c < NB; ++c)
#pragma unroll
                for (int j = 0; j < CT; ++j) s[j][c] = f32x4{};
#pragma unroll
            for (int kk = 0; kk < NK; ++kk) {
                bf16x8 qk[CT], ql[QLO ? CT : 1];
#pragma unroll
                for (int j = 0; j < CT; ++j) {
                    qk[j] = read_q(j, kk);
                    if constexpr (QLO) ql[j] = read_qlo(j, kk);
                }
#pragma unroll
                for (int c = 0; c < NB; ++c) {
                    const bf16x8 kop = read_k(c, kk);
#pragma unroll
                    for (int j = 0; j < CT; ++j) {
                        s[j][c] = mfma16(kop, qk[j], s[j][c]);
                        if constexpr (QLO) s[j][c] = mfma16(kop, ql[QLO ? j : 0], s[j][c]);
                    }
                }
            }
        } else {
#pragma unroll
            for (int c = 0; c < NB; ++c) {
                f32x4 a = f32x4{};
#pragma unroll
                for (int kk = 0; kk < NK; ++kk) a = mfma16(read_k(c, kk), read_q(0, kk), a);
                s[0][c] = a;
            }
        }

        // ---- raw scores masked outside [clo, pos] and outside valid blocks; the base-2
        // scale (> 0) is applied to the maximum and inside the exponent's FMA
        if ((kb + STEP > pmin + 1) | (kb < lomax) | (okmask != kAllBlocks)) {
            const int k0 = kb + 4 * grp;
#pragma unroll
            for (int j = 0; j < CT; ++j)
#pragma unroll
                for (int c = 0; c < NB; ++c)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int kp = k0 + c * kBlockSize + i;
                        const bool ok = kp >= clo[j] && kp <= pos[j] && ((okmask >> c) & 1u);
                        s[j][c][i] = ok ? s[j][c][i] : -INFINITY;
                    }
        }
        float mu[CT];
#pragma unroll
        for (int j = 0; j < CT; ++j) {
            float mx = -INFINITY;
#pragma unroll
            for (int c = 0; c < NB; ++c)
#pragma unroll
                for (int i = 0; i < 4; ++i) mx = fmaxf(mx, s[j][c][i]);
            mx = max_over_groups(mx) * sscale;
            // lazy reference move: only when a score exceeds it by 2^8 (or on the first keys)
            const bool move = mx > mref[j] + kRescaleLog2;
            if (__ballot(move) != 0) {
                const float f = move ? (mref[j] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(mref[j] - mx)) : 1.0f;
                if (move) {
                    mref[j] = mx;
                    l_hi[j] *= f;
                    l_lo[j] *= f;
                }
                rescale_rows(j, f);
            }
            mu[j] = mref[j] == -INFINITY ? 0.0f : mref[j];
        }

        // ---- probabilities; pair r holds blocks 2r and 2r+1, element 4c' + i of it is slot
        // 4*grp + i of block 2r + c'.  One-byte caches: one fp16 term, every probability
        // (and the normaliser with it) scaled by 2^kPShift so that small ones stay normal
        // fp16 numbers.  bf16 cache: a high (pf truncated to bf16, so pf - hi is exact) and
        // a low bf16 term.
        pv_t pa[CT][NB / 2], pb[CT][kF16 ? 1 : NB / 2];
#pragma unroll
        for (int j = 0; j < CT; ++j) {
            const float mus = kF16 ? mu[j] - (float)kPShift : mu[j];
            float psum = 0.0f;
#pragma unroll
            for (int c = 0; c < NB; ++c)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float pf = __builtin_amdgcn_exp2f(__builtin_fmaf(s[j][c][i], sscale, -mus));
                    if constexpr (kF16) {
                        pa[j][c / 2][4 * (c % 2) + i] = (_Float16)pf;   // round to nearest even
                    } else {
                        const float hf = __uint_as_float(__float_as_uint(pf) & 0xFFFF0000u);
                        pa[j][c / 2][4 * (c % 2) + i] = __builtin_bit_cast(__bf16, (uint16_t)(__float_as_uint(pf) >> 16));
                        pb[j][c / 2][4 * (c % 2) + i] = (__bf16)(pf - hf);
                    }
                    psum += pf;
                }
            comp_add(l_hi[j], l_lo[j], psum);
        }

        // ---- O += P.V per channel tile (value slots past the context were zeroed when
        // staged); each value operand read feeds the products of every column tile
#pragma unroll
        for (int t = 0; t < NT; ++t) {
#pragma unroll
            for (int r = 0; r < NB / 2; ++r) {
                const pv_t v = kEarlyV ? vb[kEarlyV ? t : 0][r] : read_v(t, r);
#pragma unroll
                for (int j = 0; j < CT; ++j) {
                    oacc[j][t] = mfma16(pa[j][r], v, oacc[j][t]);
                    if constexpr (!kF16) oacc[j][t] = mfma16(pb[j][kF16 ? 0 : r], v, oacc[j][t]);
                }
            }
        }

        // ---- second level: move the matrix-core partial sums into fp32 registers
        if (++flush == S::FLUSH) {
            flush = 0;
#pragma unroll
            for (int j = 0; j < CT; ++j)
#pragma unroll
                for (int t = 0; t < NT; ++t) {
                    osum[j][t] += oacc[j][t];
                    oacc[j][t] = f32x4{};
                }
        }
    };

    // ---- the pipeline: step s+2 is loaded into registers while step s is computed from
    // one LDS buffer and step s+1 is written into the other; one barrier per step.  The
    // ids of step s+3 are read before that barrier.  The loop always runs both halves (a
    // half past the last step computes nothing and fills a buffer no one reads), so its
    // body has no early exit between a load and its use.
    ids_t ids = load_ids(0);
    const uint32_t ok0 = ok_mask(0, ids);
    stage_t ra, rb;
    stage_load(ids, ok0, ra);
    ids = load_ids(1);
    uint32_t ok1 = ok_mask(1, ids);
    stage_load(ids, ok1, rb);
    ids = load_ids(2);                     // ids of step st + 2 at the top of the loop
    stage_store(0, 0, ok0, ra);
    uint32_t okc = ok0;                    // mask of step st
    __syncthreads();
    // Waves 4-7 stage the next step before computing this one, waves 0-3 after it.  Both
    // orders are legal between two barriers (the staged buffer is not the one being computed
    // from).  Waves w and w + 4 share a SIMD, so one's staging (vector ALU work) runs beside
    // the other's S products, and its P.V products beside the other's staging.  The loop is
    // written out once per order (E), so that no branch sits inside it.
    auto run = [&](auto stage_first) __attribute__((always_inline)) {
        constexpr bool E = decltype(stage_first)::value;
        for (int st = 0; st < nsteps; st += 2) {
            uint32_t ok2 = ok_mask(st + 2, ids);
            stage_load(ids, ok2, ra);
            if constexpr (E) stage_store(1, st + 1, ok1, rb);
            compute(st, 0, okc);
            if constexpr (!E) stage_store(1, st + 1, ok1, rb);
            const ids_t ids_next = load_ids(st + 3);
            __syncthreads();
            const uint32_t ok3 = ok_mask(st + 3, ids_next);
            stage_load(ids_next, ok3, rb);
            if constexpr (E) stage_store(0, st + 2, ok2, ra);
            compute(st + 1, 1, ok1);
            if constexpr (!E) stage_store(0, st + 2, ok2, ra);
            ids = load_ids(st + 4);
            __syncthreads();
            okc = ok2;
            ok1 = ok3;
        }
    };
    if (wave >= kWaves / 2) run(std::true_type{});
    else run(std::false_type{});
    }   // nsteps > 0
    // With an error word: wave 0 checks the ids of every block some column of the workgroup
    // attends to (staged blocks with a bad id read as empty).
    if (p.err != nullptr && wave == 0 && kend > 0) {
        const ConstI32Ptr row = (ConstI32Ptr)(p.block_tables + (int64_t)b * p.max_blocks_per_seq);
        const int n_end = (kend - 1) / kBlockSize;
        bool bad = false;
        for (int n = (pwmin >= 0 ? lo_of(pwmin) : 0) / kBlockSize + lane; n <= n_end; n += 64)
            bad |= (unsigned)row[n] >= (unsigned)p.num_blocks;
        if (__any(bad) && lane == 0) report_error(p.err, kErrBlockId);
    }
    if (!wactive) return;
    const float vscale = p.v_scales != nullptr
                             ? ((const __attribute__((address_space(4))) float*)p.v_scales)[h]
                             : p.v_scale;
#pragma unroll
    for (int j = 0; j < CT; ++j) {
#pragma unroll
        for (int t = 0; t < NT; ++t) osum[j][t] += oacc[j][t];

        // ---- normalise: the column's probability sum over its four groups, then v_scale / l
        float l_tot = l_hi[j] + l_lo[j];
        l_tot += __shfl_xor(l_tot, 16);
        l_tot += __shfl_xor(l_tot, 32);
        const float inv = l_tot > 0.0f ? vscale / l_tot : 0.0f;   // no attended key: zero row
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int orow = 4 * grp + i;                          // the column this row holds
            const float f = __shfl(inv, orow);
            const int64_t oc = c0 + kCols * j + orow;
            if (oc >= ncols) continue;
            const int otok = (int)(oc / G);
            if (q0 + otok >= p.num_rows) continue;
            const int ohq = h * G + (int)(oc % G);
            const int64_t base = ((int64_t)(q0 + otok) * p.num_q_heads + ohq) * D;
#pragma unroll
            for (int t = 0; t < NT; ++t) store_out(p.out, p.out_f32, base + 16 * t + col, osum[j][t][i] * f);
        }
    }
}

template <int D>
const void* rotated_kernel(Codec codec) {
    if constexpr (col_tiles(D) == 2) {
        switch (codec) {
            case kCodecE4M3: return reinterpret_cast<const void*>(&prefill_kernel<D, kCodecE4M3, true>);
            case kCodecBF16: return reinterpret_cast<const void*>(&prefill_kernel<D, kCodecBF16, true>);
            default: return nullptr;
        }
    }
    return nullptr;   // the low query term needs the two-tile kernel's LDS query operands
}

template <int D>
hipError_t launch_d(const PrefillParams& p, Codec codec, hipStream_t s) {
    const int G = p.num_q_heads / p.num_kv_heads;
    constexpr int kWgCols = kWaves * kCols * col_tiles(D);   // query columns per workgroup
    const int64_t tiles = ((int64_t)p.max_query_len * G + kWgCols - 1) / kWgCols;
    if (tiles <= 0 || p.num_seqs <= 0) return hipSuccess;
    const int64_t groups = (int64_t)p.num_seqs * p.num_kv_heads;   // (sequence, kv head) pairs
    if (tiles * groups > 0x7FFFFFFF) return hipErrorInvalidValue;
    const void* fn;
    if (p.query_lo != nullptr) {
        fn = rotated_kernel<D>(codec);
        if (fn == nullptr) return hipErrorInvalidValue;
        return launch_kernel(fn, dim3((unsigned)(tiles * groups)), dim3(64 * kWaves), 0, s, p);
    }
    switch (codec) {
        case kCodecE4M3: fn = reinterpret_cast<const void*>(&prefill_kernel<D, kCodecE4M3>); break;
        case kCodecBF16: fn = reinterpret_cast<const void*>(&prefill_kernel<D, kCodecBF16>); break;
        case kCodecE5M2: fn = reinterpret_cast<const void*>(&prefill_kernel<D, kCodecE5M2>); break;
        case kCodecINT8: fn = reinterpret_cast<const void*>(&prefill_kernel<D, kCodecINT8>); break;
        default: return hipErrorInvalidValue;
    }
    return launch_kernel(fn, dim3((unsigned)(tiles * groups)), dim3(64 * kWaves), 0, s, p);
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
