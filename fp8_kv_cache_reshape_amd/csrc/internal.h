// internal.h -- launch parameters and launcher declarations shared by the HIP sources of
// libfp8kv.  Not part of the public ABI (that is include/fp8kv.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "codec.h"

namespace fp8kv {

constexpr int kBlockSize = 16;     // tokens per cache block (the only supported size)
constexpr int kMaxGroup = 16;      // query heads per kv head: one MFMA column tile
#ifndef FP8KV_DECODE_WAVES
#define FP8KV_DECODE_WAVES 4
#endif
#ifndef FP8KV_HEADS_FASTEST
#define FP8KV_HEADS_FASTEST 0
#endif
constexpr int kDecodeWaves = FP8KV_DECODE_WAVES;   // waves per decode workgroup
// Grid order of the partial pass: 1 puts the kv heads of one split next to each other in
// dispatch order (the tiles of all heads of a cache block are adjacent in memory).
constexpr bool kHeadsFastest = FP8KV_HEADS_FASTEST != 0;
constexpr int kMaxSplits = 1024;   // upper bound on context splits per (seq, kv head)

struct CacheWriteParams {
    const uint16_t* key;           // bf16 [T][Hkv][D]
    const uint16_t* value;
    void* key_cache;               // [NB][Hkv][16][D]
    void* value_cache;             // [NB][Hkv][D][16]
    const int64_t* slot_mapping;   // [T]
    int num_tokens;
    int num_kv_heads;
    int num_blocks;
    float k_scale;
    float v_scale;
    const float* k_scales;         // per-kv-head scales [Hkv] (device), or null: k_scale
    const float* v_scales;         // ... or null: v_scale
    unsigned int* err;             // device error word (FP8KV_DEVERR_* bits), or null
};

struct DecodeParams {
    void* out;                     // [B][Hq][D] bf16 or f32 (final output)
    int out_f32;
    const uint16_t* query;         // bf16 [B][Hq][D]
    const uint16_t* query_lo;      // bf16 [B][Hq][D]: a second (low) query term, or null
    const void* key_cache;
    const void* value_cache;
    const int32_t* block_tables;   // [B][max_blocks]
    const int32_t* context_lens;   // [B]
    int max_blocks_per_seq;
    int max_context_len;
    int num_seqs;
    int num_q_heads;
    int num_kv_heads;
    int num_blocks;
    int sliding_window;
    float score_scale;             // k_scale * log2(e) / sqrt(D): scores in base-2 units
    float v_scale;
    int splits;                    // grid extent over context splits
    int blocks_per_split;
    float* ws_ml;                  // [B][Hq][splits][2]  (m, l)
    float* ws_acc;                 // [B][Hq][splits][D]
    int write_final;               // single split: pass 1 normalises and stores `out`
    // fused decode step (all null/unused for the plain decode)
    const uint16_t* k_new;         // bf16 [B][Hkv][D]: the token at position L-1, or null
    const uint16_t* v_new;
    float k_scale_q;               // quantisation scales of the step token (fp8 caches)
    float v_scale_q;
    unsigned int* counters;        // [B][Hkv] counter records of kCounterRecordWords words (zero
                                   // between calls), or null
    int use_claims;                // with `counters`: the last pool steps are claimed at run time
    int merge_in_kernel;           // with `counters`: the last workgroup of a group merges
    // per-attention-head scales [Hkv] (device), or null for the per-tensor values above;
    // with them score_scale excludes the key scale and v_scale / k_scale_q / v_scale_q are
    // unused
    const float* k_scales;
    const float* v_scales;
    unsigned int* err;             // device error word (FP8KV_DEVERR_* bits), or null
    // rotated cache (the rotated decode step): (float)(1/sqrt(D)), the Hadamard normaliser
    float rot_scale;
};

struct PrefillParams {
    void* out;                     // [Tq][Hq][D] bf16 or f32
    int out_f32;
    const uint16_t* query;         // bf16 [Tq][Hq][D]
    const int32_t* query_start_loc;   // [B + 1]: chunk rows of sequence b
    const void* key_cache;
    const void* value_cache;
    const int32_t* block_tables;   // [B][max_blocks]
    const int32_t* context_lens;   // [B], the chunk included
    int max_blocks_per_seq;
    int max_context_len;
    int max_query_len;             // host bound on chunk lengths (sizes the grid)
    int num_seqs;
    int num_q_heads;
    int num_kv_heads;
    int num_blocks;
    int sliding_window;
    float score_scale;             // (k_scale or 1) * log2(e) / sqrt(D)
    float v_scale;
    const float* k_scales;         // per-kv-head scales [Hkv] (device), or null
    const float* v_scales;
    unsigned int* err;             // device error word (FP8KV_DEVERR_* bits), or null
    // prefill over a rotated cache: the rotated query's low bf16 term (query holds the high
    // one), or null; and the number of query rows the caller's buffers hold (rows at or past
    // it are neither read nor written; INT_MAX for the plain prefill)
    const uint16_t* query_lo;
    int num_rows;
};

// Bits of the device error word (the public FP8KV_DEVERR_* values).
constexpr unsigned int kErrBlockId = 1u;      // a block id of an attended block is out of range
constexpr unsigned int kErrSlot = 2u;         // a slot at or past num_blocks * block_size
constexpr unsigned int kErrContextLen = 4u;   // a context length that had to be clamped
constexpr unsigned int kErrQueryLen = 8u;     // a prefill chunk that does not fit its bounds

// Record a device-side input error (a vector atomic OR into the caller's word).
__device__ inline void report_error(unsigned int* err, unsigned int bits) {
    if (err != nullptr) __hip_atomic_fetch_or(err, bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The scale of kv head h: from a per-head array (a wave-uniform scalar load), or the
// per-tensor value when there is no array.
__device__ inline float head_scale(const float* per_head, int h, float per_tensor) {
    typedef const __attribute__((address_space(4))) float* ConstF32Ptr;
    return per_head != nullptr ? ((ConstF32Ptr)per_head)[h] : per_tensor;
}

// Counter record of one (sequence, kv head) group in the caller's counter buffer: the
// split arrival counter, then one step-claim counter per decode wave, each in a 256-byte
// line of its own so that no two counters share a line.  Group b*Hkv + h's record sits at
// a fixed place whatever the batch or split plan of a call.
constexpr int kCounterLineWords = 64;
constexpr int kCounterRecordWords = kCounterLineWords * (1 + kDecodeWaves);

// Context window of one sequence in blocks: positions [lo, L), blocks [blk0, blk0+nblk).
struct SeqWindow {
    int L, lo, blk0, nblk;
};

__host__ __device__ inline SeqWindow seq_window(int ctx_len, int max_context_len,
                                                int max_blocks_per_seq, int sliding_window) {
    SeqWindow w;
    int L = ctx_len;
    int cap = max_blocks_per_seq * kBlockSize;
    if (L > max_context_len) L = max_context_len;
    if (L > cap) L = cap;
    if (L < 0) L = 0;
    int lo = (sliding_window > 0 && L > sliding_window) ? L - sliding_window : 0;
    w.L = L;
    w.lo = lo;
    w.blk0 = lo / kBlockSize;
    w.nblk = (L > lo) ? (L + kBlockSize - 1) / kBlockSize - w.blk0 : 0;
    return w;
}

// Byte offset, inside a key tile, of element (slot t, channel i) for D channels of ES bytes.
// A key tile is 16 slots x D channels stored as 16-byte chunks ordered (slot quad t/4,
// chunk c, slot t%4, channel quarter g): a decode wave's key load instruction then reads
// 256 contiguous bytes per tile.  For D = 64, ES = 1 this is plain slot-major order.
template <int D, int ES>
__host__ __device__ constexpr int key_chunk_offset(int t, int i) {
    constexpr int kQuarter = D / 4;           // channels per quarter
    constexpr int kChunks = D * ES / 64;      // 16-byte chunks per quarter of one slot
    const int g = i / kQuarter;
    const int w = (i % kQuarter) * ES;        // byte within the quarter
    return (((t / 4) * kChunks + w / 16) * 4 + t % 4) * 64 + g * 16 + w % 16;
}

// Launch a kernel whose only argument is a parameter struct and return the status of this
// launch alone (hipGetLastError would also report errors other HIP users left behind).
template <typename P>
inline hipError_t launch_kernel(const void* fn, dim3 grid, dim3 block, size_t lds, hipStream_t s,
                                const P& p) {
    void* args[] = {const_cast<P*>(&p)};
    return hipLaunchKernel(fn, grid, block, args, lds, s);
}

// Remember a HIP error for fp8kv_last_hip_error (the calling thread's most recent).
void record_hip_error(hipError_t e);

// Every host check fp8kv_decode_step makes, for counter and workspace buffers of the given
// sizes, without any HIP call: FP8KV_OK or the status the step would return.
int decode_step_check(void* out, int out_dtype, const void* query, const void* key_new,
                      const void* value_new, void* key_cache, void* value_cache, int cache_dtype,
                      const int32_t* block_tables, int max_blocks_per_seq,
                      const int32_t* context_lens, int max_context_len, int num_seqs,
                      int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                      int num_blocks, float k_scale, float v_scale, int sliding_window,
                      int num_splits, size_t counters_bytes, size_t workspace_bytes);

// `codec`: the cache element codec (kCodecBF16 or a one-byte codec).
hipError_t launch_cache_write(const CacheWriteParams& p, Codec codec, int head_dim, hipStream_t s);
hipError_t launch_decode_partial(const DecodeParams& p, Codec codec, int head_dim, hipStream_t s);
// The decode kernel over a Hadamard-rotated cache (E4M3 or BF16): the query is rotated in the
// kernel, the step token (when given) rotated before it is quantised, and a merged output
// rotated back before it is stored.  Without an in-kernel merge (or a single split) the
// partials go to the workspace as usual.
hipError_t launch_decode_partial_rotated(const DecodeParams& p, Codec codec, int head_dim,
                                         hipStream_t s);
hipError_t launch_decode_merge(const DecodeParams& p, int head_dim, hipStream_t s);
// Whether the decode kernel can merge the `splits` partials of a (sequence, kv head) group
// of `group` query heads itself, in at most two batched round trips to memory; larger
// merges run in the separate merge kernel.
bool fused_merge_fits(int group, int head_dim, int splits);
hipError_t launch_prefill(const PrefillParams& p, Codec codec, int head_dim, hipStream_t s);
// Hadamard rotation (rotation.hip): the rotated cache write (CacheWriteParams' per-tensor
// scales), the query rotation into hi + lo bf16 terms, and the output rotation back.
hipError_t launch_rotate_write(const CacheWriteParams& p, Codec codec, int head_dim, hipStream_t s);
hipError_t launch_rotate_query(const uint16_t* q, uint16_t* q_hi, uint16_t* q_lo, int64_t rows,
                               int head_dim, hipStream_t s);
hipError_t launch_rotate_out(const float* in, void* out, int out_f32, int64_t rows, int head_dim,
                             hipStream_t s);

}  // namespace fp8kv
