/*
 * fp8kv.h -- C ABI of libfp8kv: an fp8 (OCP E4M3) paged KV cache and grouped-query
 * decode attention over it, for AMD Instinct MI355X (gfx950).
 *
 * Two operations, as the source pages frame the problem:
 *   - quantise-on-write: each new K/V element is divided by its tensor's scale and
 *     cast to E4M3, then stored into fixed-size cache blocks
 *     (page "FP8 KV Cache Quantization: Capacity Gains and Accuracy Risk", sections
 *     "Scales and calibration" and "Why the KV cache sets long-context capacity");
 *   - decode attention softmax(q K^T / sqrt(d)) V that reads the fp8 blocks directly,
 *     dequantising inside the kernel (same page, "Attention backend interactions"),
 *     with GQA group ratio g = Hq / Hkv (page "ctx-fp8-kv-cache-long-context-accuracy",
 *     "Arithmetic intensity"), an optional sliding window (page "FP8 KV Cache
 *     Quantization: Capacity Gains and Accuracy Risk", "Accuracy risks to test for"), and
 *     fp32 partial results merged across context splits: the
 *     two-level accumulation that keeps long contractions accurate (page "The State of
 *     FP8 KV-Cache and Attention Quantization in vLLM", "ACCURACY AT LONG CONTEXT").
 *   A bf16 cache variant of both calls keeps chosen layers in the native dtype (page
 *   "ctx-fp8-kv-cache-long-context-accuracy", "Workarounds": skipping sliding-window
 *   layers).
 *
 * Conventions for every call
 *   - All pointers except the scalars are DEVICE pointers the caller owns.  The library
 *     allocates nothing and is thread-safe.  Its only state is, per host thread, the
 *     optional device error word set by fp8kv_set_error_word (and the fixed device array of
 *     fp8kv_decode_step_noalloc, the one entry point that takes no caller buffers).
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and the call
 *     returns without synchronising.
 *   - Arguments are validated on the host before any HIP call; a failed check returns a
 *     negative status and enqueues nothing.  A failed launch returns FP8KV_ERR_HIP.
 *   - Device-resident indices (slot_mapping, block_tables, context_lens) are not read by
 *     the host.  Out-of-range values never cause an out-of-bounds access: a slot outside
 *     [0, num_blocks*block_size) is skipped, a block id outside [0, num_blocks) is read as
 *     an empty block, and a context length is clamped to
 *     min(max_context_len, max_blocks_per_seq*block_size).  Results for such inputs are
 *     otherwise unspecified; with an error word set (fp8kv_set_error_word) the kernels
 *     report them there.
 *
 * Data layout (row-major, no padding)
 *   bf16 K/V rows written per token:  [num_tokens][num_kv_heads][head_dim]
 *   query:                            [num_seqs][num_q_heads][head_dim] bf16
 *   output:                           [num_seqs][num_q_heads][head_dim] bf16 or f32
 *   key_cache, value_cache: [num_blocks][num_kv_heads] tiles of block_size*head_dim
 *     elements (one-byte codes for FP8KV_E4M3 / FP8KV_E5M2 / FP8KV_INT8, bf16 for
 *     FP8KV_BF16), each contiguous.
 *     value tile: channel-major, element (slot t, channel i) at i*block_size + t.
 *     key tile: 16-byte chunks ordered (slot quad, chunk, slot within quad, channel
 *       quarter).  With e = element bytes, q = head_dim/4, g = i/q, w = (i%q)*e and
 *       C = head_dim*e/64, element (t, i) starts at byte
 *       ((t/4 * C + w/16) * 4 + t%4) * 64 + g*16 + w%16 of the tile.  (For head_dim 64
 *       with E4M3 this is plain slot-major order.)  Both orders let one 16-byte load
 *       per lane feed the decode kernel's matrix-core operands with whole cache lines.
 *   slot_mapping: int64 [num_tokens]; token t goes to block slot/block_size, row
 *     slot%block_size.
 *   block_tables: int32 [num_seqs][max_blocks_per_seq]; logical block n of sequence b
 *     is physical block block_tables[b][n].
 *   context_lens: int32 [num_seqs]; the number of cached tokens of sequence b, counting
 *     the token written for this decode step.  Query head hq reads kv head hq / g.
 *
 * Supported shapes: head_dim in {64, 128, 256}; block_size == 16; num_q_heads a
 * multiple of num_kv_heads with g = num_q_heads/num_kv_heads <= 16.
 */
#ifndef FP8KV_H
#define FP8KV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes (return values). */
#define FP8KV_OK               0
#define FP8KV_ERR_NULL        (-1)  /* a required pointer is NULL                         */
#define FP8KV_ERR_SHAPE       (-2)  /* a size is negative or inconsistent                 */
#define FP8KV_ERR_UNSUPPORTED (-3)  /* head_dim, block_size, group ratio or dtype code     */
#define FP8KV_ERR_SCALE       (-4)  /* an fp8 scale is not finite and positive            */
#define FP8KV_ERR_WORKSPACE   (-5)  /* workspace NULL, too small, or not 256-byte aligned */
#define FP8KV_ERR_HIP         (-6)  /* a kernel launch failed                             */
#define FP8KV_ERR_SCRATCH     (-7)  /* fp8kv_decode_step_noalloc: the call needs more than
                                       its fixed device array holds                       */

/* Element type codes. */
#define FP8KV_E4M3 0   /* OCP FP8 E4M3 ("fn"): bias 7, max 448, no infinities, NaN = S.1111.111 */
#define FP8KV_BF16 1
#define FP8KV_F32  2   /* output only */
/* The other one-byte cache codecs the pages name (page "ctx-fp8-kv-cache-long-context-
 * accuracy", "Workarounds" and "notes": E5M2 and INT8 KV, no measured advantage).  Every
 * entry point that takes a cache_dtype accepts them wherever it accepts FP8KV_E4M3, with
 * the same layout, scales and error behaviour. */
#define FP8KV_E5M2 3   /* OCP FP8 E5M2: bias 15, max 57344; encoded like E4M3 (RNE, ties to even,
                          saturating at +-57344, NaN -> 0x7F | sign) */
#define FP8KV_INT8 4   /* symmetric INT8: nearest integer to x/scale, ties to even, clamped to
                          [-127, 127], NaN -> 0; two's-complement byte */

/* Human-readable name of a status code (static storage; never NULL). */
const char* fp8kv_status_string(int status);

/* Library version as MAJOR*10000 + MINOR*100 + PATCH. */
int fp8kv_version(void);

/* Name of the HIP error behind the most recent FP8KV_ERR_HIP returned on the calling
 * thread ("hipSuccess" if none).  Static storage; never NULL. */
const char* fp8kv_last_hip_error(void);

/* Bits of the device error word (see fp8kv_set_error_word). */
#define FP8KV_DEVERR_BLOCK_ID     1u  /* a block_tables entry of a block some query attends to is
                                         outside [0, num_blocks): the block was read as empty (a
                                         decode step's token was not written) */
#define FP8KV_DEVERR_SLOT         2u  /* a slot_mapping entry >= num_blocks*block_size: that token
                                         was not written (negative slots are skipped silently, as
                                         padding) */
#define FP8KV_DEVERR_CONTEXT_LEN  4u  /* a context length < 0 or above min(max_context_len,
                                         max_blocks_per_seq*block_size): it was clamped */
#define FP8KV_DEVERR_QUERY_LEN    8u  /* prefill: query_start_loc decreases, or a chunk is longer
                                         than max_query_len (its rows past that are not computed) */

/*
 * fp8kv_set_error_word -- from now on, kernels enqueued by the calling host thread OR the
 * FP8KV_DEVERR_* bits above into *word (a device uint32, 4-byte aligned, owned by the
 * caller) when they meet device-resident inputs that break the preconditions stated below;
 * NULL (the initial state) switches reporting off.  The library never clears the word:
 * zero it, run the calls, then read it after the stream has reached that point.  Reports
 * are atomic ORs made only when an error is found (prefill also reads the attended block
 * ids once more per workgroup while a word is set).  The pointer is per host thread.
 * Returns FP8KV_OK, or FP8KV_ERR_SHAPE for a misaligned word.
 */
int fp8kv_set_error_word(unsigned int* word);

/*
 * fp8kv_cache_write -- quantise new K/V rows and scatter them into the paged caches.
 *
 * For every token t with a valid slot, kv head h and channel i:
 *   E4M3 caches: code = E4M3(f32(x) / scale), where "/" is the IEEE-754 binary32 division
 *     (round to nearest even) and E4M3() rounds to nearest with ties to the even code,
 *     saturates magnitudes >= 448 (and infinities) to +-448, keeps the sign of zero, and
 *     maps NaN to 0x7F | sign.  k uses k_scale, v uses v_scale (page "FP8 KV Cache
 *     Quantization: Capacity Gains and Accuracy Risk", "Scales and calibration": one
 *     scale per tensor, elements divided by it before the cast).
 *   E5M2 / INT8 caches: the same f32 division, then that codec's cast (see the codes).
 *   BF16 caches: the bf16 bits are stored unchanged; the scales are ignored.
 * Bytes of the caches that no valid slot addresses are left untouched.  Two tokens that
 * name the same slot race; the result is one of the two rows.
 *
 *   key, value      device bf16 [num_tokens][num_kv_heads][head_dim]
 *   key_cache,
 *   value_cache     device caches in the layout above, of cache_dtype elements
 *   slot_mapping    device int64 [num_tokens]
 *   num_tokens      >= 0 (0 enqueues nothing)
 *   k_scale,v_scale finite and > 0 for the one-byte codecs (else FP8KV_ERR_SCALE)
 */
int fp8kv_cache_write(const void* key, const void* value,
                      void* key_cache, void* value_cache, int cache_dtype,
                      const int64_t* slot_mapping, int num_tokens,
                      int num_kv_heads, int head_dim, int block_size, int num_blocks,
                      float k_scale, float v_scale, void* stream);

/*
 * fp8kv_cache_write_per_head -- fp8kv_cache_write with one key and one value scale per kv
 * head: elements of kv head h are divided by k_scales[h] / v_scales[h] (page "FP8 KV Cache
 * Quantization: Capacity Gains and Accuracy Risk", "Scales and calibration": the
 * per-attention-head granularity, scale arrays of length num_kv_heads).  Rounding,
 * saturation, layout, slot handling and the BF16 case (scales ignored) as above.
 *
 *   k_scales, v_scales  device float32 [num_kv_heads], 4-byte aligned, read by the kernel
 *                       on `stream`; the caller owns them.  For FP8KV_E4M3 both must be
 *                       non-NULL (else FP8KV_ERR_NULL; misaligned: FP8KV_ERR_SHAPE) and
 *                       every entry finite and > 0 -- a precondition the library does not
 *                       check (it does not read device memory on the host).  Ignored for
 *                       FP8KV_BF16 (may be NULL).
 */
int fp8kv_cache_write_per_head(const void* key, const void* value,
                               void* key_cache, void* value_cache, int cache_dtype,
                               const int64_t* slot_mapping, int num_tokens,
                               int num_kv_heads, int head_dim, int block_size, int num_blocks,
                               const float* k_scales, const float* v_scales, void* stream);

/*
 * fp8kv_paged_decode_num_splits -- number of context splits a decode will use.
 *
 * The context window of every (sequence, kv head) is cut into splits of a fixed number
 * of blocks; each split yields fp32 partials (running max m, sum l, unnormalised
 * accumulator acc[head_dim]) that a second pass merges.  num_splits > 0 requests at most
 * that many splits for the longest sequence; 0 lets the library choose.  Returns the
 * split count (>= 1) or a negative status.
 *
 * Reproducibility (decode calls that take a counter buffer): with num_splits > 0 every
 * workgroup's share of the context is fixed by the arguments and every merge sums in a
 * fixed order, so the output is bit-for-bit the same on every run.  With num_splits = 0 and
 * a counter buffer the last context steps of each (sequence, kv head) are handed at run
 * time to whichever workgroup is free (load balancing across compute units), so the fp32
 * summation order, and the last bits of the output, may differ from run to run, within the
 * accuracy stated for fp8kv_paged_decode.  Calls without a counter buffer are always
 * reproducible.
 */
int fp8kv_paged_decode_num_splits(int num_seqs, int num_kv_heads, int head_dim,
                                  int block_size, int max_context_len, int sliding_window,
                                  int num_splits);

/*
 * fp8kv_paged_decode_workspace_size -- bytes of device workspace a decode (or decode step)
 * with these arguments needs (0 on invalid arguments).  The workspace holds the fp32 split
 * partials: num_seqs * num_q_heads * splits * (head_dim + 2) floats, rounded up.  Its
 * contents on entry never matter.
 */
size_t fp8kv_paged_decode_workspace_size(int num_seqs, int num_q_heads, int num_kv_heads,
                                         int head_dim, int block_size, int max_context_len,
                                         int sliding_window, int num_splits);

/*
 * fp8kv_decode_counters_size -- bytes of the counter buffer that decode calls with up to
 * max_num_seqs sequences of num_kv_heads kv heads use (0 on invalid arguments):
 * max_num_seqs * num_kv_heads records of 1280 bytes.  The record of (sequence b, kv head h)
 * sits at byte (b*num_kv_heads + h)*1280 whatever the batch, split plan or window of a call;
 * it holds the split arrival counter and four step-claim counters, each in a 256-byte line.
 *
 * Contract: allocate the buffer once for the largest batch, 256-byte aligned, and zero it
 * before its first use.  Every call leaves the records it used at zero again, so the buffer
 * serves any later call with at most max_num_seqs sequences (of the same or fewer kv heads)
 * with no clearing in between.  It holds counters only (no partials).  Calls that share a
 * counter buffer must not run concurrently; give each stream its own.
 */
size_t fp8kv_decode_counters_size(int max_num_seqs, int num_kv_heads);

/*
 * fp8kv_paged_decode -- one decode step of GQA attention over the paged cache.
 *
 * For each sequence b and query head hq, with h = hq / g, L = min(context_lens[b],
 * max_context_len, max_blocks_per_seq*block_size) and lo = (sliding_window > 0) ?
 * max(0, L - sliding_window) : 0:
 *   K_j = dequant(key_cache row of position j) * k_scale,  V_j likewise with v_scale,
 *   s_j = q . K_j / sqrt(head_dim)  for j in [lo, L),
 *   out = sum_j exp(s_j - max s) V_j / sum_j exp(s_j - max s);   out = 0 if L <= lo.
 * (For FP8KV_BF16 caches K_j and V_j are the stored bf16 values and the scales are
 * ignored.)  Arithmetic: fp8 -> bf16 conversion is exact; q.K and p.V products are
 * formed on the matrix cores with fp32 accumulation; softmax statistics and all merges
 * are fp32; p enters the p.V product as the sum of two bf16 values (about 16 significant
 * bits).  The output is rounded to bf16 with round-to-nearest-even (or stored as f32).
 *
 *   out           device [num_seqs][num_q_heads][head_dim] of out_dtype (BF16 or F32)
 *   query         device bf16 [num_seqs][num_q_heads][head_dim]
 *   key_cache,
 *   value_cache   device caches of cache_dtype (E4M3 or BF16), num_blocks blocks
 *                 (num_blocks >= 1 and max_blocks_per_seq >= 1 when max_context_len > 0)
 *   block_tables  device int32 [num_seqs][max_blocks_per_seq]
 *   context_lens  device int32 [num_seqs]
 *   max_context_len  host upper bound on context_lens (sizes the grid and workspace)
 *   sliding_window   0 = full attention, W > 0 = the last W positions
 *   num_splits    0 = automatic, else requested split count (see above)
 *   counters      optional (NULL: none).  A counter buffer (fp8kv_decode_counters_size,
 *                 with its zero-on-entry contract) of at least num_seqs*num_kv_heads
 *                 records: the last workgroup of each (sequence, kv head) to finish then
 *                 merges the split partials inside the decode kernel, and no separate merge
 *                 launch follows (except for groups with more partials than one workgroup
 *                 merges quickly -- more than 64 splits, or more than 32 float4 per thread);
 *                 see fp8kv_paged_decode_num_splits for reproducibility.  Without it the
 *                 partials are merged by a second kernel launch on `stream`.
 *   workspace     device buffer of at least fp8kv_paged_decode_workspace_size() bytes,
 *                 256-byte aligned; may be NULL when that size is 0.  Its contents on
 *                 entry do not matter; on return it holds the split partials.
 * Errors: FP8KV_ERR_WORKSPACE also for a counter buffer that is too small or not 256-byte
 * aligned (checked only when the call uses more than one split).
 */
int fp8kv_paged_decode(void* out, int out_dtype, const void* query,
                       const void* key_cache, const void* value_cache, int cache_dtype,
                       const int32_t* block_tables, int max_blocks_per_seq,
                       const int32_t* context_lens, int max_context_len,
                       int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                       int block_size, int num_blocks,
                       float k_scale, float v_scale, int sliding_window, int num_splits,
                       void* counters, size_t counters_bytes,
                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * fp8kv_paged_decode_per_head -- fp8kv_paged_decode with per-kv-head scales: for query
 * head hq, K_j and V_j are dequantised with k_scales[h] and v_scales[h], h = hq / g (page
 * "FP8 KV Cache Quantization: Capacity Gains and Accuracy Risk", "Scales and
 * calibration", per-attention-head granularity).  The key scale multiplies
 * log2(e)/sqrt(head_dim) (rounded to float) inside the kernel; the value scale multiplies
 * the merged output.  k_scales / v_scales as for fp8kv_cache_write_per_head; every other
 * argument, the counters, the workspace and the error behaviour as for fp8kv_paged_decode.
 */
int fp8kv_paged_decode_per_head(void* out, int out_dtype, const void* query,
                                const void* key_cache, const void* value_cache, int cache_dtype,
                                const int32_t* block_tables, int max_blocks_per_seq,
                                const int32_t* context_lens, int max_context_len,
                                int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                                int block_size, int num_blocks,
                                const float* k_scales, const float* v_scales,
                                int sliding_window, int num_splits,
                                void* counters, size_t counters_bytes,
                                void* workspace, size_t workspace_bytes, void* stream);

/*
 * fp8kv_paged_decode_partial -- the first pass of fp8kv_paged_decode alone: writes the
 * fp32 split partials (m, l, acc) of every (sequence, query head, split) into the
 * workspace and nothing else.  Partials of different context ranges combine exactly
 * like splits, so a sequence whose blocks are spread over several devices can run this
 * pass per device, gather the partials, and finish with fp8kv_paged_decode_merge.
 * Arguments as for fp8kv_paged_decode (v_scale is applied by the merge).  The partial
 * m is kept in base-2 units: m = max_j s_j * log2(e).  The _per_head variants below take
 * one key (partial pass) and one value (merge) scale per kv head.
 */
int fp8kv_paged_decode_partial(const void* query,
                               const void* key_cache, const void* value_cache, int cache_dtype,
                               const int32_t* block_tables, int max_blocks_per_seq,
                               const int32_t* context_lens, int max_context_len,
                               int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                               int block_size, int num_blocks,
                               float k_scale, int sliding_window, int num_splits,
                               void* workspace, size_t workspace_bytes, void* stream);

/*
 * fp8kv_paged_decode_merge -- the second pass: log-sum-exp merge of the split partials
 * in the workspace, multiplication by v_scale, normalisation, and the store to `out`.
 * Must be called with the same shape, window and num_splits arguments as the partial
 * pass that filled the workspace, on the same stream (or after it completes).
 */
int fp8kv_paged_decode_merge(void* out, int out_dtype,
                             const int32_t* context_lens, int max_context_len,
                             int max_blocks_per_seq, int num_seqs, int num_q_heads,
                             int num_kv_heads, int head_dim, int block_size,
                             float v_scale, int sliding_window, int num_splits,
                             const void* workspace, size_t workspace_bytes, void* stream);

/*
 * fp8kv_paged_decode_partial_per_head / fp8kv_paged_decode_merge_per_head -- the two passes
 * with per-kv-head scales (page "FP8 KV Cache Quantization: Capacity Gains and Accuracy
 * Risk", "Scales and calibration"): the partial pass dequantises the keys of kv head h with
 * k_scales[h], the merge multiplies the merged output of query head hq by v_scales[hq / g].
 * Together they equal fp8kv_paged_decode_per_head without a counter buffer.  k_scales /
 * v_scales: device float32 [num_kv_heads], 4-byte aligned, read on `stream` (for one-byte
 * caches the array must be non-NULL and its entries finite and > 0; ignored for
 * FP8KV_BF16).  Everything else as for the per-tensor passes.
 */
int fp8kv_paged_decode_partial_per_head(const void* query,
                                        const void* key_cache, const void* value_cache,
                                        int cache_dtype, const int32_t* block_tables,
                                        int max_blocks_per_seq, const int32_t* context_lens,
                                        int max_context_len, int num_seqs, int num_q_heads,
                                        int num_kv_heads, int head_dim, int block_size,
                                        int num_blocks, const float* k_scales,
                                        int sliding_window, int num_splits,
                                        void* workspace, size_t workspace_bytes, void* stream);
int fp8kv_paged_decode_merge_per_head(void* out, int out_dtype, int cache_dtype,
                                      const int32_t* context_lens, int max_context_len,
                                      int max_blocks_per_seq, int num_seqs, int num_q_heads,
                                      int num_kv_heads, int head_dim, int block_size,
                                      const float* v_scales, int sliding_window, int num_splits,
                                      const void* workspace, size_t workspace_bytes,
                                      void* stream);

/*
 * fp8kv_decode_step -- one whole decode step: write each sequence's new token into the
 * cache, then decode attention over the cache, normally in a single kernel launch (when the
 * split partials of one (sequence, kv head) are too many for one workgroup to merge
 * quickly -- more than 64 splits, or more than 32 float4 per thread -- a second, merge
 * launch follows on `stream`).
 *
 * Equivalent to fp8kv_cache_write(key_new, value_new, ...) with num_tokens = num_seqs and
 * slot_mapping[b] = block_tables[b][(L_b-1)/16]*16 + (L_b-1)%16 for every sequence with
 * L_b >= 1 (L_b as clamped in fp8kv_paged_decode; sequences with L_b = 0 write nothing,
 * and a block id outside [0, num_blocks) writes nothing), followed by
 * fp8kv_paged_decode(...) with the same arguments and the counter buffer.  The bytes written
 * are identical; the output agrees with the two-call path to within fp32 rounding (the split
 * partials are combined by the last workgroup of each (sequence, kv head) to finish, in a
 * different order from the merge kernel).  Reproducibility as stated at
 * fp8kv_paged_decode_num_splits: bit-for-bit with num_splits > 0; with num_splits = 0 the
 * run-time step claims may change the last bits from run to run.
 *
 *   key_new, value_new  device bf16 [num_seqs][num_kv_heads][head_dim]: the token at
 *                       position L_b - 1 of every sequence.  The block holding position
 *                       L_b - 1 must belong to sequence b alone (as with any write, two
 *                       sequences may not write one slot).
 *   key_cache,
 *   value_cache         written and read
 *   counters            a counter buffer of at least num_seqs*num_kv_heads records (see
 *                       fp8kv_decode_counters_size and its zero-on-entry contract); required
 *                       when the call uses more than one split, else it may be NULL.
 *   workspace           at least fp8kv_paged_decode_workspace_size() bytes, 256-byte
 *                       aligned, contents on entry irrelevant (it receives the partials).
 * Other arguments, layout and error behaviour as for fp8kv_paged_decode.
 */
int fp8kv_decode_step(void* out, int out_dtype, const void* query,
                      const void* key_new, const void* value_new,
                      void* key_cache, void* value_cache, int cache_dtype,
                      const int32_t* block_tables, int max_blocks_per_seq,
                      const int32_t* context_lens, int max_context_len,
                      int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                      int block_size, int num_blocks,
                      float k_scale, float v_scale, int sliding_window, int num_splits,
                      void* counters, size_t counters_bytes,
                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * fp8kv_decode_step_per_head -- fp8kv_decode_step with per-kv-head scales: the new token
 * of kv head h is quantised with k_scales[h] / v_scales[h] exactly as
 * fp8kv_cache_write_per_head does, and the attention dequantises as
 * fp8kv_paged_decode_per_head does (page "FP8 KV Cache Quantization: Capacity Gains and
 * Accuracy Risk", "Scales and calibration").  k_scales / v_scales as for
 * fp8kv_cache_write_per_head; everything else, the counters and workspace included, as for
 * fp8kv_decode_step.
 */
int fp8kv_decode_step_per_head(void* out, int out_dtype, const void* query,
                               const void* key_new, const void* value_new,
                               void* key_cache, void* value_cache, int cache_dtype,
                               const int32_t* block_tables, int max_blocks_per_seq,
                               const int32_t* context_lens, int max_context_len,
                               int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                               int block_size, int num_blocks,
                               const float* k_scales, const float* v_scales,
                               int sliding_window, int num_splits,
                               void* counters, size_t counters_bytes,
                               void* workspace, size_t workspace_bytes, void* stream);

/*
 * fp8kv_decode_step_noalloc -- fp8kv_decode_step with no counter buffer and no workspace, for
 * callers that cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation).  The split counters and partials live in a fixed
 * 16 MiB device array of the library, one per GPU, held until the process ends: counter
 * records for up to FP8KV_NOALLOC_MAX_GROUPS (sequence, kv head) groups and up to
 * FP8KV_NOALLOC_MAX_PARTIAL_BYTES of partials (fp8kv_paged_decode_workspace_size of the
 * call).  A call over either limit returns FP8KV_ERR_SCRATCH and enqueues nothing.  The call
 * allocates nothing (no hipMalloc, no allocating library routine).
 *
 * The array belongs to the current device (hipGetDevice) of the calling thread; `stream`
 * must be a stream of that device.  The first call on a device looks up the array's address
 * and enqueues a clear of its counter region on `stream`, before its own kernel; every call
 * leaves the counters zero again.  All calls on one device share the array: calls that
 * overlap in time on one GPU (other streams, other threads) race and give wrong results --
 * serialise them (one stream), or use fp8kv_decode_step with buffers of their own.
 * Arguments, results, reproducibility and errors otherwise as for fp8kv_decode_step.
 */
#define FP8KV_NOALLOC_MAX_GROUPS        2048
#define FP8KV_NOALLOC_MAX_PARTIAL_BYTES ((size_t)14155776)   /* 16 MiB - 2048 * 1280 */
int fp8kv_decode_step_noalloc(void* out, int out_dtype, const void* query,
                              const void* key_new, const void* value_new,
                              void* key_cache, void* value_cache, int cache_dtype,
                              const int32_t* block_tables, int max_blocks_per_seq,
                              const int32_t* context_lens, int max_context_len,
                              int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                              int block_size, int num_blocks,
                              float k_scale, float v_scale, int sliding_window, int num_splits,
                              void* stream);

/*
 * fp8kv_paged_prefill -- prefill / chunked-prefill attention over the paged cache: the
 * query tokens of each sequence's prompt chunk attend causally to its cached context, the
 * chunk included, with K and V dequantised inside the kernel (page "FP8 KV Cache
 * Quantization: Capacity Gains and Accuracy Risk", "Attention backend interactions"); the
 * contraction over the context keeps two-level accumulation (page "The State of FP8
 * KV-Cache and Attention Quantization in vLLM", "ACCURACY AT LONG CONTEXT").
 *
 * Sequence b's chunk is the query rows [query_start_loc[b], query_start_loc[b+1]); its
 * n_b tokens are the last n_b positions of the context, L_b = context_lens[b] (clamped as
 * in fp8kv_paged_decode), so row query_start_loc[b] + j sits at position
 * p = L_b - n_b + j.  For every such row and query head hq (h = hq / g):
 *   lo = (sliding_window > 0) ? max(0, p + 1 - sliding_window) : 0,
 *   s_j = q . K_j / sqrt(head_dim) for j in [lo, p],
 *   out = sum_j exp(s_j - max s) V_j / sum_j exp(s_j - max s);   out = 0 if p < 0.
 * K_j and V_j as in fp8kv_paged_decode.  The chunk's own K/V must already be in the cache
 * (fp8kv_cache_write first, on the same stream).  Arithmetic: S = K.Q^T and O = P.V on
 * the matrix cores with fp32 accumulation.  S takes bf16 operands.  With a one-byte cache
 * P.V takes fp16 operands: the codes are exact fp16 values and each probability is
 * rounded once to fp16 (11 significant bits); with the bf16 cache P.V takes bf16 operands
 * and each probability enters as the sum of two bf16 values (about 16 significant bits).
 * The matrix-core accumulator holds at most 256 keys before its sums move into fp32
 * registers.
 *
 *   out              device [num_query_tokens][num_q_heads][head_dim] of out_dtype
 *   query            device bf16 [num_query_tokens][num_q_heads][head_dim]
 *   query_start_loc  device int32 [num_seqs + 1], non-decreasing, query_start_loc[0] = 0
 *   max_query_len    host bound on every n_b (sizes the grid; rows beyond it are not
 *                    computed)
 *   other arguments as for fp8kv_paged_decode; no workspace.  num_seqs and num_kv_heads
 *   are at most 65535 (else FP8KV_ERR_UNSUPPORTED).
 */
int fp8kv_paged_prefill(void* out, int out_dtype, const void* query,
                        const int32_t* query_start_loc,
                        const void* key_cache, const void* value_cache, int cache_dtype,
                        const int32_t* block_tables, int max_blocks_per_seq,
                        const int32_t* context_lens, int max_context_len,
                        int num_seqs, int max_query_len, int num_q_heads, int num_kv_heads,
                        int head_dim, int block_size, int num_blocks,
                        float k_scale, float v_scale, int sliding_window, void* stream);

/*
 * fp8kv_paged_prefill_per_head -- fp8kv_paged_prefill with per-kv-head scales (page "FP8
 * KV Cache Quantization: Capacity Gains and Accuracy Risk", "Scales and calibration"):
 * k_scales / v_scales as for fp8kv_cache_write_per_head, applied as in
 * fp8kv_paged_decode_per_head.
 */
int fp8kv_paged_prefill_per_head(void* out, int out_dtype, const void* query,
                                 const int32_t* query_start_loc,
                                 const void* key_cache, const void* value_cache, int cache_dtype,
                                 const int32_t* block_tables, int max_blocks_per_seq,
                                 const int32_t* context_lens, int max_context_len,
                                 int num_seqs, int max_query_len, int num_q_heads,
                                 int num_kv_heads, int head_dim, int block_size, int num_blocks,
                                 const float* k_scales, const float* v_scales,
                                 int sliding_window, void* stream);

/*
 * Hadamard rotation around the cache (page "KV Cache Quantization: What FP8 and q8_0 Cost
 * in Accuracy", paragraph on the llama.cpp rotation merged on 2026-04-01): K and V rows
 * are rotated by the normalized Sylvester Hadamard matrix H/sqrt(d) before they are cached,
 * attention runs in the rotated space with the query rotated the same way, and the output
 * is rotated back.  Dot products are unchanged; outliers spread across coordinates, which
 * lowers the quantisation error of per-tensor scales.  A cache written by
 * fp8kv_cache_write_rotated must be read by fp8kv_paged_decode_rotated (and vice versa);
 * scales should be calibrated on the rotated rows.  Cache dtypes: FP8KV_E4M3 and FP8KV_BF16
 * (others: FP8KV_ERR_UNSUPPORTED).
 *
 * fp8kv_cache_write_rotated -- fp8kv_cache_write of rotated rows.  Each row x (d elements
 * of one token and kv head, widened to f32) becomes y = R(x): the fast Walsh-Hadamard
 * butterflies in f32 in the order h = 1, 2, ..., d/2 (each pair of a 2h-block becomes
 * (a + b, a - b), one rounding each), then each element times the f32 constant
 * (float)(1/sqrt(d)).  E4M3 caches store E4M3(y / scale) exactly as fp8kv_cache_write does
 * for an f32 input; BF16 caches store bf16(y) (round to nearest even).  Arguments, layout
 * and errors as for fp8kv_cache_write.
 */
int fp8kv_cache_write_rotated(const void* key, const void* value,
                              void* key_cache, void* value_cache, int cache_dtype,
                              const int64_t* slot_mapping, int num_tokens,
                              int num_kv_heads, int head_dim, int block_size, int num_blocks,
                              float k_scale, float v_scale, void* stream);

/*
 * fp8kv_paged_decode_rotated_workspace_size -- bytes of device workspace
 * fp8kv_paged_decode_rotated needs (0 on invalid arguments): the decode's split partials,
 * the rotated query (two bf16 terms) and the f32 output before it is rotated back.
 */
size_t fp8kv_paged_decode_rotated_workspace_size(int num_seqs, int num_q_heads,
                                                 int num_kv_heads, int head_dim,
                                                 int block_size, int max_context_len,
                                                 int sliding_window, int num_splits);

/*
 * fp8kv_paged_decode_rotated -- fp8kv_paged_decode over a rotated cache:
 *   out = H/sqrt(d) . Attention(H/sqrt(d) . q, K_rot, V_rot)
 * with K_rot, V_rot the dequantised rotated rows.  The query is rotated in f32 and enters
 * S = K.q^T as the sum of two bf16 terms (one bf16 term alone would move the scores by up
 * to 2^-9 relative); the output is rotated back from f32.  Three launches on `stream`
 * (query rotation, decode, output rotation; four with a separate merge).  workspace: at
 * least fp8kv_paged_decode_rotated_workspace_size() bytes, 256-byte aligned, contents on
 * entry irrelevant.  Other arguments, layout and errors as for fp8kv_paged_decode
 * (per-tensor scales).
 */
int fp8kv_paged_decode_rotated(void* out, int out_dtype, const void* query,
                               const void* key_cache, const void* value_cache, int cache_dtype,
                               const int32_t* block_tables, int max_blocks_per_seq,
                               const int32_t* context_lens, int max_context_len,
                               int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                               int block_size, int num_blocks,
                               float k_scale, float v_scale, int sliding_window, int num_splits,
                               void* workspace, size_t workspace_bytes, void* stream);

/*
 * fp8kv_decode_step_rotated -- one whole decode step over a rotated cache, normally in a
 * single kernel launch: each sequence's new K/V token is rotated and written exactly as
 * fp8kv_cache_write_rotated writes it (same f32 butterflies, same division and cast), the
 * query is rotated inside the kernel into the same two bf16 terms fp8kv_paged_decode_rotated
 * uses, and the merged output is rotated back before it is stored:
 *   out = H/sqrt(d) . Attention(H/sqrt(d) . q, K_rot, V_rot).
 * When the split partials of a (sequence, kv head) are more than one workgroup merges
 * quickly (as in fp8kv_decode_step), the merge kernel writes f32 rows into the workspace and
 * one more launch rotates them back.  Token rows, slots, counters, reproducibility and errors
 * as for fp8kv_decode_step; per-tensor scales; cache dtypes FP8KV_E4M3 and FP8KV_BF16 (else
 * FP8KV_ERR_UNSUPPORTED).
 *
 *   workspace  at least fp8kv_paged_decode_rotated_workspace_size() bytes, 256-byte aligned,
 *              contents on entry irrelevant.
 */
int fp8kv_decode_step_rotated(void* out, int out_dtype, const void* query,
                              const void* key_new, const void* value_new,
                              void* key_cache, void* value_cache, int cache_dtype,
                              const int32_t* block_tables, int max_blocks_per_seq,
                              const int32_t* context_lens, int max_context_len,
                              int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                              int block_size, int num_blocks,
                              float k_scale, float v_scale, int sliding_window, int num_splits,
                              void* counters, size_t counters_bytes,
                              void* workspace, size_t workspace_bytes, void* stream);

/*
 * fp8kv_paged_prefill_rotated_workspace_size -- bytes of device workspace
 * fp8kv_paged_prefill_rotated needs for num_query_tokens query rows (0 on invalid
 * arguments): the rotated query (two bf16 terms) and the f32 output before it is rotated
 * back.
 */
size_t fp8kv_paged_prefill_rotated_workspace_size(int num_query_tokens, int num_q_heads,
                                                  int head_dim);

/*
 * fp8kv_paged_prefill_rotated -- fp8kv_paged_prefill over a rotated cache: every chunk row
 *   out = H/sqrt(d) . Attention(H/sqrt(d) . q, K_rot, V_rot)
 * over its causal prefix, as fp8kv_paged_decode_rotated computes it for one token: the
 * query rotated in f32 and split into two bf16 terms that both enter S = K.q^T, the
 * output rotated back from f32.  Three launches on `stream` (query rotation, prefill,
 * output rotation).
 *
 *   num_query_tokens  host count of query rows, query_start_loc[num_seqs]; rows at or past
 *                     it are neither read nor written
 *   workspace         at least fp8kv_paged_prefill_rotated_workspace_size(num_query_tokens,
 *                     num_q_heads, head_dim) bytes, 256-byte aligned, contents on entry
 *                     irrelevant (else FP8KV_ERR_WORKSPACE)
 *
 * Cache dtypes FP8KV_E4M3 and FP8KV_BF16, head_dim 64 or 128 (the low query term lives in
 * the LDS query operands of the kernel's two-column-tile form; head_dim 256:
 * FP8KV_ERR_UNSUPPORTED).  Per-tensor scales; everything else as for fp8kv_paged_prefill.
 */
int fp8kv_paged_prefill_rotated(void* out, int out_dtype, const void* query,
                                const int32_t* query_start_loc,
                                const void* key_cache, const void* value_cache, int cache_dtype,
                                const int32_t* block_tables, int max_blocks_per_seq,
                                const int32_t* context_lens, int max_context_len,
                                int num_seqs, int max_query_len, int num_query_tokens,
                                int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                                int num_blocks, float k_scale, float v_scale, int sliding_window,
                                void* workspace, size_t workspace_bytes, void* stream);

/*
 * Per-kv-head scales on the rotated path (page "FP8 KV Cache Quantization: Capacity Gains
 * and Accuracy Risk", "Scales and calibration", combined with the rotation above):
 * fp8kv_cache_write_rotated_per_head, fp8kv_paged_decode_rotated_per_head and
 * fp8kv_decode_step_rotated_per_head are the three rotated calls with k_scales / v_scales
 * as for fp8kv_cache_write_per_head (device float32 [num_kv_heads] each, 4-byte aligned,
 * caller-owned; null: FP8KV_ERR_NULL; read by the kernels, not validated on the host): kv
 * head h's rotated rows are divided by k_scales[h] / v_scales[h] before the cast, and its
 * codes are dequantised with the same two scales.  Calibrate them on the rotated rows of
 * each head.  Everything else as for the per-tensor calls.
 */
int fp8kv_cache_write_rotated_per_head(const void* key, const void* value,
                                       void* key_cache, void* value_cache, int cache_dtype,
                                       const int64_t* slot_mapping, int num_tokens,
                                       int num_kv_heads, int head_dim, int block_size,
                                       int num_blocks, const float* k_scales,
                                       const float* v_scales, void* stream);

int fp8kv_paged_decode_rotated_per_head(void* out, int out_dtype, const void* query,
                                        const void* key_cache, const void* value_cache,
                                        int cache_dtype, const int32_t* block_tables,
                                        int max_blocks_per_seq, const int32_t* context_lens,
                                        int max_context_len, int num_seqs, int num_q_heads,
                                        int num_kv_heads, int head_dim, int block_size,
                                        int num_blocks, const float* k_scales,
                                        const float* v_scales, int sliding_window,
                                        int num_splits, void* workspace, size_t workspace_bytes,
                                        void* stream);

int fp8kv_decode_step_rotated_per_head(void* out, int out_dtype, const void* query,
                                       const void* key_new, const void* value_new,
                                       void* key_cache, void* value_cache, int cache_dtype,
                                       const int32_t* block_tables, int max_blocks_per_seq,
                                       const int32_t* context_lens, int max_context_len,
                                       int num_seqs, int num_q_heads, int num_kv_heads,
                                       int head_dim, int block_size, int num_blocks,
                                       const float* k_scales, const float* v_scales,
                                       int sliding_window, int num_splits, void* counters,
                                       size_t counters_bytes, void* workspace,
                                       size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FP8KV_H */
