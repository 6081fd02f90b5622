// api.hip -- the extern "C" entry points of libfp8kv (declared in include/fp8kv.h):
// host-side validation (before any HIP call), split planning, workspace layout, and the
// kernel launches on the caller's stream.
#include <limits.h>
#include <math.h>
#include <stddef.h>
#include <stdint.h>

#include "fp8kv.h"
#include "internal.h"

namespace {

using fp8kv::kBlockSize;
using fp8kv::kMaxGroup;
using fp8kv::kMaxSplits;

// Workgroups the automatic split plan aims for: one long-lived decode workgroup per compute
// unit, or two at head_dim 64, whose wave steps carry half the bytes (so twice the waves keep
// as many bytes in flight; the kernel's registers allow it).  Measured: gpt-oss shape
// (d 64, 8 x 20K) 35.2 us at 256 workgroups, 33.9 us at 512.
inline int target_workgroups(int head_dim) { return head_dim <= 64 ? 512 : 256; }
constexpr int kMinBlocksPerSplit = 16;    // one wave step (4 blocks) for each of 4 waves
// Automatic planning keeps one split up to this many blocks per (sequence, kv head): a
// 512-position window straddles at most 33 blocks, at most 3 wave steps per wave of one
// workgroup.  A second split costs a merge -- the arrival count, then one round trip for
// partials written on other XCDs -- measured at 2.5-4.6 us on such layers (d256 512-window
// layer 13.1 us per step with one split, 17.7 with three), while at 64 blocks the best
// count depends on the batch.
constexpr int kSingleSplitBlocks = 2 * kMinBlocksPerSplit + 1;

bool head_dim_ok(int d) { return d == 64 || d == 128 || d == 256; }
bool cache_dtype_ok(int d) {
    return d == FP8KV_E4M3 || d == FP8KV_BF16 || d == FP8KV_E5M2 || d == FP8KV_INT8;
}
// The C-ABI element codes are the kernels' codec values.
fp8kv::Codec codec_of(int cache_dtype) { return static_cast<fp8kv::Codec>(cache_dtype); }
static_assert(FP8KV_E4M3 == fp8kv::kCodecE4M3 && FP8KV_BF16 == fp8kv::kCodecBF16 &&
                  FP8KV_E5M2 == fp8kv::kCodecE5M2 && FP8KV_INT8 == fp8kv::kCodecINT8,
              "element codes and codecs must agree");
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool scale_ok(float s) { return isfinite(s) && s > 0.0f; }

// Scales of one call: per tensor (arrays null) or per kv head (device arrays of num_kv_heads
// floats, whose values the kernels read; they are not inspected here).
struct Scales {
    float k, v;
    const float* ks;
    const float* vs;
    bool per_head() const { return ks != nullptr || vs != nullptr; }
};

Scales tensor_scales(float k, float v) { return Scales{k, v, nullptr, nullptr}; }
Scales head_scales(const float* ks, const float* vs) { return Scales{1.0f, 1.0f, ks, vs}; }

bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

// Validation shared by every entry point that takes scales, for an fp8 cache (a bf16 cache
// ignores them).  A per-head call must give both arrays.
int check_scales(const Scales& sc, bool per_head_call) {
    if (per_head_call) {
        if (!sc.ks || !sc.vs) return FP8KV_ERR_NULL;
        if (!aligned4(sc.ks) || !aligned4(sc.vs)) return FP8KV_ERR_SHAPE;
        return FP8KV_OK;
    }
    return scale_ok(sc.k) && scale_ok(sc.v) ? FP8KV_OK : FP8KV_ERR_SCALE;
}

int check_decode_shape(int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                       int block_size, int max_context_len, int sliding_window, int num_splits) {
    if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || max_context_len < 0 ||
        sliding_window < 0 || num_splits < 0)
        return FP8KV_ERR_SHAPE;
    if (num_q_heads % num_kv_heads != 0) return FP8KV_ERR_SHAPE;
    if (!head_dim_ok(head_dim) || block_size != kBlockSize) return FP8KV_ERR_UNSUPPORTED;
    if (num_q_heads / num_kv_heads > kMaxGroup) return FP8KV_ERR_UNSUPPORTED;
    if (num_splits > kMaxSplits) return FP8KV_ERR_UNSUPPORTED;
    return FP8KV_OK;
}

// Longest block span any sequence can need: full context, or a window of W positions
// that may straddle one extra block boundary.
int max_window_blocks(int max_context_len, int sliding_window) {
    if (max_context_len <= 0) return 0;
    int nb = (max_context_len + kBlockSize - 1) / kBlockSize;
    if (sliding_window > 0) {
        const int wb = (sliding_window + kBlockSize - 1) / kBlockSize + 1;
        if (wb < nb) nb = wb;
    }
    return nb;
}

struct Plan {
    int splits;
    int blocks_per_split;
};

Plan make_plan(int num_seqs, int num_kv_heads, int head_dim, int max_context_len,
               int sliding_window, int num_splits) {
    Plan pl;
    const int nb = max_window_blocks(max_context_len, sliding_window);
    if (nb == 0) {
        pl.splits = 1;
        pl.blocks_per_split = kMinBlocksPerSplit;
        return pl;
    }
    int bps;
    if (num_splits > 0) {
        const int s = num_splits < nb ? num_splits : nb;
        bps = (nb + s - 1) / s;
    } else {
        const long long units = (long long)(num_seqs > 0 ? num_seqs : 1) * num_kv_heads;
        long long s = (target_workgroups(head_dim) + units - 1) / units;
        if (s < 1 || nb <= kSingleSplitBlocks) s = 1;
        if (s > nb) s = nb;
        bps = (int)((nb + s - 1) / s);
        bps = (bps + kMinBlocksPerSplit - 1) / kMinBlocksPerSplit * kMinBlocksPerSplit;
    }
    if ((nb + bps - 1) / bps > kMaxSplits) bps = (nb + kMaxSplits - 1) / kMaxSplits;
    pl.blocks_per_split = bps;
    pl.splits = (nb + bps - 1) / bps;
    return pl;
}

struct WorkspaceLayout {
    size_t ml_bytes, acc_offset, total;
};

WorkspaceLayout workspace_layout(int num_seqs, int num_q_heads, int head_dim, int splits) {
    WorkspaceLayout l;
    const size_t rows = (size_t)num_seqs * num_q_heads * splits;
    l.ml_bytes = rows * 2 * sizeof(float);
    l.acc_offset = (l.ml_bytes + 255) / 256 * 256;
    l.total = l.acc_offset + rows * (size_t)head_dim * sizeof(float);
    return l;
}

// The counter buffer holds one record per (sequence, kv head) group, group b*Hkv + h at
// byte (b*Hkv + h) * kCounterRecordBytes: the split arrival counter and one step-claim
// counter per decode wave, each in a 256-byte line of its own.
constexpr size_t kCounterRecordBytes = fp8kv::kCounterRecordWords * sizeof(unsigned int);
static_assert(kCounterRecordBytes == 1280, "the public header documents 1280-byte counter records");

size_t counter_bytes(int num_seqs, int num_kv_heads) {
    return (size_t)num_seqs * num_kv_heads * kCounterRecordBytes;
}

thread_local hipError_t g_last_hip_error = hipSuccess;
// device error word of the calling thread's launches (fp8kv_set_error_word), or null
thread_local unsigned int* g_error_word = nullptr;

int hip_status(hipError_t e) {
    if (e == hipSuccess) return FP8KV_OK;
    g_last_hip_error = e;
    return FP8KV_ERR_HIP;
}

}  // namespace

void fp8kv::record_hip_error(hipError_t e) { g_last_hip_error = e; }

namespace {

// Shared validation and parameter setup of the decode entry points.
int setup_decode(fp8kv::DecodeParams& p, bool& fp8, const void* query, const void* key_cache,
                 const void* value_cache, int cache_dtype, const int32_t* block_tables,
                 int max_blocks_per_seq, const int32_t* context_lens, int max_context_len,
                 int num_seqs, int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                 int num_blocks, const Scales& sc, bool per_head_call, int sliding_window,
                 int num_splits, void* workspace, size_t workspace_bytes,
                 bool need_workspace_for_single) {
    int st = check_decode_shape(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                                max_context_len, sliding_window, num_splits);
    if (st != FP8KV_OK) return st;
    if (max_blocks_per_seq < 0 || num_blocks < 0) return FP8KV_ERR_SHAPE;
    if (!cache_dtype_ok(cache_dtype)) return FP8KV_ERR_UNSUPPORTED;
    fp8 = cache_dtype != FP8KV_BF16;   // one-byte codes (E4M3, E5M2, INT8)
    if (fp8) {
        st = check_scales(sc, per_head_call);
        if (st != FP8KV_OK) return st;
    }
    if (num_seqs > 0) {
        if (!query || !context_lens || !block_tables || !key_cache || !value_cache)
            return FP8KV_ERR_NULL;
        if (!aligned16(query) || !aligned16(key_cache) || !aligned16(value_cache))
            return FP8KV_ERR_SHAPE;
        if ((max_blocks_per_seq == 0 || num_blocks == 0) && max_context_len > 0) return FP8KV_ERR_SHAPE;
    }
    const Plan pl = make_plan(num_seqs, num_kv_heads, head_dim, max_context_len, sliding_window, num_splits);
    const WorkspaceLayout wl = workspace_layout(num_seqs, num_q_heads, head_dim, pl.splits);
    const bool single = pl.splits == 1 && !need_workspace_for_single;
    if (!single && num_seqs > 0) {
        if (!workspace || workspace_bytes < wl.total) return FP8KV_ERR_WORKSPACE;
        if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return FP8KV_ERR_WORKSPACE;
    }
    p.query = static_cast<const uint16_t*>(query);
    p.query_lo = nullptr;
    p.key_cache = key_cache;
    p.value_cache = value_cache;
    p.block_tables = block_tables;
    p.context_lens = context_lens;
    p.max_blocks_per_seq = max_blocks_per_seq;
    p.max_context_len = max_context_len;
    p.num_seqs = num_seqs;
    p.num_q_heads = num_q_heads;
    p.num_kv_heads = num_kv_heads;
    p.num_blocks = num_blocks;
    p.sliding_window = sliding_window;
    // per-head key scales are applied in the kernel, to log2(e)/sqrt(D) rounded to float
    const double log2e = 1.4426950408889634;
    const bool heads = fp8 && per_head_call;
    p.score_scale = (float)((fp8 && !heads ? (double)sc.k : 1.0) * log2e / sqrt((double)head_dim));
    p.v_scale = fp8 && !heads ? sc.v : 1.0f;
    p.k_scales = heads ? sc.ks : nullptr;
    p.v_scales = heads ? sc.vs : nullptr;
    p.splits = pl.splits;
    p.blocks_per_split = pl.blocks_per_split;
    p.ws_ml = single ? nullptr : reinterpret_cast<float*>(workspace);
    p.ws_acc = single ? nullptr
                      : reinterpret_cast<float*>(static_cast<char*>(workspace) + wl.acc_offset);
    p.write_final = single ? 1 : 0;
    p.out = nullptr;
    p.out_f32 = 0;
    p.k_new = nullptr;
    p.v_new = nullptr;
    p.k_scale_q = 1.0f;
    p.v_scale_q = 1.0f;
    p.counters = nullptr;
    p.use_claims = 0;
    p.merge_in_kernel = 0;
    p.err = g_error_word;
    p.rot_scale = 1.0f;
    return FP8KV_OK;
}

// Attach the caller's counter buffer to a decode with several splits: the last workgroup of
// each (sequence, kv head) merges the partials inside the decode kernel when one workgroup
// merges a group cheaply (else the merge kernel still runs), and with the automatic split
// plan the last steps of each group are claimed at run time.  Returns whether the merge is
// fused, or a negative status for a buffer that is too small or misaligned.
int attach_counters(fp8kv::DecodeParams& p, int head_dim, void* counters, size_t counters_bytes,
                    int num_splits) {
    if (p.write_final || p.num_seqs == 0) return 0;
    if (!counters || counters_bytes < counter_bytes(p.num_seqs, p.num_kv_heads))
        return FP8KV_ERR_WORKSPACE;
    if ((reinterpret_cast<uintptr_t>(counters) & 255u) != 0) return FP8KV_ERR_WORKSPACE;
    const bool fused = fp8kv::fused_merge_fits(p.num_q_heads / p.num_kv_heads, head_dim, p.splits);
    p.counters = static_cast<unsigned int*>(counters);
    p.use_claims = num_splits == 0 ? 1 : 0;
    p.merge_in_kernel = fused ? 1 : 0;
    return fused ? 1 : 0;
}

int cache_write_impl(const void* key, const void* value, void* key_cache, void* value_cache,
                     int cache_dtype, const int64_t* slot_mapping, int num_tokens,
                     int num_kv_heads, int head_dim, int block_size, int num_blocks,
                     const Scales& sc, bool per_head_call, void* stream) {
    if (num_tokens < 0 || num_kv_heads <= 0 || num_blocks < 0) return FP8KV_ERR_SHAPE;
    if (!head_dim_ok(head_dim) || block_size != kBlockSize) return FP8KV_ERR_UNSUPPORTED;
    if (!cache_dtype_ok(cache_dtype)) return FP8KV_ERR_UNSUPPORTED;
    const bool fp8 = cache_dtype != FP8KV_BF16;   // one-byte codes (E4M3, E5M2, INT8)
    if (fp8) {
        const int st = check_scales(sc, per_head_call);
        if (st != FP8KV_OK) return st;
    }
    if (num_tokens == 0) return FP8KV_OK;
    if (!key || !value || !key_cache || !value_cache || !slot_mapping) return FP8KV_ERR_NULL;
    if (!aligned16(key) || !aligned16(value) || !aligned16(key_cache) || !aligned16(value_cache))
        return FP8KV_ERR_SHAPE;
    fp8kv::CacheWriteParams p;
    p.key = static_cast<const uint16_t*>(key);
    p.value = static_cast<const uint16_t*>(value);
    p.key_cache = key_cache;
    p.value_cache = value_cache;
    p.slot_mapping = slot_mapping;
    p.num_tokens = num_tokens;
    p.num_kv_heads = num_kv_heads;
    p.num_blocks = num_blocks;
    p.k_scale = sc.k;
    p.v_scale = sc.v;
    p.k_scales = fp8 && per_head_call ? sc.ks : nullptr;
    p.v_scales = fp8 && per_head_call ? sc.vs : nullptr;
    p.err = g_error_word;
    return hip_status(fp8kv::launch_cache_write(p, codec_of(cache_dtype), head_dim, static_cast<hipStream_t>(stream)));
}

int paged_decode_impl(void* out, int out_dtype, const void* query, const void* key_cache,
                      const void* value_cache, int cache_dtype, const int32_t* block_tables,
                      int max_blocks_per_seq, const int32_t* context_lens, int max_context_len,
                      int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                      int block_size, int num_blocks, const Scales& sc, bool per_head_call,
                      int sliding_window, int num_splits, void* counters, size_t counters_bytes,
                      void* workspace, size_t workspace_bytes, void* stream) {
    if (out_dtype != FP8KV_BF16 && out_dtype != FP8KV_F32) return FP8KV_ERR_UNSUPPORTED;
    fp8kv::DecodeParams p;
    bool fp8 = true;
    int st = setup_decode(p, fp8, query, key_cache, value_cache, cache_dtype, block_tables,
                          max_blocks_per_seq, context_lens, max_context_len, num_seqs,
                          num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, sc,
                          per_head_call, sliding_window, num_splits, workspace, workspace_bytes,
                          false);
    if (st != FP8KV_OK) return st;
    if (num_seqs == 0) return FP8KV_OK;
    if (!out) return FP8KV_ERR_NULL;
    if (!aligned16(out)) return FP8KV_ERR_SHAPE;
    // optional counters: the in-kernel merge
    const int fused = counters != nullptr
                          ? attach_counters(p, head_dim, counters, counters_bytes, num_splits) : 0;
    if (fused < 0) return fused;
    p.out = out;
    p.out_f32 = out_dtype == FP8KV_F32;
    hipStream_t s = static_cast<hipStream_t>(stream);
    st = hip_status(fp8kv::launch_decode_partial(p, codec_of(cache_dtype), head_dim, s));
    if (st != FP8KV_OK || p.write_final || fused) return st;
    return hip_status(fp8kv::launch_decode_merge(p, head_dim, s));
}

int decode_step_impl(void* out, int out_dtype, const void* query, const void* key_new,
                     const void* value_new, void* key_cache, void* value_cache, int cache_dtype,
                     const int32_t* block_tables, int max_blocks_per_seq,
                     const int32_t* context_lens, int max_context_len, int num_seqs,
                     int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                     int num_blocks, const Scales& sc, bool per_head_call, int sliding_window,
                     int num_splits, void* counters, size_t counters_bytes, void* workspace,
                     size_t workspace_bytes, void* stream, bool launch = true) {
    if (out_dtype != FP8KV_BF16 && out_dtype != FP8KV_F32) return FP8KV_ERR_UNSUPPORTED;
    fp8kv::DecodeParams p;
    bool fp8 = true;
    int st = setup_decode(p, fp8, query, key_cache, value_cache, cache_dtype, block_tables,
                          max_blocks_per_seq, context_lens, max_context_len, num_seqs,
                          num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, sc,
                          per_head_call, sliding_window, num_splits, workspace, workspace_bytes,
                          false);
    if (st != FP8KV_OK) return st;
    if (num_seqs == 0) return FP8KV_OK;
    if (!out || !key_new || !value_new) return FP8KV_ERR_NULL;
    if (!aligned16(out) || !aligned16(key_new) || !aligned16(value_new)) return FP8KV_ERR_SHAPE;
    // several splits: the counters are required (arrival, and claims with the automatic plan)
    const int fused = attach_counters(p, head_dim, counters, counters_bytes, num_splits);
    if (fused < 0) return fused;
    if (!launch) return FP8KV_OK;   // validation only
    p.out = out;
    p.out_f32 = out_dtype == FP8KV_F32;
    p.k_new = static_cast<const uint16_t*>(key_new);
    p.v_new = static_cast<const uint16_t*>(value_new);
    p.k_scale_q = fp8 && !per_head_call ? sc.k : 1.0f;
    p.v_scale_q = fp8 && !per_head_call ? sc.v : 1.0f;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    st = hip_status(fp8kv::launch_decode_partial(p, codec_of(cache_dtype), head_dim, s));
    if (st != FP8KV_OK || p.write_final || fused) return st;
    return hip_status(fp8kv::launch_decode_merge(p, head_dim, s));
}

// Workspace of the rotated prefill: the rotated query's two bf16 terms and the f32 output
// before it is rotated back, each 256-byte aligned.
struct PrefillRotLayout {
    size_t q_hi, q_lo, out, total;
};

PrefillRotLayout prefill_rot_layout(int64_t rows, int head_dim) {
    const auto up = [](size_t x) { return (x + 255) / 256 * 256; };
    PrefillRotLayout l;
    const size_t n = (size_t)rows * head_dim;
    l.q_hi = 0;
    l.q_lo = up(n * 2);
    l.out = l.q_lo + up(n * 2);
    l.total = l.out + up(n * 4);
    return l;
}

// The rotated prefill's extra arguments: the caller's row count and workspace.
struct PrefillRot {
    int num_query_tokens;
    void* workspace;
    size_t workspace_bytes;
};

int paged_prefill_impl(void* out, int out_dtype, const void* query,
                       const int32_t* query_start_loc, const void* key_cache,
                       const void* value_cache, int cache_dtype, const int32_t* block_tables,
                       int max_blocks_per_seq, const int32_t* context_lens, int max_context_len,
                       int num_seqs, int max_query_len, int num_q_heads, int num_kv_heads,
                       int head_dim, int block_size, int num_blocks, const Scales& sc,
                       bool per_head_call, int sliding_window, void* stream,
                       const PrefillRot* rot = nullptr) {
    if (out_dtype != FP8KV_BF16 && out_dtype != FP8KV_F32) return FP8KV_ERR_UNSUPPORTED;
    if (rot != nullptr) {
        // the rotated path is defined for the E4M3 and BF16 caches; its low query term lives
        // in the two-tile kernel's LDS, which head_dim 256 does not use
        if (cache_dtype != FP8KV_E4M3 && cache_dtype != FP8KV_BF16) return FP8KV_ERR_UNSUPPORTED;
        if (head_dim == 256) return FP8KV_ERR_UNSUPPORTED;
        if (rot->num_query_tokens < 0) return FP8KV_ERR_SHAPE;
    }
    int st = check_decode_shape(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                                max_context_len, sliding_window, 0);
    if (st != FP8KV_OK) return st;
    if (max_query_len < 0 || max_blocks_per_seq < 0 || num_blocks < 0) return FP8KV_ERR_SHAPE;
    if (!cache_dtype_ok(cache_dtype)) return FP8KV_ERR_UNSUPPORTED;
    const bool fp8 = cache_dtype != FP8KV_BF16;   // one-byte codes (E4M3, E5M2, INT8)
    if (fp8) {
        st = check_scales(sc, per_head_call);
        if (st != FP8KV_OK) return st;
    }
    if (num_seqs > 65535 || num_kv_heads > 65535) return FP8KV_ERR_UNSUPPORTED;   // grid extents
    if (num_seqs == 0 || max_query_len == 0) return FP8KV_OK;
    if (!out || !query || !query_start_loc || !context_lens || !block_tables || !key_cache ||
        !value_cache)
        return FP8KV_ERR_NULL;
    if (!aligned16(out) || !aligned16(query) || !aligned16(key_cache) || !aligned16(value_cache))
        return FP8KV_ERR_SHAPE;
    if ((max_blocks_per_seq == 0 || num_blocks == 0) && max_context_len > 0) return FP8KV_ERR_SHAPE;
    fp8kv::PrefillParams p;
    p.out = out;
    p.out_f32 = out_dtype == FP8KV_F32;
    p.query = static_cast<const uint16_t*>(query);
    p.query_start_loc = query_start_loc;
    p.key_cache = key_cache;
    p.value_cache = value_cache;
    p.block_tables = block_tables;
    p.context_lens = context_lens;
    p.max_blocks_per_seq = max_blocks_per_seq;
    p.max_context_len = max_context_len;
    p.max_query_len = max_query_len;
    p.num_seqs = num_seqs;
    p.num_q_heads = num_q_heads;
    p.num_kv_heads = num_kv_heads;
    p.num_blocks = num_blocks;
    p.sliding_window = sliding_window;
    const double log2e = 1.4426950408889634;
    const bool heads = fp8 && per_head_call;
    p.score_scale = (float)((fp8 && !heads ? (double)sc.k : 1.0) * log2e / sqrt((double)head_dim));
    p.v_scale = fp8 && !heads ? sc.v : 1.0f;
    p.k_scales = heads ? sc.ks : nullptr;
    p.v_scales = heads ? sc.vs : nullptr;
    p.err = g_error_word;
    p.query_lo = nullptr;
    p.num_rows = INT_MAX;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    if (rot == nullptr) return hip_status(fp8kv::launch_prefill(p, codec_of(cache_dtype), head_dim, s));
    // rotated: query rotation into two bf16 terms, the prefill in the rotated space into f32
    // rows, then the rotation back into `out`
    if (rot->num_query_tokens == 0) return FP8KV_OK;
    const int64_t rows = (int64_t)rot->num_query_tokens * num_q_heads;
    const PrefillRotLayout rl = prefill_rot_layout(rows, head_dim);
    if (!rot->workspace || rot->workspace_bytes < rl.total) return FP8KV_ERR_WORKSPACE;
    if ((reinterpret_cast<uintptr_t>(rot->workspace) & 255u) != 0) return FP8KV_ERR_WORKSPACE;
    char* ws = static_cast<char*>(rot->workspace);
    uint16_t* q_hi = reinterpret_cast<uint16_t*>(ws + rl.q_hi);
    uint16_t* q_lo = reinterpret_cast<uint16_t*>(ws + rl.q_lo);
    float* out_rot = reinterpret_cast<float*>(ws + rl.out);
    int st2 = hip_status(fp8kv::launch_rotate_query(static_cast<const uint16_t*>(query), q_hi, q_lo,
                                                    rows, head_dim, s));
    if (st2 != FP8KV_OK) return st2;
    p.query = q_hi;
    p.query_lo = q_lo;
    p.num_rows = rot->num_query_tokens;
    p.out = out_rot;
    p.out_f32 = 1;
    st2 = hip_status(fp8kv::launch_prefill(p, codec_of(cache_dtype), head_dim, s));
    if (st2 != FP8KV_OK) return st2;
    return hip_status(fp8kv::launch_rotate_out(out_rot, out, out_dtype == FP8KV_F32, rows, head_dim, s));
}

int partial_impl(const void* query, const void* key_cache, const void* value_cache,
                 int cache_dtype, const int32_t* block_tables, int max_blocks_per_seq,
                 const int32_t* context_lens, int max_context_len, int num_seqs, int num_q_heads,
                 int num_kv_heads, int head_dim, int block_size, int num_blocks, const Scales& sc,
                 bool per_head_call, int sliding_window, int num_splits, void* workspace,
                 size_t workspace_bytes, void* stream) {
    fp8kv::DecodeParams p;
    bool fp8 = true;
    // the per-head call's key array stands in for both arrays in the shared checks
    int st = setup_decode(p, fp8, query, key_cache, value_cache, cache_dtype, block_tables,
                          max_blocks_per_seq, context_lens, max_context_len, num_seqs,
                          num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, sc,
                          per_head_call, sliding_window, num_splits, workspace, workspace_bytes,
                          true);
    if (st != FP8KV_OK || num_seqs == 0) return st;
    p.v_scales = nullptr;   // the merge applies the value scales
    return hip_status(fp8kv::launch_decode_partial(p, codec_of(cache_dtype), head_dim, static_cast<hipStream_t>(stream)));
}

int merge_impl(void* out, int out_dtype, const int32_t* context_lens, int max_context_len,
               int max_blocks_per_seq, int num_seqs, int num_q_heads, int num_kv_heads,
               int head_dim, int block_size, float v_scale, const float* v_scales,
               int sliding_window, int num_splits, const void* workspace, size_t workspace_bytes,
               void* stream) {
    if (out_dtype != FP8KV_BF16 && out_dtype != FP8KV_F32) return FP8KV_ERR_UNSUPPORTED;
    int st = check_decode_shape(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                                max_context_len, sliding_window, num_splits);
    if (st != FP8KV_OK) return st;
    if (max_blocks_per_seq < 0) return FP8KV_ERR_SHAPE;
    if (num_seqs == 0) return FP8KV_OK;
    if (!out || !context_lens) return FP8KV_ERR_NULL;
    if (!aligned16(out)) return FP8KV_ERR_SHAPE;
    const Plan pl = make_plan(num_seqs, num_kv_heads, head_dim, max_context_len, sliding_window, num_splits);
    const WorkspaceLayout wl = workspace_layout(num_seqs, num_q_heads, head_dim, pl.splits);
    if (!workspace || workspace_bytes < wl.total) return FP8KV_ERR_WORKSPACE;
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return FP8KV_ERR_WORKSPACE;
    fp8kv::DecodeParams p = {};
    p.out = out;
    p.out_f32 = out_dtype == FP8KV_F32;
    p.context_lens = context_lens;
    p.max_blocks_per_seq = max_blocks_per_seq;
    p.max_context_len = max_context_len;
    p.num_seqs = num_seqs;
    p.num_q_heads = num_q_heads;
    p.num_kv_heads = num_kv_heads;
    p.sliding_window = sliding_window;
    p.v_scale = v_scale;
    p.v_scales = v_scales;
    p.splits = pl.splits;
    p.blocks_per_split = pl.blocks_per_split;
    p.ws_ml = reinterpret_cast<float*>(const_cast<void*>(workspace));
    p.ws_acc = reinterpret_cast<float*>(static_cast<char*>(const_cast<void*>(workspace)) + wl.acc_offset);
    return hip_status(fp8kv::launch_decode_merge(p, head_dim, static_cast<hipStream_t>(stream)));
}

// The rotated decode's workspace: the decode's own (split partials), then the rotated
// query as two bf16 terms, then the f32 output before it is rotated back; each 256-aligned.
struct RotatedLayout {
    size_t q_hi, q_lo, out, total;
};

RotatedLayout rotated_layout(size_t decode_bytes, int num_seqs, int num_q_heads, int head_dim) {
    auto up = [](size_t x) { return (x + 255) / 256 * 256; };
    const size_t rows = (size_t)num_seqs * num_q_heads * head_dim;
    RotatedLayout l;
    l.q_hi = up(decode_bytes);
    l.q_lo = l.q_hi + up(rows * 2);
    l.out = l.q_lo + up(rows * 2);
    l.total = l.out + up(rows * 4);
    return l;
}

}  // namespace

int fp8kv::decode_step_check(void* out, int out_dtype, const void* query, const void* key_new,
                             const void* value_new, void* key_cache, void* value_cache,
                             int cache_dtype, const int32_t* block_tables, int max_blocks_per_seq,
                             const int32_t* context_lens, int max_context_len, int num_seqs,
                             int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                             int num_blocks, float k_scale, float v_scale, int sliding_window,
                             int num_splits, size_t counters_bytes, size_t workspace_bytes) {
    // placeholder buffers of the given sizes (256-byte aligned, never dereferenced here)
    void* const buf = reinterpret_cast<void*>(static_cast<uintptr_t>(256));
    return decode_step_impl(out, out_dtype, query, key_new, value_new, key_cache, value_cache,
                            cache_dtype, block_tables, max_blocks_per_seq, context_lens,
                            max_context_len, num_seqs, num_q_heads, num_kv_heads, head_dim,
                            block_size, num_blocks, tensor_scales(k_scale, v_scale), false,
                            sliding_window, num_splits, buf, counters_bytes, buf, workspace_bytes,
                            nullptr, false);
}

extern "C" {

const char* fp8kv_status_string(int status) {
    switch (status) {
        case FP8KV_OK: return "ok";
        case FP8KV_ERR_NULL: return "a required pointer is NULL";
        case FP8KV_ERR_SHAPE: return "a size is negative or inconsistent, or a buffer is misaligned";
        case FP8KV_ERR_UNSUPPORTED: return "unsupported head_dim, block_size, group ratio, split count or dtype";
        case FP8KV_ERR_SCALE: return "a scale of a one-byte cache is not finite and positive";
        case FP8KV_ERR_WORKSPACE: return "workspace is NULL, too small, or not 256-byte aligned";
        case FP8KV_ERR_HIP: return "a HIP kernel launch failed";
        case FP8KV_ERR_SCRATCH: return "the call needs more than the fixed device array of fp8kv_decode_step_noalloc holds";
        default: return "unknown status";
    }
}

int fp8kv_version(void) { return 200; }

const char* fp8kv_last_hip_error(void) { return hipGetErrorName(g_last_hip_error); }

int fp8kv_set_error_word(unsigned int* word) {
    if (word != nullptr && !aligned4(word)) return FP8KV_ERR_SHAPE;
    g_error_word = word;
    return FP8KV_OK;
}

size_t fp8kv_decode_counters_size(int max_num_seqs, int num_kv_heads) {
    if (max_num_seqs < 0 || num_kv_heads <= 0) return 0;
    return counter_bytes(max_num_seqs, num_kv_heads);
}

int fp8kv_cache_write(const void* key, const void* value, void* key_cache, void* value_cache,
                      int cache_dtype, const int64_t* slot_mapping, int num_tokens,
                      int num_kv_heads, int head_dim, int block_size, int num_blocks,
                      float k_scale, float v_scale, void* stream) {
    return cache_write_impl(key, value, key_cache, value_cache, cache_dtype, slot_mapping,
                            num_tokens, num_kv_heads, head_dim, block_size, num_blocks,
                            tensor_scales(k_scale, v_scale), false, stream);
}

int fp8kv_cache_write_per_head(const void* key, const void* value, void* key_cache,
                               void* value_cache, int cache_dtype, const int64_t* slot_mapping,
                               int num_tokens, int num_kv_heads, int head_dim, int block_size,
                               int num_blocks, const float* k_scales, const float* v_scales,
                               void* stream) {
    return cache_write_impl(key, value, key_cache, value_cache, cache_dtype, slot_mapping,
                            num_tokens, num_kv_heads, head_dim, block_size, num_blocks,
                            head_scales(k_scales, v_scales), true, stream);
}


int fp8kv_paged_decode_num_splits(int num_seqs, int num_kv_heads, int head_dim, int block_size,
                                  int max_context_len, int sliding_window, int num_splits) {
    int st = check_decode_shape(num_seqs, num_kv_heads, num_kv_heads, head_dim, block_size,
                                max_context_len, sliding_window, num_splits);
    if (st != FP8KV_OK) return st;
    return make_plan(num_seqs, num_kv_heads, head_dim, max_context_len, sliding_window, num_splits).splits;
}

size_t fp8kv_paged_decode_workspace_size(int num_seqs, int num_q_heads, int num_kv_heads,
                                         int head_dim, int block_size, int max_context_len,
                                         int sliding_window, int num_splits) {
    if (check_decode_shape(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                           max_context_len, sliding_window, num_splits) != FP8KV_OK)
        return 0;
    const Plan pl = make_plan(num_seqs, num_kv_heads, head_dim, max_context_len, sliding_window, num_splits);
    return workspace_layout(num_seqs, num_q_heads, head_dim, pl.splits).total;
}

int fp8kv_paged_decode(void* out, int out_dtype, const void* query, const void* key_cache,
                       const void* value_cache, int cache_dtype, const int32_t* block_tables,
                       int max_blocks_per_seq, const int32_t* context_lens, int max_context_len,
                       int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                       int block_size, int num_blocks, float k_scale, float v_scale,
                       int sliding_window, int num_splits, void* counters, size_t counters_bytes,
                       void* workspace, size_t workspace_bytes, void* stream) {
    return paged_decode_impl(out, out_dtype, query, key_cache, value_cache, cache_dtype,
                             block_tables, max_blocks_per_seq, context_lens, max_context_len,
                             num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                             num_blocks, tensor_scales(k_scale, v_scale), false, sliding_window,
                             num_splits, counters, counters_bytes, workspace, workspace_bytes,
                             stream);
}

int fp8kv_paged_decode_per_head(void* out, int out_dtype, const void* query,
                                const void* key_cache, const void* value_cache, int cache_dtype,
                                const int32_t* block_tables, int max_blocks_per_seq,
                                const int32_t* context_lens, int max_context_len, int num_seqs,
                                int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                                int num_blocks, const float* k_scales, const float* v_scales,
                                int sliding_window, int num_splits, void* counters,
                                size_t counters_bytes, void* workspace, size_t workspace_bytes,
                                void* stream) {
    return paged_decode_impl(out, out_dtype, query, key_cache, value_cache, cache_dtype,
                             block_tables, max_blocks_per_seq, context_lens, max_context_len,
                             num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                             num_blocks, head_scales(k_scales, v_scales), true, sliding_window,
                             num_splits, counters, counters_bytes, workspace, workspace_bytes,
                             stream);
}


int fp8kv_decode_step(void* out, int out_dtype, const void* query, const void* key_new,
                      const void* value_new, void* key_cache, void* value_cache, int cache_dtype,
                      const int32_t* block_tables, int max_blocks_per_seq,
                      const int32_t* context_lens, int max_context_len, int num_seqs,
                      int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                      int num_blocks, float k_scale, float v_scale, int sliding_window,
                      int num_splits, void* counters, size_t counters_bytes, void* workspace,
                      size_t workspace_bytes, void* stream) {
    return decode_step_impl(out, out_dtype, query, key_new, value_new, key_cache, value_cache,
                            cache_dtype, block_tables, max_blocks_per_seq, context_lens,
                            max_context_len, num_seqs, num_q_heads, num_kv_heads, head_dim,
                            block_size, num_blocks, tensor_scales(k_scale, v_scale), false,
                            sliding_window, num_splits, counters, counters_bytes, workspace,
                            workspace_bytes, stream);
}

int fp8kv_decode_step_per_head(void* out, int out_dtype, const void* query, const void* key_new,
                               const void* value_new, void* key_cache, void* value_cache,
                               int cache_dtype, const int32_t* block_tables,
                               int max_blocks_per_seq, const int32_t* context_lens,
                               int max_context_len, int num_seqs, int num_q_heads,
                               int num_kv_heads, int head_dim, int block_size, int num_blocks,
                               const float* k_scales, const float* v_scales, int sliding_window,
                               int num_splits, void* counters, size_t counters_bytes,
                               void* workspace, size_t workspace_bytes, void* stream) {
    return decode_step_impl(out, out_dtype, query, key_new, value_new, key_cache, value_cache,
                            cache_dtype, block_tables, max_blocks_per_seq, context_lens,
                            max_context_len, num_seqs, num_q_heads, num_kv_heads, head_dim,
                            block_size, num_blocks, head_scales(k_scales, v_scales), true,
                            sliding_window, num_splits, counters, counters_bytes, workspace,
                            workspace_bytes, stream);
}


int fp8kv_paged_decode_partial(const void* query, const void* key_cache, const void* value_cache,
                               int cache_dtype, const int32_t* block_tables,
                               int max_blocks_per_seq, const int32_t* context_lens,
                               int max_context_len, int num_seqs, int num_q_heads,
                               int num_kv_heads, int head_dim, int block_size, int num_blocks,
                               float k_scale, int sliding_window, int num_splits, void* workspace,
                               size_t workspace_bytes, void* stream) {
    return partial_impl(query, key_cache, value_cache, cache_dtype, block_tables,
                        max_blocks_per_seq, context_lens, max_context_len, num_seqs, num_q_heads,
                        num_kv_heads, head_dim, block_size, num_blocks, tensor_scales(k_scale, 1.0f),
                        false, sliding_window, num_splits, workspace, workspace_bytes, stream);
}

int fp8kv_paged_decode_partial_per_head(const void* query, const void* key_cache,
                                        const void* value_cache, int cache_dtype,
                                        const int32_t* block_tables, int max_blocks_per_seq,
                                        const int32_t* context_lens, int max_context_len,
                                        int num_seqs, int num_q_heads, int num_kv_heads,
                                        int head_dim, int block_size, int num_blocks,
                                        const float* k_scales, int sliding_window, int num_splits,
                                        void* workspace, size_t workspace_bytes, void* stream) {
    // the value scales belong to the merge: only the key array is checked here
    if (cache_dtype != FP8KV_BF16) {
        if (!k_scales) return FP8KV_ERR_NULL;
        if (!aligned4(k_scales)) return FP8KV_ERR_SHAPE;
    }
    return partial_impl(query, key_cache, value_cache, cache_dtype, block_tables,
                        max_blocks_per_seq, context_lens, max_context_len, num_seqs, num_q_heads,
                        num_kv_heads, head_dim, block_size, num_blocks, head_scales(k_scales, k_scales),
                        true, sliding_window, num_splits, workspace, workspace_bytes, stream);
}

int fp8kv_paged_decode_merge(void* out, int out_dtype, const int32_t* context_lens,
                             int max_context_len, int max_blocks_per_seq, int num_seqs,
                             int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                             float v_scale, int sliding_window, int num_splits,
                             const void* workspace, size_t workspace_bytes, void* stream) {
    if (!scale_ok(v_scale)) return FP8KV_ERR_SCALE;
    return merge_impl(out, out_dtype, context_lens, max_context_len, max_blocks_per_seq, num_seqs,
                      num_q_heads, num_kv_heads, head_dim, block_size, v_scale, nullptr,
                      sliding_window, num_splits, workspace, workspace_bytes, stream);
}

int fp8kv_paged_decode_merge_per_head(void* out, int out_dtype, int cache_dtype,
                                      const int32_t* context_lens, int max_context_len,
                                      int max_blocks_per_seq, int num_seqs, int num_q_heads,
                                      int num_kv_heads, int head_dim, int block_size,
                                      const float* v_scales, int sliding_window, int num_splits,
                                      const void* workspace, size_t workspace_bytes,
                                      void* stream) {
    if (!cache_dtype_ok(cache_dtype)) return FP8KV_ERR_UNSUPPORTED;
    const bool fp8 = cache_dtype != FP8KV_BF16;
    if (fp8) {
        if (!v_scales) return FP8KV_ERR_NULL;
        if (!aligned4(v_scales)) return FP8KV_ERR_SHAPE;
    }
    return merge_impl(out, out_dtype, context_lens, max_context_len, max_blocks_per_seq, num_seqs,
                      num_q_heads, num_kv_heads, head_dim, block_size, 1.0f,
                      fp8 ? v_scales : nullptr, sliding_window, num_splits, workspace,
                      workspace_bytes, stream);
}

int fp8kv_paged_prefill(void* out, int out_dtype, const void* query,
                        const int32_t* query_start_loc, const void* key_cache,
                        const void* value_cache, int cache_dtype, const int32_t* block_tables,
                        int max_blocks_per_seq, const int32_t* context_lens, int max_context_len,
                        int num_seqs, int max_query_len, int num_q_heads, int num_kv_heads,
                        int head_dim, int block_size, int num_blocks, float k_scale,
                        float v_scale, int sliding_window, void* stream) {
    return paged_prefill_impl(out, out_dtype, query, query_start_loc, key_cache, value_cache,
                              cache_dtype, block_tables, max_blocks_per_seq, context_lens,
                              max_context_len, num_seqs, max_query_len, num_q_heads, num_kv_heads,
                              head_dim, block_size, num_blocks, tensor_scales(k_scale, v_scale),
                              false, sliding_window, stream);
}

int fp8kv_paged_prefill_per_head(void* out, int out_dtype, const void* query,
                                 const int32_t* query_start_loc, const void* key_cache,
                                 const void* value_cache, int cache_dtype,
                                 const int32_t* block_tables, int max_blocks_per_seq,
                                 const int32_t* context_lens, int max_context_len, int num_seqs,
                                 int max_query_len, int num_q_heads, int num_kv_heads,
                                 int head_dim, int block_size, int num_blocks,
                                 const float* k_scales, const float* v_scales,
                                 int sliding_window, void* stream) {
    return paged_prefill_impl(out, out_dtype, query, query_start_loc, key_cache, value_cache,
                              cache_dtype, block_tables, max_blocks_per_seq, context_lens,
                              max_context_len, num_seqs, max_query_len, num_q_heads, num_kv_heads,
                              head_dim, block_size, num_blocks, head_scales(k_scales, v_scales),
                              true, sliding_window, stream);
}

size_t fp8kv_paged_prefill_rotated_workspace_size(int num_query_tokens, int num_q_heads,
                                                  int head_dim) {
    if (num_query_tokens < 0 || num_q_heads <= 0 || !head_dim_ok(head_dim)) return 0;
    return prefill_rot_layout((int64_t)num_query_tokens * num_q_heads, head_dim).total;
}

int fp8kv_paged_prefill_rotated(void* out, int out_dtype, const void* query,
                                const int32_t* query_start_loc, const void* key_cache,
                                const void* value_cache, int cache_dtype,
                                const int32_t* block_tables, int max_blocks_per_seq,
                                const int32_t* context_lens, int max_context_len, int num_seqs,
                                int max_query_len, int num_query_tokens, int num_q_heads,
                                int num_kv_heads, int head_dim, int block_size, int num_blocks,
                                float k_scale, float v_scale, int sliding_window,
                                void* workspace, size_t workspace_bytes, void* stream) {
    const PrefillRot rot{num_query_tokens, workspace, workspace_bytes};
    return paged_prefill_impl(out, out_dtype, query, query_start_loc, key_cache, value_cache,
                              cache_dtype, block_tables, max_blocks_per_seq, context_lens,
                              max_context_len, num_seqs, max_query_len, num_q_heads, num_kv_heads,
                              head_dim, block_size, num_blocks, tensor_scales(k_scale, v_scale),
                              false, sliding_window, stream, &rot);
}

}  // extern "C"

namespace {

int rotated_write_impl(const void* key, const void* value, void* key_cache, void* value_cache,
                       int cache_dtype, const int64_t* slot_mapping, int num_tokens,
                       int num_kv_heads, int head_dim, int block_size, int num_blocks,
                       const Scales& sc, bool per_head_call, void* stream) {
    if (num_tokens < 0 || num_kv_heads <= 0 || num_blocks < 0) return FP8KV_ERR_SHAPE;
    if (!head_dim_ok(head_dim) || block_size != kBlockSize) return FP8KV_ERR_UNSUPPORTED;
    if (cache_dtype != FP8KV_E4M3 && cache_dtype != FP8KV_BF16) return FP8KV_ERR_UNSUPPORTED;
    const bool fp8 = cache_dtype != FP8KV_BF16;   // one-byte codes (E4M3)
    if (fp8) {
        const int st = check_scales(sc, per_head_call);
        if (st != FP8KV_OK) return st;
    }
    if (num_tokens == 0) return FP8KV_OK;
    if (!key || !value || !key_cache || !value_cache || !slot_mapping) return FP8KV_ERR_NULL;
    if (!aligned16(key) || !aligned16(value) || !aligned16(key_cache) || !aligned16(value_cache))
        return FP8KV_ERR_SHAPE;
    fp8kv::CacheWriteParams p = {};
    p.key = static_cast<const uint16_t*>(key);
    p.value = static_cast<const uint16_t*>(value);
    p.key_cache = key_cache;
    p.value_cache = value_cache;
    p.slot_mapping = slot_mapping;
    p.num_tokens = num_tokens;
    p.num_kv_heads = num_kv_heads;
    p.num_blocks = num_blocks;
    const bool heads = fp8 && per_head_call;
    p.k_scale = fp8 && !heads ? sc.k : 1.0f;
    p.v_scale = fp8 && !heads ? sc.v : 1.0f;
    p.k_scales = heads ? sc.ks : nullptr;
    p.v_scales = heads ? sc.vs : nullptr;
    p.err = g_error_word;
    return hip_status(fp8kv::launch_rotate_write(p, codec_of(cache_dtype), head_dim, static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

int fp8kv_cache_write_rotated(const void* key, const void* value, void* key_cache,
                              void* value_cache, int cache_dtype, const int64_t* slot_mapping,
                              int num_tokens, int num_kv_heads, int head_dim, int block_size,
                              int num_blocks, float k_scale, float v_scale, void* stream) {
    return rotated_write_impl(key, value, key_cache, value_cache, cache_dtype, slot_mapping,
                              num_tokens, num_kv_heads, head_dim, block_size, num_blocks,
                              tensor_scales(k_scale, v_scale), false, stream);
}

int fp8kv_cache_write_rotated_per_head(const void* key, const void* value, void* key_cache,
                                       void* value_cache, int cache_dtype,
                                       const int64_t* slot_mapping, int num_tokens,
                                       int num_kv_heads, int head_dim, int block_size,
                                       int num_blocks, const float* k_scales,
                                       const float* v_scales, void* stream) {
    return rotated_write_impl(key, value, key_cache, value_cache, cache_dtype, slot_mapping,
                              num_tokens, num_kv_heads, head_dim, block_size, num_blocks,
                              head_scales(k_scales, v_scales), true, stream);
}

size_t fp8kv_paged_decode_rotated_workspace_size(int num_seqs, int num_q_heads, int num_kv_heads,
                                                 int head_dim, int block_size, int max_context_len,
                                                 int sliding_window, int num_splits) {
    if (check_decode_shape(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                           max_context_len, sliding_window, num_splits) != FP8KV_OK)
        return 0;
    const Plan pl = make_plan(num_seqs, num_kv_heads, head_dim, max_context_len, sliding_window, num_splits);
    const size_t dec = workspace_layout(num_seqs, num_q_heads, head_dim, pl.splits).total;
    return rotated_layout(dec, num_seqs, num_q_heads, head_dim).total;
}

}  // extern "C"

namespace {

int rotated_decode_impl(void* out, int out_dtype, const void* query, const void* key_cache,
                        const void* value_cache, int cache_dtype, const int32_t* block_tables,
                        int max_blocks_per_seq, const int32_t* context_lens, int max_context_len,
                        int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                        int block_size, int num_blocks, const Scales& sc, bool per_head_call,
                        int sliding_window, int num_splits, void* workspace,
                        size_t workspace_bytes, void* stream) {
    if (out_dtype != FP8KV_BF16 && out_dtype != FP8KV_F32) return FP8KV_ERR_UNSUPPORTED;
    // the rotated path is defined for the E4M3 and BF16 caches
    if (cache_dtype != FP8KV_E4M3 && cache_dtype != FP8KV_BF16) return FP8KV_ERR_UNSUPPORTED;
    int st = check_decode_shape(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                                max_context_len, sliding_window, num_splits);
    if (st != FP8KV_OK) return st;
    const Plan pl = make_plan(num_seqs, num_kv_heads, head_dim, max_context_len, sliding_window, num_splits);
    const size_t dec = workspace_layout(num_seqs, num_q_heads, head_dim, pl.splits).total;
    const RotatedLayout rl = rotated_layout(dec, num_seqs, num_q_heads, head_dim);
    fp8kv::DecodeParams p;
    bool fp8 = true;
    // the decode's part of the workspace is checked by setup_decode; the rotation buffers here
    st = setup_decode(p, fp8, query, key_cache, value_cache, cache_dtype, block_tables,
                      max_blocks_per_seq, context_lens, max_context_len, num_seqs, num_q_heads,
                      num_kv_heads, head_dim, block_size, num_blocks, sc, per_head_call,
                      sliding_window, num_splits, workspace,
                      workspace_bytes < dec ? workspace_bytes : dec, false);
    if (st != FP8KV_OK) return st;
    if (num_seqs == 0) return FP8KV_OK;
    if (!workspace || workspace_bytes < rl.total) return FP8KV_ERR_WORKSPACE;
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return FP8KV_ERR_WORKSPACE;
    if (!out) return FP8KV_ERR_NULL;
    if (!aligned16(out)) return FP8KV_ERR_SHAPE;
    char* ws = static_cast<char*>(workspace);
    uint16_t* q_hi = reinterpret_cast<uint16_t*>(ws + rl.q_hi);
    uint16_t* q_lo = reinterpret_cast<uint16_t*>(ws + rl.q_lo);
    float* out_rot = reinterpret_cast<float*>(ws + rl.out);
    const hipStream_t s = static_cast<hipStream_t>(stream);
    const int64_t rows = (int64_t)num_seqs * num_q_heads;
    st = hip_status(fp8kv::launch_rotate_query(static_cast<const uint16_t*>(query), q_hi, q_lo, rows,
                                               head_dim, s));
    if (st != FP8KV_OK) return st;
    p.query = q_hi;
    p.query_lo = q_lo;
    p.out = out_rot;
    p.out_f32 = 1;
    st = hip_status(fp8kv::launch_decode_partial(p, codec_of(cache_dtype), head_dim, s));
    if (st != FP8KV_OK) return st;
    if (!p.write_final) {
        st = hip_status(fp8kv::launch_decode_merge(p, head_dim, s));
        if (st != FP8KV_OK) return st;
    }
    return hip_status(fp8kv::launch_rotate_out(out_rot, out, out_dtype == FP8KV_F32, rows, head_dim, s));
}

int rotated_step_impl(void* out, int out_dtype, const void* query, const void* key_new,
                      const void* value_new, void* key_cache, void* value_cache, int cache_dtype,
                      const int32_t* block_tables, int max_blocks_per_seq,
                      const int32_t* context_lens, int max_context_len, int num_seqs,
                      int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                      int num_blocks, const Scales& sc, bool per_head_call, int sliding_window,
                      int num_splits, void* counters, size_t counters_bytes, void* workspace,
                      size_t workspace_bytes, void* stream) {
    if (out_dtype != FP8KV_BF16 && out_dtype != FP8KV_F32) return FP8KV_ERR_UNSUPPORTED;
    // the rotated path is defined for the E4M3 and BF16 caches
    if (cache_dtype != FP8KV_E4M3 && cache_dtype != FP8KV_BF16) return FP8KV_ERR_UNSUPPORTED;
    int st = check_decode_shape(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                                max_context_len, sliding_window, num_splits);
    if (st != FP8KV_OK) return st;
    const Plan pl = make_plan(num_seqs, num_kv_heads, head_dim, max_context_len, sliding_window, num_splits);
    const size_t dec = workspace_layout(num_seqs, num_q_heads, head_dim, pl.splits).total;
    const RotatedLayout rl = rotated_layout(dec, num_seqs, num_q_heads, head_dim);
    fp8kv::DecodeParams p;
    bool fp8 = true;
    st = setup_decode(p, fp8, query, key_cache, value_cache, cache_dtype, block_tables,
                      max_blocks_per_seq, context_lens, max_context_len, num_seqs, num_q_heads,
                      num_kv_heads, head_dim, block_size, num_blocks, sc, per_head_call,
                      sliding_window, num_splits, workspace,
                      workspace_bytes < dec ? workspace_bytes : dec, false);
    if (st != FP8KV_OK) return st;
    if (num_seqs == 0) return FP8KV_OK;
    if (!out || !key_new || !value_new) return FP8KV_ERR_NULL;
    if (!aligned16(out) || !aligned16(key_new) || !aligned16(value_new)) return FP8KV_ERR_SHAPE;
    const int fused = attach_counters(p, head_dim, counters, counters_bytes, num_splits);
    if (fused < 0) return fused;
    const bool one_launch = p.write_final || fused;
    if (!one_launch) {   // the merge kernel writes f32 rows that one more launch rotates back
        if (!workspace || workspace_bytes < rl.total) return FP8KV_ERR_WORKSPACE;
        if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return FP8KV_ERR_WORKSPACE;
    }
    float* out_rot = one_launch ? nullptr : reinterpret_cast<float*>(static_cast<char*>(workspace) + rl.out);
    p.out = one_launch ? out : out_rot;
    p.out_f32 = one_launch ? (out_dtype == FP8KV_F32) : 1;
    p.k_new = static_cast<const uint16_t*>(key_new);
    p.v_new = static_cast<const uint16_t*>(value_new);
    p.k_scale_q = fp8 && !per_head_call ? sc.k : 1.0f;
    p.v_scale_q = fp8 && !per_head_call ? sc.v : 1.0f;
    p.rot_scale = (float)(1.0 / sqrt((double)head_dim));
    const hipStream_t s = static_cast<hipStream_t>(stream);
    st = hip_status(fp8kv::launch_decode_partial_rotated(p, codec_of(cache_dtype), head_dim, s));
    if (st != FP8KV_OK || one_launch) return st;
    st = hip_status(fp8kv::launch_decode_merge(p, head_dim, s));
    if (st != FP8KV_OK) return st;
    return hip_status(fp8kv::launch_rotate_out(out_rot, out, out_dtype == FP8KV_F32,
                                               (int64_t)num_seqs * num_q_heads, head_dim, s));
}

}  // namespace

extern "C" {

int fp8kv_paged_decode_rotated(void* out, int out_dtype, const void* query, const void* key_cache,
                               const void* value_cache, int cache_dtype,
                               const int32_t* block_tables, int max_blocks_per_seq,
                               const int32_t* context_lens, int max_context_len, int num_seqs,
                               int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                               int num_blocks, float k_scale, float v_scale, int sliding_window,
                               int num_splits, void* workspace, size_t workspace_bytes,
                               void* stream) {
    return rotated_decode_impl(out, out_dtype, query, key_cache, value_cache, cache_dtype,
                               block_tables, max_blocks_per_seq, context_lens, max_context_len,
                               num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                               num_blocks, tensor_scales(k_scale, v_scale), false, sliding_window,
                               num_splits, workspace, workspace_bytes, stream);
}

int fp8kv_paged_decode_rotated_per_head(void* out, int out_dtype, const void* query,
                                        const void* key_cache, const void* value_cache,
                                        int cache_dtype, const int32_t* block_tables,
                                        int max_blocks_per_seq, const int32_t* context_lens,
                                        int max_context_len, int num_seqs, int num_q_heads,
                                        int num_kv_heads, int head_dim, int block_size,
                                        int num_blocks, const float* k_scales,
                                        const float* v_scales, int sliding_window, int num_splits,
                                        void* workspace, size_t workspace_bytes, void* stream) {
    return rotated_decode_impl(out, out_dtype, query, key_cache, value_cache, cache_dtype,
                               block_tables, max_blocks_per_seq, context_lens, max_context_len,
                               num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                               num_blocks, head_scales(k_scales, v_scales), true, sliding_window,
                               num_splits, workspace, workspace_bytes, stream);
}

int fp8kv_decode_step_rotated(void* out, int out_dtype, const void* query, const void* key_new,
                              const void* value_new, void* key_cache, void* value_cache,
                              int cache_dtype, const int32_t* block_tables, int max_blocks_per_seq,
                              const int32_t* context_lens, int max_context_len, int num_seqs,
                              int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                              int num_blocks, float k_scale, float v_scale, int sliding_window,
                              int num_splits, void* counters, size_t counters_bytes,
                              void* workspace, size_t workspace_bytes, void* stream) {
    return rotated_step_impl(out, out_dtype, query, key_new, value_new, key_cache, value_cache,
                             cache_dtype, block_tables, max_blocks_per_seq, context_lens,
                             max_context_len, num_seqs, num_q_heads, num_kv_heads, head_dim,
                             block_size, num_blocks, tensor_scales(k_scale, v_scale), false,
                             sliding_window, num_splits, counters, counters_bytes, workspace,
                             workspace_bytes, stream);
}

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
                                       size_t workspace_bytes, void* stream) {
    return rotated_step_impl(out, out_dtype, query, key_new, value_new, key_cache, value_cache,
                             cache_dtype, block_tables, max_blocks_per_seq, context_lens,
                             max_context_len, num_seqs, num_q_heads, num_kv_heads, head_dim,
                             block_size, num_blocks, head_scales(k_scales, v_scales), true,
                             sliding_window, num_splits, counters, counters_bytes, workspace,
                             workspace_bytes, stream);
}

}  // extern "C"
