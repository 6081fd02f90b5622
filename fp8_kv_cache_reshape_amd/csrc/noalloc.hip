// noalloc.hip -- fp8kv_decode_step_noalloc: the fused decode step with its counters and split
// partials in a fixed device array of the library instead of caller buffers, for callers that
// cannot allocate device memory (code under HIP graph capture, tight serving loops, harnesses
// that forbid allocation).  The kernels are fp8kv_decode_step's; only the buffers differ.
#include <hip/hip_runtime.h>

#include <mutex>

#include "fp8kv.h"
#include "internal.h"

namespace {

// The array: counter records for up to FP8KV_NOALLOC_MAX_GROUPS (sequence, kv head) groups
// first, then up to FP8KV_NOALLOC_MAX_PARTIAL_BYTES of split partials (16 MiB in all).  Each
// GPU the library runs on holds its own copy until the process ends.
constexpr size_t kScratchCounterBytes = (size_t)FP8KV_NOALLOC_MAX_GROUPS * 1280;
constexpr size_t kScratchBytes = kScratchCounterBytes + FP8KV_NOALLOC_MAX_PARTIAL_BYTES;
static_assert(kScratchCounterBytes % 256 == 0, "partials start 256-byte aligned");
static_assert(kScratchBytes == (size_t)16 << 20, "the header documents a 16 MiB array");

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

// Zero the counter region (a fill kernel rather than a memset node: the first call may be
// recorded into a graph).
__global__ __launch_bounds__(256) void clear_words(unsigned int* p, size_t n) {
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) p[i] = 0u;
}

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};   // device address of `scratch` on each device, once known

// The array's device address on the current device (set up on the first call there: the
// address lookup, then a clear of the counter region enqueued on `stream`), or null with
// *st set to a negative status.
unsigned char* scratch_on_current_device(hipStream_t stream, int* st) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        fp8kv::record_hip_error(e != hipSuccess ? e : hipErrorInvalidDevice);
        *st = FP8KV_ERR_HIP;
        return nullptr;
    }
    std::lock_guard<std::mutex> lock(g_mu);
    if (g_ptr[dev] == nullptr) {
        void* ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || ptr == nullptr) {
            fp8kv::record_hip_error(e != hipSuccess ? e : hipErrorInvalidSymbol);
            *st = FP8KV_ERR_HIP;
            return nullptr;
        }
        // the array is zero-initialised when the code object loads; clear the counters once
        // more, in stream order before this call's kernel
        unsigned int* words = static_cast<unsigned int*>(ptr);
        size_t n = kScratchCounterBytes / 4;
        void* args[] = {&words, &n};
        e = hipLaunchKernel(reinterpret_cast<const void*>(&clear_words), dim3(1024), dim3(256), args, 0,
                            stream);
        if (e != hipSuccess) {
            fp8kv::record_hip_error(e);
            *st = FP8KV_ERR_HIP;
            return nullptr;
        }
        g_ptr[dev] = ptr;
    }
    *st = FP8KV_OK;
    return static_cast<unsigned char*>(g_ptr[dev]);
}

}  // namespace

extern "C" {

int fp8kv_decode_step_noalloc(void* out, int out_dtype, const void* query, const void* key_new,
                              const void* value_new, void* key_cache, void* value_cache,
                              int cache_dtype, const int32_t* block_tables, int max_blocks_per_seq,
                              const int32_t* context_lens, int max_context_len, int num_seqs,
                              int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                              int num_blocks, float k_scale, float v_scale, int sliding_window,
                              int num_splits, void* stream) {
    // every host check first, with no HIP call: the step's own checks, then the array's limits
    int st = fp8kv::decode_step_check(out, out_dtype, query, key_new, value_new, key_cache,
                                      value_cache, cache_dtype, block_tables, max_blocks_per_seq,
                                      context_lens, max_context_len, num_seqs, num_q_heads,
                                      num_kv_heads, head_dim, block_size, num_blocks, k_scale,
                                      v_scale, sliding_window, num_splits, kScratchCounterBytes,
                                      FP8KV_NOALLOC_MAX_PARTIAL_BYTES);
    if (st == FP8KV_ERR_WORKSPACE) return FP8KV_ERR_SCRATCH;   // the array is the workspace
    if (st != FP8KV_OK) return st;
    if (num_seqs == 0) return FP8KV_OK;
    unsigned char* base = scratch_on_current_device(static_cast<hipStream_t>(stream), &st);
    if (base == nullptr) return st;
    return fp8kv_decode_step(out, out_dtype, query, key_new, value_new, key_cache, value_cache,
                             cache_dtype, block_tables, max_blocks_per_seq, context_lens,
                             max_context_len, num_seqs, num_q_heads, num_kv_heads, head_dim,
                             block_size, num_blocks, k_scale, v_scale, sliding_window, num_splits,
                             base, kScratchCounterBytes, base + kScratchCounterBytes,
                             FP8KV_NOALLOC_MAX_PARTIAL_BYTES, stream);
}

}  // extern "C"
