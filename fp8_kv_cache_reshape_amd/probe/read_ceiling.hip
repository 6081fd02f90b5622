// Streaming-read ceiling of the GPU, measured beside the decode kernels by bench.py: a plain
// kernel that reads a buffer once with 16-byte nontemporal loads and keeps nothing, in a
// streaming pattern (grid-stride or contiguous runs per workgroup) or a paged one (1 or 2 KiB
// pieces at scattered places, the way a paged cache's blocks are read).  It is measurement
// infrastructure, not part of the fp8kv C ABI.
#include <hip/hip_runtime.h>
#include <cstddef>
#include <cstdint>

namespace {

constexpr int kThreads = 256;

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// U: independent 16-byte loads in flight per thread.  CHUNK = false: grid-stride (load u of
// a thread is u grid-widths after its first); CHUNK = true: each workgroup reads a contiguous
// run of U * 4 KiB per iteration (load u is u * 4 KiB after the first), the next run a grid
// of runs further on.
template <int U, bool CHUNK>
__global__ __launch_bounds__(kThreads) void read_ceiling_kernel(const u32x4* p, size_t n16, unsigned* sink) {
    const size_t tid = (size_t)blockIdx.x * kThreads + threadIdx.x;
    const size_t stride = (size_t)gridDim.x * kThreads;
    u32x4 acc = {0u, 0u, 0u, 0u};
    // the host guarantees n16 is a multiple of U * stride: every index below is < n16
    const size_t first = CHUNK ? (size_t)blockIdx.x * U * kThreads + threadIdx.x : tid;
    const size_t step = CHUNK ? kThreads : stride;
    for (size_t base = first; base < n16; base += U * stride) {
        u32x4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(p + base + u * step);
#pragma unroll
        for (int u = 0; u < U; ++u) acc ^= v[u];
    }
    if ((acc.x ^ acc.y ^ acc.z ^ acc.w) == 0x9E3779B9u) sink[0] = 1u;   // keeps the loads
}

// Paged reads: the buffer is nchunks chunks of P KiB (P = 1 or 2), each wave's load reads one
// KiB (64 lanes x 16 bytes), and piece k of the sweep is KiB (k mod P) of chunk
// perm(k / P), perm(c) = (c * 0x9E3779B1) mod nchunks (a bijection: nchunks is a power of
// two and the multiplier odd), so every byte is read once and consecutive chunks land far
// apart.  A wave's U loads are consecutive pieces.
template <int U, int P>
__global__ __launch_bounds__(kThreads) void read_paged_kernel(const u32x4* p, size_t n16, unsigned* sink) {
    const unsigned lane = threadIdx.x & 63u;
    const size_t wave = (size_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
    const size_t waves = (size_t)gridDim.x * (kThreads / 64);
    const size_t pieces = n16 / 64;                 // KiB pieces
    const size_t chunk_mask = pieces / P - 1;
    u32x4 acc = {0u, 0u, 0u, 0u};
    // the host guarantees pieces is a multiple of U * waves: every index below is < n16
    for (size_t base = wave * U; base < pieces; base += (size_t)U * waves) {
        u32x4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const size_t k = base + u;
            const size_t chunk = ((k / P) * 0x9E3779B1ull) & chunk_mask;
            v[u] = __builtin_nontemporal_load(p + (chunk * P + k % P) * 64 + lane);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) acc ^= v[u];
    }
    if ((acc.x ^ acc.y ^ acc.z ^ acc.w) == 0x9E3779B9u) sink[0] = 1u;   // keeps the loads
}

template <int P>
const void* paged_kernel_for(int u) {
    return u == 4 ? reinterpret_cast<const void*>(&read_paged_kernel<4, P>)
         : u == 8 ? reinterpret_cast<const void*>(&read_paged_kernel<8, P>)
                  : reinterpret_cast<const void*>(&read_paged_kernel<16, P>);
}

template <bool CHUNK>
const void* kernel_for(int u) {
    return u == 4 ? reinterpret_cast<const void*>(&read_ceiling_kernel<4, CHUNK>)
         : u == 8 ? reinterpret_cast<const void*>(&read_ceiling_kernel<8, CHUNK>)
                  : reinterpret_cast<const void*>(&read_ceiling_kernel<16, CHUNK>);
}

bool unroll_ok(int u) { return u == 4 || u == 8 || u == 16; }

}  // namespace

extern "C" {

// Bytes per launch must be a positive multiple of this, for a launch of `grid` workgroups
// with `unroll` loads in flight per thread (4, 8 or 16; else 0).
size_t fp8kv_probe_read_granule(int grid, int unroll) {
    if (!unroll_ok(unroll)) return 0;
    return (size_t)16 * unroll * kThreads * (size_t)(grid > 0 ? grid : 0);
}

// Reads `bytes` of device memory at `buf` (16-byte aligned) once, with `grid` workgroups of 256
// threads, each thread keeping `unroll` loads in flight; pattern 0 = grid-stride, 1 =
// contiguous runs per workgroup, 2 / 3 = paged reads of 1 / 2 KiB pieces (bytes a power of
// two).  `sink` is a device word the kernel may write.  Returns 0, -2 for a bad size, grid,
// unroll, pattern or alignment, -6 for a launch error.
int fp8kv_probe_read(const void* buf, size_t bytes, int grid, int unroll, int pattern, void* sink,
                     void* stream) {
    if (grid <= 0 || grid > 65536 || !unroll_ok(unroll) || pattern < 0 || pattern > 3) return -2;
    const size_t g = fp8kv_probe_read_granule(grid, unroll);
    if (!buf || !sink || bytes == 0 || bytes % g != 0 || (reinterpret_cast<uintptr_t>(buf) & 15u) != 0)
        return -2;
    if (pattern >= 2 && ((bytes & (bytes - 1)) != 0 || bytes < 4096)) return -2;
    const u32x4* p = static_cast<const u32x4*>(buf);
    size_t n16 = bytes / 16;
    unsigned* s = static_cast<unsigned*>(sink);
    void* args[] = {&p, &n16, &s};
    const void* fn = pattern == 3 ? paged_kernel_for<2>(unroll)
                   : pattern == 2 ? paged_kernel_for<1>(unroll)
                   : pattern == 1 ? kernel_for<true>(unroll) : kernel_for<false>(unroll);
    return hipLaunchKernel(fn, dim3(grid), dim3(kThreads), args, 0, static_cast<hipStream_t>(stream)) ==
                   hipSuccess ? 0 : -6;
}

}  // extern "C"
