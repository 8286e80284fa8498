// Measurement helpers for the benchmark (not part of the decode ABI):
//  - a pure 16-byte-vector nontemporal read stream, the practical HBM read
//    ceiling the decode kernels are compared with;
//  - a plain copy of known size, whose hardware-counter readings calibrate the
//    fetch/write byte counters;
//  - a bounded spin kernel, and timing events for the decode library's
//    per-launch profiling request.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace {

__global__ __launch_bounds__(256) void read_stream_kernel(
    const uint4 *__restrict__ src, size_t n16, uint32_t *__restrict__ sink) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 *p = reinterpret_cast<const u32x4 *>(src);
  uint32_t acc = 0;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const u32x4 a = __builtin_nontemporal_load(p + i);
    const u32x4 b = __builtin_nontemporal_load(p + i + stride);
    const u32x4 c = __builtin_nontemporal_load(p + i + 2 * stride);
    const u32x4 d = __builtin_nontemporal_load(p + i + 3 * stride);
    acc ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w;
    acc ^= c.x ^ c.y ^ c.z ^ c.w ^ d.x ^ d.y ^ d.z ^ d.w;
  }
  for (; i < n16; i += stride) {
    const u32x4 a = __builtin_nontemporal_load(p + i);
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  // One word per block, written only if the xor is a value no input makes
  // likely; keeps the loads alive without a store per thread.
  if (acc == 0x9e3779b9u) sink[blockIdx.x] = acc;
}

__global__ __launch_bounds__(256) void copy_kernel(uint4 *__restrict__ dst,
                                                   const uint4 *__restrict__ src,
                                                   size_t n16) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16;
       i += stride)
    dst[i] = src[i];
}

// Keeps one wavefront busy for `ticks` of the 100 MHz real-time counter, so
// that work enqueued behind it runs back to back whatever the host's pace.
__global__ void spin_kernel(unsigned long long ticks) {
  const unsigned long long t0 = __builtin_amdgcn_s_memrealtime();
  while (__builtin_amdgcn_s_memrealtime() - t0 < ticks) __builtin_amdgcn_s_sleep(64);
}

}  // namespace

extern "C" {

// Occupies the stream for about `microseconds` (bounded).
__attribute__((visibility("default"))) int gqa_bench_spin(int microseconds,
                                                          hipStream_t stream) {
  if (microseconds <= 0 || microseconds > 1000000) return 1;
  hipLaunchKernelGGL(spin_kernel, dim3(1), dim3(64), 0, stream,
                     (unsigned long long)microseconds * 100ull);
  return hipGetLastError() == hipSuccess ? 0 : 5;
}


// Creates `n` timing events into `ev` (handles as 64-bit words).  They only
// time the launch they bracket, so they are recorded without the
// system-scope release fence (a write-back and invalidate of the L2 caches
// at each record, which would be counted in the bracketed time); the
// kernels' own completion still orders their results for the next launch.
__attribute__((visibility("default"))) int gqa_bench_events_create(
    int n, hipEvent_t *ev) {
  if (n <= 0 || !ev) return 1;
  for (int i = 0; i < n; ++i)
    if (hipEventCreateWithFlags(&ev[i], hipEventDisableSystemFence) !=
        hipSuccess)
      return 5;
  return 0;
}

__attribute__((visibility("default"))) int gqa_bench_events_destroy(
    int n, hipEvent_t *ev) {
  for (int i = 0; i < n; ++i)
    if (ev[i] && hipEventDestroy(ev[i]) != hipSuccess) return 5;
  return 0;
}

// Milliseconds between two recorded events (waits for the second).
__attribute__((visibility("default"))) int gqa_bench_events_elapsed(
    hipEvent_t a, hipEvent_t b, float *ms) {
  if (hipEventSynchronize(b) != hipSuccess) return 5;
  return hipEventElapsedTime(ms, a, b) == hipSuccess ? 0 : 5;
}

// Reads `bytes` (a multiple of 16) from `src`; `sink` needs `blocks` words.
__attribute__((visibility("default"))) int gqa_bench_read_stream(
    const void *src, size_t bytes, uint32_t *sink, int blocks,
    hipStream_t stream) {
  if (!src || !sink || bytes % 16 || blocks <= 0) return 1;
  hipLaunchKernelGGL(read_stream_kernel, dim3(blocks), dim3(256), 0, stream,
                     static_cast<const uint4 *>(src), bytes / 16, sink);
  return hipGetLastError() == hipSuccess ? 0 : 5;
}

// Copies `bytes` (a multiple of 16) from `src` to `dst`.
__attribute__((visibility("default"))) int gqa_bench_copy(void *dst,
                                                          const void *src,
                                                          size_t bytes,
                                                          int blocks,
                                                          hipStream_t stream) {
  if (!src || !dst || bytes % 16 || blocks <= 0) return 1;
  hipLaunchKernelGGL(copy_kernel, dim3(blocks), dim3(256), 0, stream,
                     static_cast<uint4 *>(dst), static_cast<const uint4 *>(src),
                     bytes / 16);
  return hipGetLastError() == hipSuccess ? 0 : 5;
}

}  // extern "C"
