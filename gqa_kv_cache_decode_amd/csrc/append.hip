// kv_append: needle-core KvCache::push_kv, one work-group per sequence.
//
// With n = lens_in[b]: if 0 <= n < max_len the token's rows for every KV head
// ([num_kv_heads][d], contiguous in the [max_len][num_kv_heads][d] layout)
// are copied to slot n and lens_out[b] = n + 1.  Otherwise nothing is written
// and the drop is counted: the page warns that the cache is full and returns
// without writing.
#include "device_common.h"
#include "launch.h"

namespace gqa {
namespace {

constexpr int kThreads = 256;
constexpr int kPieces = 4;  // 16-byte pieces per thread held in registers

// Copies one row; pieces of 16 bytes when everything is 16-byte aligned.
// The source pieces are loaded before the destination slot is known, so the
// loads overlap the read of the length.
__device__ __forceinline__ void copy_rows(unsigned char *kd, const unsigned char *ks,
                                          int kbytes, unsigned char *vd,
                                          const unsigned char *vs, int vbytes,
                                          bool aligned, bool ok) {
  if (aligned) {
    const int nk = kbytes / 16, nv = vbytes / 16;
    const u32x4 *k16 = reinterpret_cast<const u32x4 *>(ks);
    const u32x4 *v16 = reinterpret_cast<const u32x4 *>(vs);
    u32x4 kb[kPieces], vb[kPieces];
#pragma unroll
    for (int p = 0; p < kPieces; ++p) {
      const int i = threadIdx.x + p * kThreads;
      if (i < nk) kb[p] = k16[i];
      if (i < nv) vb[p] = v16[i];
    }
    if (!ok) return;
#pragma unroll
    for (int p = 0; p < kPieces; ++p) {
      const int i = threadIdx.x + p * kThreads;
      if (i < nk) reinterpret_cast<u32x4 *>(kd)[i] = kb[p];
      if (i < nv) reinterpret_cast<u32x4 *>(vd)[i] = vb[p];
    }
    for (int i = threadIdx.x + kPieces * kThreads; i < nk; i += kThreads)
      reinterpret_cast<u32x4 *>(kd)[i] = k16[i];
    for (int i = threadIdx.x + kPieces * kThreads; i < nv; i += kThreads)
      reinterpret_cast<u32x4 *>(vd)[i] = v16[i];
  } else if (ok) {
    for (int i = threadIdx.x; i < kbytes / 2; i += kThreads)
      reinterpret_cast<uint16_t *>(kd)[i] = reinterpret_cast<const uint16_t *>(ks)[i];
    for (int i = threadIdx.x; i < vbytes / 2; i += kThreads)
      reinterpret_cast<uint16_t *>(vd)[i] = reinterpret_cast<const uint16_t *>(vs)[i];
  }
}

__global__ __launch_bounds__(kThreads) void append_kernel(AppendArgs a) {
  const int b = blockIdx.x;
  const int n = a.lens_in[b];
  const bool ok = n >= 0 && n < a.max_len;
  const size_t slot = (size_t)b * a.max_len + (ok ? n : 0);
  unsigned char *kd = static_cast<unsigned char *>(a.k) + slot * a.row_bytes_k;
  unsigned char *vd = static_cast<unsigned char *>(a.v) + slot * a.row_bytes_v;
  const unsigned char *ks =
      static_cast<const unsigned char *>(a.k_new) + (size_t)b * a.row_bytes_k;
  const unsigned char *vs =
      static_cast<const unsigned char *>(a.v_new) + (size_t)b * a.row_bytes_v;
  const bool aligned = ((reinterpret_cast<uintptr_t>(a.k) |
                         reinterpret_cast<uintptr_t>(a.v) |
                         reinterpret_cast<uintptr_t>(a.k_new) |
                         reinterpret_cast<uintptr_t>(a.v_new) |
                         (uintptr_t)a.row_bytes_k | (uintptr_t)a.row_bytes_v) &
                        15) == 0;
  copy_rows(kd, ks, a.row_bytes_k, vd, vs, a.row_bytes_v, aligned, ok);
  __syncthreads();  // lens_in is read by every thread before lens_out is set
  if (threadIdx.x == 0) {
    a.lens_out[b] = ok ? n + 1 : n;
    if (!ok && a.dropped) atomicAdd(a.dropped, 1);
  }
}

}  // namespace

hipError_t launch_append(const AppendArgs &a, hipStream_t s) {
  hipLaunchKernelGGL(append_kernel, dim3(a.batch), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace gqa
