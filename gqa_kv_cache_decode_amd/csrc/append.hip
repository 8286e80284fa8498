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

__device__ __forceinline__ void copy_row(unsigned char *dst,
                                         const unsigned char *src, int bytes) {
  const bool v16 = (((uintptr_t)dst | (uintptr_t)src | (uintptr_t)bytes) & 15) == 0;
  if (v16) {
    uint4 *d = reinterpret_cast<uint4 *>(dst);
    const uint4 *s = reinterpret_cast<const uint4 *>(src);
    for (int i = threadIdx.x; i < bytes / 16; i += blockDim.x) d[i] = s[i];
  } else {
    uint16_t *d = reinterpret_cast<uint16_t *>(dst);
    const uint16_t *s = reinterpret_cast<const uint16_t *>(src);
    for (int i = threadIdx.x; i < bytes / 2; i += blockDim.x) d[i] = s[i];
  }
}

__global__ __launch_bounds__(256) void append_kernel(AppendArgs a) {
  const int b = blockIdx.x;
  const int n = a.lens_in[b];
  const bool ok = n >= 0 && n < a.max_len;
  if (ok) {
    const size_t slot = (size_t)b * a.max_len + n;
    copy_row(static_cast<unsigned char *>(a.k) + slot * a.row_bytes_k,
             static_cast<const unsigned char *>(a.k_new) +
                 (size_t)b * a.row_bytes_k,
             a.row_bytes_k);
    copy_row(static_cast<unsigned char *>(a.v) + slot * a.row_bytes_v,
             static_cast<const unsigned char *>(a.v_new) +
                 (size_t)b * a.row_bytes_v,
             a.row_bytes_v);
  }
  __syncthreads();  // lens_in is read by every thread before lens_out is set
  if (threadIdx.x == 0) {
    a.lens_out[b] = ok ? n + 1 : n;
    if (!ok && a.dropped) atomicAdd(a.dropped, 1);
  }
}

}  // namespace

hipError_t launch_append(const AppendArgs &a, hipStream_t s) {
  hipLaunchKernelGGL(append_kernel, dim3(a.batch), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace gqa
