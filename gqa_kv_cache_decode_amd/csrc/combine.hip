// Log-sum-exp combine of split-K partials, and the carry merge.
//
// Both fold online-softmax states (usearch DenseAttendConfig.carry: one state
// per query row folds a call into another over the same queries by
// partial-softmax rescaling; DenseSoftmaxState: m is the largest logit seen,
// l the sum of exponentials taken against it).  For states (m_i, l_i, acc_i)
// with M = max_i m_i:  l = sum_i e^(m_i - M) l_i,  acc = sum_i e^(m_i - M) acc_i.
// A state with l == 0 is empty and contributes nothing.  The output row is
// acc / l, already divided by the partition (usearch attend); a row with no
// keys anywhere gets 0 and the carry (-inf, 0, 0) (the DSA reference's guard:
// a softmax over nothing has weight 0, not NaN).
#include "device_common.h"
#include "launch.h"

namespace gqa {
namespace {

template <int THREADS>
__device__ __forceinline__ float block_max(float x, float *red) {
  x = wave_max(x);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  if (lane == 0) red[w] = x;
  __syncthreads();
  float r = red[0];
#pragma unroll
  for (int i = 1; i < THREADS / 64; ++i) r = fmaxf(r, red[i]);
  return r;
}

// One work-group per query row; threads are (slice, column) pairs: column
// threads cover dv, slices split the chunk list.
template <int THREADS>
__global__ __launch_bounds__(THREADS) void combine_kernel(CombineArgs a) {
  __shared__ float red[THREADS / 64];
  __shared__ float sacc[THREADS];
  __shared__ float sl[THREADS];

  const int row = blockIdx.x;
  const int b = row / a.num_q_heads;
  const int n = clamp_len(a.lens[b], a.max_len);
  const int nc = (n + a.chunk_tokens - 1) / a.chunk_tokens;
  const float *pm = a.part_m + (size_t)row * a.num_chunks;
  const float *pl = a.part_l + (size_t)row * a.num_chunks;
  const float *pa = a.part_acc + (size_t)row * a.num_chunks * a.dv;

  const float in_l = a.in_l ? a.in_l[row] : 0.0f;
  const bool has_in = in_l > 0.0f;
  const float in_m = has_in ? a.in_m[row] : -INFINITY;

  float mx = -INFINITY;
  for (int i = threadIdx.x; i < nc; i += THREADS) mx = fmaxf(mx, pm[i]);
  mx = fmaxf(block_max<THREADS>(mx, red), in_m);

  const int tps = min(THREADS, ((a.dv + 63) / 64) * 64);  // threads per slice
  const int nslice = THREADS / tps;
  const int slice = threadIdx.x / tps;
  const int col = threadIdx.x % tps;

  float acc = 0.0f, L = 0.0f;
  if (slice < nslice && col < a.dv) {
    int i = slice;
#pragma unroll 4
    for (; i < nc; i += nslice) {
      const float f = fast_exp2((pm[i] - mx) * kLog2e);
      acc += f * pa[(size_t)i * a.dv + col];
      L += f * pl[i];
    }
  }
  sacc[threadIdx.x] = acc;
  sl[threadIdx.x] = L;
  __syncthreads();
  if (slice != 0 || col >= a.dv) return;
  for (int s = 1; s < nslice; ++s) {
    acc += sacc[s * tps + col];
    L += sl[s * tps + col];
  }
  if (has_in) {
    const float f = fast_exp2((in_m - mx) * kLog2e);
    acc += f * a.in_acc[(size_t)row * a.dv + col];
    L += f * in_l;
  }
  const bool live = L > 0.0f;
  if (a.out) a.out[(size_t)row * a.dv + col] = live ? acc / L : 0.0f;
  if (a.out_acc) {
    a.out_acc[(size_t)row * a.dv + col] = live ? acc : 0.0f;
    if (col == 0) {
      a.out_m[row] = live ? mx : -INFINITY;
      a.out_l[row] = live ? L : 0.0f;
    }
  }
}

__global__ __launch_bounds__(256) void merge_kernel(MergeArgs a) {
  const size_t row = blockIdx.x;
  const float la = a.a_l[row], lb = a.b_l[row];
  const float ma = la > 0.0f ? a.a_m[row] : -INFINITY;
  const float mb = lb > 0.0f ? a.b_m[row] : -INFINITY;
  const float M = fmaxf(ma, mb);
  const float fa = la > 0.0f ? fast_exp2((ma - M) * kLog2e) : 0.0f;
  const float fb = lb > 0.0f ? fast_exp2((mb - M) * kLog2e) : 0.0f;
  const float L = fa * la + fb * lb;
  const bool live = L > 0.0f;
  __syncthreads();  // every read of m and l precedes any write (dst may alias)
  for (int d = threadIdx.x; d < a.dv; d += 256) {
    const size_t e = row * a.dv + d;
    float x = 0.0f;
    if (la > 0.0f) x += fa * a.a_acc[e];
    if (lb > 0.0f) x += fb * a.b_acc[e];
    a.d_acc[e] = live ? x : 0.0f;
    if (a.out) a.out[e] = live ? x / L : 0.0f;
  }
  if (threadIdx.x == 0) {
    a.d_m[row] = live ? M : -INFINITY;
    a.d_l[row] = live ? L : 0.0f;
  }
}

}  // namespace

hipError_t launch_combine(const CombineArgs &a, hipStream_t s) {
  const int rows = a.batch * a.num_q_heads;
  if (a.num_chunks >= 32)
    hipLaunchKernelGGL(combine_kernel<1024>, dim3(rows), dim3(1024), 0, s, a);
  else
    hipLaunchKernelGGL(combine_kernel<256>, dim3(rows), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_merge(const MergeArgs &a, hipStream_t s) {
  hipLaunchKernelGGL(merge_kernel, dim3((unsigned)a.rows), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace gqa
