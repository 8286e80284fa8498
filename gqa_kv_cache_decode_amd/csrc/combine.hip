// Log-sum-exp combine of split-K partials, and the carry merge.
//
// Both fold online-softmax states (usearch DenseAttendConfig.carry: a state per
// query row lets one call resume another on the same query rows, rescaling
// the partial softmaxes; DenseSoftmaxState: m is the maximum logit so far and
// l the sum of exponentials relative to m).  For states (m_i, l_i, acc_i)
// with M = max_i m_i:  l = sum_i e^(m_i - M) l_i,  acc = sum_i e^(m_i - M) acc_i.
// A state with l == 0 is empty and contributes nothing.  The output row is
// acc / l, i.e. normalised by the partition (usearch attend); a row with no
// keys anywhere gets 0 and the carry (-inf, 0, 0) (the DSA reference's guard:
// an empty softmax contributes zero weight instead of a NaN).
#include "device_common.h"
#include "launch.h"

namespace gqa {
namespace {

// One work-group per query row; threads are (slice, column) pairs: column
// threads cover dv, slices split the chunk list.  Each thread folds its chunks
// online (so every partial load can be in flight at once), then the slices
// fold through LDS.
template <int THREADS>
__global__ __launch_bounds__(THREADS) void combine_kernel(CombineArgs a) {
  __shared__ float sm[THREADS];
  __shared__ float sl[THREADS];
  __shared__ float sacc[THREADS];

  const int row = blockIdx.x;
  const int b = row / a.num_q_heads;
  const int tps = min(THREADS, ((a.dv + 63) / 64) * 64);  // threads per slice
  const int nslice = THREADS / tps;
  const int slice = threadIdx.x / tps;
  const int col = threadIdx.x % tps;
  const bool worker = slice < nslice && col < a.dv;

  const float in_l = a.in_l ? a.in_l[row] : 0.0f;
  const bool has_in = in_l > 0.0f;
  const float in_m = has_in ? a.in_m[row] : -INFINITY;
  const float in_acc =
      (has_in && worker) ? a.in_acc[(size_t)row * a.dv + col] : 0.0f;

  const float *pm = a.part_m + (size_t)row * a.total_cols;
  const float *pl = a.part_l + (size_t)row * a.total_cols;
  const float *pa = a.part_acc + (size_t)row * a.total_cols * a.dv;

  float m = -INFINITY, L = 0.0f, acc = 0.0f;  // base-2 running state
  if (worker) {
    // every branch's live chunks: columns col_base .. col_base + nc - 1
    for (int br = 0; br < a.num_branches; ++br) {
      const CombineBranch &x = a.br[br];
      const int n = clamp_len(x.lens[b], x.max_len);
      const int nc = (n + x.chunk_tokens - 1) / x.chunk_tokens;
#pragma unroll 4
      for (int i = x.col_base + slice; i < x.col_base + nc; i += nslice) {
        const float mi = pm[i] * kLog2e;
        const float li = pl[i];
        const float ai = pa[(size_t)i * a.dv + col];
        // a chunk whose keys were all removed by the bias has m = -inf, l = 0
        const float mn = fmaxf(m, mi), ref = exp_ref(mn);
        const float fo = fast_exp2(m - ref), fi = fast_exp2(mi - ref);
        acc = acc * fo + ai * fi;
        L = L * fo + li * fi;
        m = mn;
      }
    }
  }
  sm[threadIdx.x] = m;
  sl[threadIdx.x] = L;
  sacc[threadIdx.x] = acc;
  __syncthreads();
  if (slice != 0 || !worker) return;

  float M = has_in ? in_m * kLog2e : -INFINITY;
  for (int s = 0; s < nslice; ++s) M = fmaxf(M, sm[s * tps + col]);
  acc = 0.0f;
  L = 0.0f;
  if (M != -INFINITY) {
    for (int s = 0; s < nslice; ++s) {
      const float f = fast_exp2(sm[s * tps + col] - M);
      acc += f * sacc[s * tps + col];
      L += f * sl[s * tps + col];
    }
    if (has_in) {
      const float f = fast_exp2(in_m * kLog2e - M);
      acc += f * in_acc;
      L += f * in_l;
    }
  }
  const bool live = L > 0.0f;
  if (a.out) a.out[(size_t)row * a.dv + col] = live ? acc / L : 0.0f;
  if (a.out_acc) {
    a.out_acc[(size_t)row * a.dv + col] = live ? acc : 0.0f;
    if (col == 0) {
      a.out_m[row] = live ? M * kLn2 : -INFINITY;
      a.out_l[row] = live ? L : 0.0f;
    }
  }
}

// Balanced plans: one work-group per query row, one thread per value column.
// The row's sequence b has, in each phase k of the work queue, the runs
// base[k] + pre_k[b] .. base[k] + pre_k[b + 1] - 1; queue item r *
// num_kv_heads + g (g the row's KV group) left its piece in that slot.  The
// pieces and carry_in fold by log-sum-exp merge.
//
// The fold is shaped for latency: the three phases' bounds are read in one
// round, then every piece's m and l (one piece per thread, into LDS) and
// each column's first kCombineRegs values go out together; the weights
// 2^(m_i - M) are formed from LDS by every thread, so no piece waits for the
// one before it.  More pieces than a batch of LDS slots fold batch by batch
// with the usual rescale.
constexpr int kCombineRegs = 16;
constexpr int kCombineBatch = 256;

// Slot of piece i of a row whose phases hold n0, n01 - n0 and the rest of
// its pieces, from runs r0 + i, r1 + i and r2 + i (r1, r2 offset by the
// earlier phases' counts).
__device__ __forceinline__ size_t piece_slot(int i, int n0, int n01, int r0,
                                             int r1, int r2,
                                             size_t run_stride, size_t col) {
  const int r = i < n0 ? r0 + i : i < n01 ? r1 + i : r2 + i;
  return (size_t)r * run_stride + col;
}

__global__ __launch_bounds__(256) void combine_balanced_kernel(CombineArgs a) {
  __shared__ int s_r0[kQueuePhases], s_n[kQueuePhases];
  __shared__ float s_m[kCombineBatch], s_l[kCombineBatch];
  const int row = blockIdx.x;
  const int d = threadIdx.x, nt = blockDim.x;
  const int Hq = a.num_q_heads, hpk = a.hpk, Hkv = Hq / hpk;
  const int b = row / Hq, h = row % Hq, g = h / hpk, hh = h % hpk;
  const int B = a.batch;
  const bool worker = d < a.dv;
  // carry_in is read before the barriers below: carry_out may alias it
  const float in_l = a.in_l ? a.in_l[row] : 0.0f;
  const float in_m = in_l > 0.0f ? a.in_m[row] : -INFINITY;
  const float in_acc =
      in_l > 0.0f && worker ? a.in_acc[(size_t)row * a.dv + d] : 0.0f;
  if (d < kQueuePhases) {
    const int *pre = a.queue + kQueuePre + d * (B + 1);
    s_r0[d] = a.queue[kQueueBase + d] + pre[b];
    s_n[d] = pre[b + 1] - pre[b];
  }
  __syncthreads();
  const int n0 = s_n[0], n01 = n0 + s_n[1], n = n01 + s_n[2];
  const int r0 = s_r0[0], r1 = s_r0[1] - n0, r2 = s_r0[2] - n01;
  const size_t col = (size_t)g * hpk + hh;
  const size_t run_stride = (size_t)Hkv * hpk;
  auto slot = [=](int i) {
    return piece_slot(i, n0, n01, r0, r1, r2, run_stride, col);
  };
  // The loads carry no branch of their own (a branch per load would make the
  // compiler wait for each before the next): pieces past n repeat the last.
  const int dd = worker ? d : 0;
  float av[kCombineRegs];
  if (n > 0) {
#pragma unroll
    for (int i = 0; i < kCombineRegs; ++i)
      av[i] = a.part_acc[slot(min(i, n - 1)) * a.dv + dd];
  }

  float m = -INFINITY, L = 0.0f, acc = 0.0f;  // base-2 running state
  for (int i0 = 0; i0 < n; i0 += kCombineBatch) {
    const int nb = min(kCombineBatch, n - i0);
    for (int i = d; i < nb; i += nt) {
      const size_t pr = slot(i0 + i);
      const float li = a.part_l[pr], mi = a.part_m[pr];
      // a piece whose keys were all removed by the bias has l = 0
      s_m[i] = li > 0.0f ? mi * kLog2e : -INFINITY;
      s_l[i] = li;
    }
    __syncthreads();
    float mb = -INFINITY;
    for (int i = 0; i < nb; ++i) mb = fmaxf(mb, s_m[i]);
    const float mn = fmaxf(m, mb), ref = exp_ref(mn);
    const float fo = fast_exp2(m - ref);
    acc *= fo;
    L *= fo;
    m = mn;
    int i = 0;
    if (i0 == 0) {
#pragma unroll
      for (int j = 0; j < kCombineRegs; ++j) {
        const int jj = min(j, nb - 1);
        const float w = j < nb ? fast_exp2(s_m[jj] - ref) : 0.0f;
        L += w * s_l[jj];
        acc += w * av[j];
      }
      i = kCombineRegs;
    }
#pragma unroll 8
    for (; i < nb; ++i) {
      const float w = fast_exp2(s_m[i] - ref);
      L += w * s_l[i];
      if (worker) acc += w * a.part_acc[slot(i0 + i) * a.dv + d];
    }
    __syncthreads();  // the batch's LDS slots are read before the next fill
  }
  if (in_l > 0.0f) {
    const float mi = in_m * kLog2e;
    const float mn = fmaxf(m, mi), ref = exp_ref(mn);
    const float fo = fast_exp2(m - ref), fi = fast_exp2(mi - ref);
    acc = acc * fo + in_acc * fi;
    L = L * fo + in_l * fi;
    m = mn;
  }
  if (!worker) return;
  const bool live = L > 0.0f;
  if (a.out) a.out[(size_t)row * a.dv + d] = live ? acc / L : 0.0f;
  if (a.out_acc) {
    a.out_acc[(size_t)row * a.dv + d] = live ? acc : 0.0f;
    if (d == 0) {
      a.out_m[row] = live ? m * kLn2 : -INFINITY;
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
  if (a.balanced) {
    if (a.dv > 256 || a.num_branches != 1) return hipErrorInvalidValue;
    hipLaunchKernelGGL(combine_balanced_kernel, dim3(rows),
                       dim3((a.dv + 63) / 64 * 64), 0, s, a);
    return hipGetLastError();
  }
  if (a.total_cols >= 32)
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
