// Work schedule of a multi-round split-K partition launch (gfx950, 8 XCDs).
//
// The hardware hands block i of a launch to XCD i % 8 and each XCD has its own
// share of the path to memory, so a launch is only as fast as its most loaded
// XCD.  With ragged lengths a fixed block -> item map leaves some XCDs with
// far more live chunks than others.  This kernel (one work-group, run just
// before the partition launch on the same stream) builds the block -> item
// table the partition kernel then reads:
//
//  1. each sequence's weight is its live chunk count nl(b) (the work of its
//     (KV group, chunk) items is at most one chunk each);
//  2. sequences are ranked by nl, largest first (a counting sort: nl takes at
//     most num_chunks + 1 values);
//  3. rank r goes to XCD snake(r): 0..7 on even rounds of eight, 7..0 on odd
//     ones, which keeps the XCD totals within one sequence's weight of each
//     other;
//  4. XCD x's items are its sequences in rank order, each contributing all of
//     its live (g, c) items, g-major (the chunks of one KV group of one
//     sequence stay together on one XCD and start together);
//  5. table entry i = j * 8 + x holds the j-th item of XCD x, or -1 past the
//     end of its list (those blocks exit at once).
//
// Items are (b * num_kv_heads + g) * num_chunks + c, the partition kernel's
// own numbering.  For a decode step this kernel also writes every sequence's
// new length and counts the drops (the partition kernels leave that to it
// when a schedule is present).  Sequences with no live token contribute nothing: with a
// schedule the partition writes partials only, and the combine kernel covers
// empty rows.
#include "device_common.h"
#include "launch.h"

namespace gqa {
namespace {

constexpr int kScheduleThreads = 1024;

// Rank of XCD x's k-th sequence under the snake order.
__device__ __forceinline__ int snake_rank(int k, int x) {
  return 8 * k + ((k & 1) ? 7 - x : x);
}

__global__ __launch_bounds__(kScheduleThreads) void schedule_kernel(
    ScheduleArgs a) {
  extern __shared__ int smem[];
  const int B = a.batch, nc = a.num_chunks;
  const int per = (B + 7) / 8;    // sequences per XCD, at most
  int *nl = smem;                 // [B] live chunks of sequence b
  int *order = nl + B;            // [B] sequence at rank r
  int *pre = order + B;           // [8][per] exclusive item prefix per XCD
  int *hist = pre + 8 * per;      // [nc + 1] then bucket cursors
  __shared__ int total[8];

  for (int v = threadIdx.x; v <= nc; v += blockDim.x) hist[v] = 0;
  __syncthreads();
  for (int b = threadIdx.x; b < B; b += blockDim.x) {
    int n;
    if (a.step) {  // decode step: the new token is attended when appended
      const int n_old = a.lens[b];
      const bool fresh = n_old >= 0 && n_old < a.max_len;
      n = fresh ? n_old + 1 : clamp_len(n_old, a.max_len);
      // needle-core push_kv: the length grows by one, or a full cache (or a
      // negative length) is left as it is and the drop counted
      a.lens_out[b] = fresh ? n_old + 1 : n_old;
      if (!fresh && a.dropped) atomicAdd(a.dropped, 1);
    } else {
      n = clamp_len(a.lens[b], a.max_len);
    }
    const int c = (n + a.chunk_tokens - 1) / a.chunk_tokens;
    nl[b] = c;
    atomicAdd(&hist[c], 1);
  }
  __syncthreads();
  // Bucket starts, largest weight first (nc + 1 buckets, one thread).
  if (threadIdx.x == 0) {
    int run = 0;
    for (int v = nc; v >= 0; --v) {
      const int h = hist[v];
      hist[v] = run;
      run += h;
    }
  }
  __syncthreads();
  // Scatter into rank order; the order inside a bucket does not matter.
  for (int b = threadIdx.x; b < B; b += blockDim.x)
    order[atomicAdd(&hist[nl[b]], 1)] = b;
  __syncthreads();
  // Per-XCD exclusive prefix of item counts over that XCD's ranks, one
  // wavefront per XCD, 64 ranks at a time.
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (wave < 8) {
    const int x = wave;
    int carry = 0;
    for (int k0 = 0; k0 < per; k0 += 64) {
      const int k = k0 + lane;
      int cnt = 0;
      if (k < per) {
        const int r = snake_rank(k, x);
        if (r < B) cnt = a.num_kv_heads * nl[order[r]];
      }
      int inc = cnt;  // inclusive scan across the wavefront
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(inc, off, 64);
        if (lane >= off) inc += y;
      }
      if (k < per) pre[x * per + k] = carry + inc - cnt;
      carry += __shfl(inc, 63, 64);
    }
    if (lane == 0) total[x] = carry;
  }
  __syncthreads();
  // Table entries: entry i = j * 8 + x is the j-th item of XCD x.
  for (int i = threadIdx.x; i < a.table_len; i += blockDim.x) {
    const int x = i & 7, j = i >> 3;
    int item = -1;
    if (j < total[x]) {
      // largest k with pre[x][k] <= j: ranks without items sort last and
      // carry the XCD total as their prefix, so they are never found
      const int *p = pre + x * per;
      int lo = 0, hi = per - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (p[mid] <= j) lo = mid; else hi = mid - 1;
      }
      const int r = snake_rank(lo, x);
      const int b = order[r];
      const int t = j - p[lo];
      const int g = t / nl[b], c = t % nl[b];
      item = (b * a.num_kv_heads + g) * nc + c;
    }
    a.table[i] = item;
  }
}

}  // namespace

size_t schedule_lds_bytes(int batch, int num_chunks) {
  const int per = (batch + 7) / 8;
  return sizeof(int) * ((size_t)2 * batch + 8 * (size_t)per + num_chunks + 1);
}

// ---------------------------------------------------------------------------
// Work queue of a balanced plan (layout in launch.h): every sequence's
// 32-token tiles are cut into runs of three shrinking lengths, listed phase
// by phase and, within a phase, sequence by sequence, so that the queue ends
// with short items whatever the lengths.  A decode step's lengths count the
// new token, and its per-sequence bookkeeping is done here as well.
namespace {

constexpr int kBalanceThreads = 1024;

// Runs of each phase for a sequence of nt tiles.
struct PhaseRuns {
  int start[kQueuePhases + 1];  // tile where each phase starts; [3] = nt
  int count[kQueuePhases];
};

__device__ __forceinline__ PhaseRuns phase_runs(int nt) {
  PhaseRuns p;
  const int64_t n = nt;
  const int e0 = (int)(n * 3 / 4 / kQueueRun0 * kQueueRun0);
  const int t1 = (int)(n * 23 / 25);
  const int e1 = e0 + max(t1 - e0, 0) / kQueueRun1 * kQueueRun1;
  p.start[0] = 0;
  p.start[1] = e0;
  p.start[2] = e1;
  p.start[3] = nt;
  p.count[0] = e0 / kQueueRun0;
  p.count[1] = (e1 - e0) / kQueueRun1;
  p.count[2] = (nt - e1 + kQueueRun2 - 1) / kQueueRun2;
  return p;
}

__device__ __forceinline__ int seq_tiles(const ScheduleArgs &a, int b,
                                         bool bookkeeping) {
  int n;
  if (a.step) {
    const int n_old = a.lens[b];
    const bool fresh = n_old >= 0 && n_old < a.max_len;
    n = fresh ? n_old + 1 : clamp_len(n_old, a.max_len);
    if (bookkeeping) {
      // needle-core push_kv: the length grows by one, or a full cache (or a
      // negative length) is left as it is and the drop counted
      a.lens_out[b] = fresh ? n_old + 1 : n_old;
      if (!fresh && a.dropped) atomicAdd(a.dropped, 1);
    }
  } else {
    n = clamp_len(a.lens[b], a.max_len);
  }
  return (n + kBalanceTile - 1) / kBalanceTile;
}

__global__ __launch_bounds__(kBalanceThreads) void balance_kernel(
    ScheduleArgs a) {
  __shared__ int wave_tot[kQueuePhases][kBalanceThreads / 64];
  __shared__ int base[kQueuePhases + 1];
  const int B = a.batch;
  int *q = a.table;
  const int per = (B + kBalanceThreads - 1) / kBalanceThreads;
  const int b0 = min((int)threadIdx.x * per, B), b1 = min(b0 + per, B);
  int mine[kQueuePhases] = {0, 0, 0};
  for (int b = b0; b < b1; ++b) {
    const PhaseRuns p = phase_runs(seq_tiles(a, b, true));
    for (int k = 0; k < kQueuePhases; ++k) mine[k] += p.count[k];
  }
  // exclusive prefix of each phase's counts across the work-group
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int inc[kQueuePhases];
  for (int k = 0; k < kQueuePhases; ++k) {
    inc[k] = mine[k];
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(inc[k], off, 64);
      if (lane >= off) inc[k] += y;
    }
    if (lane == 63) wave_tot[k][wave] = inc[k];
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int run = 0;
    for (int k = 0; k < kQueuePhases; ++k) {
      base[k] = run;
      for (int w = 0; w < kBalanceThreads / 64; ++w) run += wave_tot[k][w];
    }
    base[kQueuePhases] = run;
    q[kQueueCounter] = 0;
    q[kQueueItems] = run * a.num_kv_heads;
    for (int k = 0; k <= kQueuePhases; ++k) q[kQueueBase + k] = base[k];
  }
  __syncthreads();
  int run_at[kQueuePhases];
  for (int k = 0; k < kQueuePhases; ++k) {
    int before = 0;
    for (int w = 0; w < wave; ++w) before += wave_tot[k][w];
    run_at[k] = before + inc[k] - mine[k];  // within phase k
  }
  int *runs = q + queue_runs_offset(B);
  for (int b = b0; b < b1; ++b) {
    const PhaseRuns p = phase_runs(seq_tiles(a, b, false));
    for (int k = 0; k < kQueuePhases; ++k) {
      q[kQueuePre + k * (B + 1) + b] = run_at[k];
      const int len = k == 0 ? kQueueRun0 : k == 1 ? kQueueRun1 : kQueueRun2;
      for (int j = 0; j < p.count[k]; ++j) {
        int *r = runs + 3 * (base[k] + run_at[k] + j);
        r[0] = b;
        r[1] = p.start[k] + j * len;
        r[2] = min(p.start[k] + (j + 1) * len, p.start[k + 1]);
      }
      run_at[k] += p.count[k];
    }
  }
  if (threadIdx.x == kBalanceThreads - 1)
    for (int k = 0; k < kQueuePhases; ++k)
      q[kQueuePre + k * (B + 1) + B] = base[k + 1] - base[k];
}

}  // namespace

hipError_t launch_balance(const ScheduleArgs &a, hipStream_t s) {
  hipLaunchKernelGGL(balance_kernel, dim3(1), dim3(kBalanceThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_schedule(const ScheduleArgs &a, hipStream_t s) {
  const size_t lds = schedule_lds_bytes(a.batch, a.num_chunks);
  if (lds > 65536) {
    const hipError_t e = hipFuncSetAttribute(
        reinterpret_cast<const void *>(schedule_kernel),
        hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(schedule_kernel, dim3(1), dim3(kScheduleThreads), lds, s,
                     a);
  return hipGetLastError();
}

}  // namespace gqa
