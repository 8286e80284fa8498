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
// own numbering.  Sequences with no live token contribute nothing: with a
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
      n = (n_old >= 0 && n_old < a.max_len) ? n_old + 1
                                            : clamp_len(n_old, a.max_len);
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

// ---------------------------------------------------------------------------
// Index-row selection for index-gathered decode (metrale DSA topk_to_mask:
// a slot named several times counts once; INVALID and out-of-range entries
// are dropped).  One work-group per sequence marks the
// named slots in an LDS bitmap of the sequence's live length, then writes
// the set slots in ascending order (a prefix count over the bitmap words),
// which also leaves the gathered rows in address order.
namespace gqa {
namespace {

constexpr int kSelectThreads = 1024;

__global__ __launch_bounds__(kSelectThreads) void select_kernel(SelectArgs a) {
  extern __shared__ uint32_t bits[];
  __shared__ int wave_sum[kSelectThreads / 64];
  const int b = blockIdx.x;
  const int n = clamp_len(a.lens[b], a.max_len);
  const int nw = (n + 31) >> 5;
  for (int w = threadIdx.x; w < nw; w += blockDim.x) bits[w] = 0u;
  __syncthreads();
  const int32_t *row = a.idx + (size_t)b * a.width;
  for (int j = threadIdx.x; j < a.width; j += blockDim.x) {
    const int i = row[j];
    if (i >= 0 && i < n) atomicOr(&bits[i >> 5], 1u << (i & 31));
  }
  __syncthreads();
  // each thread owns a contiguous run of words; exclusive prefix of the
  // runs' bit counts across the work-group
  const int per = (nw + kSelectThreads - 1) / kSelectThreads;
  const int w0 = threadIdx.x * per, w1 = min(w0 + per, nw);
  int cnt = 0;
  for (int w = w0; w < w1; ++w) cnt += __popc(bits[w]);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int inc = cnt;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(inc, off, 64);
    if (lane >= off) inc += y;
  }
  if (lane == 63) wave_sum[wave] = inc;
  __syncthreads();
  int base = 0, total = 0;
  for (int w = 0; w < kSelectThreads / 64; ++w) {
    if (w < wave) base += wave_sum[w];
    total += wave_sum[w];
  }
  int pos = base + inc - cnt;
  int32_t *sel = a.sel + (size_t)b * a.sel_stride;
  for (int w = w0; w < w1; ++w) {
    uint32_t m = bits[w];
    while (m) {
      const int bit = __ffs(m) - 1;
      sel[pos++] = (w << 5) + bit;
      m &= m - 1;
    }
  }
  if (threadIdx.x == 0) a.count[b] = total;
}

}  // namespace

size_t select_lds_bytes(int max_len) {
  return sizeof(uint32_t) * (size_t)((max_len + 31) / 32);
}

hipError_t launch_select(const SelectArgs &a, hipStream_t s) {
  const size_t lds = select_lds_bytes(a.max_len);
  if (lds > 65536) {
    const hipError_t e = hipFuncSetAttribute(
        reinterpret_cast<const void *>(select_kernel),
        hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(select_kernel, dim3(a.batch), dim3(kSelectThreads), lds,
                     s, a);
  return hipGetLastError();
}

}  // namespace gqa
