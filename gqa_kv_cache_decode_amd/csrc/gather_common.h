// Index-row selection inside an index-gathered partition launch (metrale DSA
// topk_to_mask: a slot named several times counts once; INVALID (negative)
// entries and slots at or past the live length are dropped).
//
// Every work-group of sequence b rebuilds the sequence's selection from its
// index row, so no selection kernel runs before the partition launch: the
// named slots are marked in an LDS bitmap, the bitmap's words are counted
// and prefix-summed across the work-group, and the work-group keeps the
// selected slots whose ascending rank falls in its chunk.  The bitmap and
// its word list borrow LDS the work-group uses only later (its K/V tile
// area); a live length longer than the bitmap is covered window by window,
// with the ranks carried from one window to the next.
#pragma once

#include "device_common.h"

namespace gqa {

// Index entries loaded per thread before their bitmap updates are issued
// (the loads of one batch are all in flight together).
constexpr int kSelectBatch = 16;

// Exclusive prefix sum of v over the NT threads of the work-group; `total`
// receives the sum of all.  s_wave holds NT / 64 ints; the caller puts a
// barrier between two uses of the same s_wave.
template <int NT>
__device__ __forceinline__ int block_exclusive_sum(int v, int *s_wave,
                                                   int &total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int inc = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(inc, off, 64);
    if (lane >= off) inc += y;
  }
  if (lane == 63) s_wave[wave] = inc;
  __syncthreads();
  int before = 0;
  total = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) {
    const int t = s_wave[w];
    before += w < wave ? t : 0;
    total += t;
  }
  return before + inc - v;
}

// Sequence b's selection (`row`: its `width` index entries; n: its live
// length): writes the selected slots of ascending rank lo, lo + 1, ...,
// below lo + cap to s_slot[0, 1, ...] and returns the selection's size.
// `lds` is LDS scratch of lds_words words (its contents are lost): a
// quarter holds the window's bitmap, the rest the list of the words that
// hold ranks of the chunk (each word's index, bits and first rank).  s_wave
// holds 2 * NT / 64 ints.  Every thread of the work-group calls it; when
// n > 0 it ends with a barrier, after which s_slot is complete.
//
// Expanding the words into slots is spread over the whole work-group: each
// half-wavefront takes one listed word at a time, lane j placing bit j, so
// a dense run of slots (a pool of consecutive tokens) costs no more than a
// sparse one.
template <int NT>
__device__ int gather_select(const int32_t *row, int width, int n, int lo,
                             int cap, int *s_slot, uint32_t *lds,
                             int lds_words, int *s_wave) {
  const int hi = lo + cap;
  const int win = lds_words / 4;  // bitmap words per window
  uint32_t *bits = lds;
  int *list_w = reinterpret_cast<int *>(lds + win);
  int *list_r = list_w + win;
  uint32_t *list_m = reinterpret_cast<uint32_t *>(list_r + win);
  const int j = threadIdx.x & 31;
  const int half = threadIdx.x >> 5;  // half-wavefront index
  int base = 0;  // rank of the window's first selected slot
  for (int s0 = 0; s0 < n; s0 += win * 32) {
    const int s1 = min(s0 + win * 32, n);
    const int nw = (s1 - s0 + 31) >> 5;
    // the first batch of index entries is loaded while the bitmap clears
    int v[kSelectBatch];
#pragma unroll
    for (int k = 0; k < kSelectBatch; ++k)
      v[k] = row[min(k * NT + (int)threadIdx.x, width - 1)];
    for (int w = threadIdx.x; w < nw; w += NT) bits[w] = 0u;
    __syncthreads();
    for (int j0 = 0; j0 < width; j0 += NT * kSelectBatch) {
      if (j0 > 0) {
        // clamped indices, no branch per load: each load is issued before
        // any result is needed
#pragma unroll
        for (int k = 0; k < kSelectBatch; ++k)
          v[k] = row[min(j0 + k * NT + (int)threadIdx.x, width - 1)];
      }
#pragma unroll
      for (int k = 0; k < kSelectBatch; ++k) {
        const int i = v[k];
        if (j0 + k * NT + (int)threadIdx.x < width && i >= s0 && i < s1)
          atomicOr(&bits[(i - s0) >> 5], 1u << ((i - s0) & 31));
      }
    }
    __syncthreads();
    // each thread takes a contiguous run of words: their set bits, prefix-
    // summed across the work-group, give each word's first rank; the words
    // holding ranks in [lo, hi) are then listed, in order
    const int per = (nw + NT - 1) / NT;
    const int w0 = min((int)threadIdx.x * per, nw), w1 = min(w0 + per, nw);
    int cnt = 0;
    for (int w = w0; w < w1; ++w) cnt += __popc(bits[w]);
    int total, listed;
    const int pos0 = base + block_exclusive_sum<NT>(cnt, s_wave, total);
    int mine = 0, pos = pos0;
    for (int w = w0; w < w1 && pos < hi; ++w) {
      const int pc = __popc(bits[w]);
      mine += pc != 0 && pos + pc > lo;
      pos += pc;
    }
    int k = block_exclusive_sum<NT>(mine, s_wave + NT / 64, listed);
    pos = pos0;
    for (int w = w0; w < w1 && pos < hi; ++w) {
      const uint32_t m = bits[w];
      const int pc = __popc(m);
      if (pc != 0 && pos + pc > lo) {
        list_w[k] = w;
        list_r[k] = pos;
        list_m[k] = m;
        ++k;
      }
      pos += pc;
    }
    __syncthreads();
    for (int e = half; e < listed; e += NT / 32) {
      const uint32_t m = list_m[e];
      if ((m >> j) & 1u) {
        const int r = list_r[e] + __popc(m & ((1u << j) - 1u));
        if (r >= lo && r < hi) s_slot[r - lo] = s0 + (list_w[e] << 5) + j;
      }
    }
    base += total;
    __syncthreads();  // the bitmap, list and s_wave are reused next window
  }
  return base;
}

}  // namespace gqa
