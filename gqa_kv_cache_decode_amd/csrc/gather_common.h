// Index-row selection inside an index-gathered partition launch (metrale DSA
// topk_to_mask: a slot named several times counts once; INVALID (negative)
// entries and slots at or past the live length are dropped).
//
// Every work-group of sequence b rebuilds the sequence's selection from its
// index row, so no selection kernel runs before the partition launch: the
// named slots are marked in an LDS bitmap, the bitmap's words are counted
// and prefix-summed across the work-group, and the work-group keeps the
// selected slots whose ascending rank falls in its chunk.  The bitmap and
// its words' first ranks borrow LDS the work-group uses only later (its K/V
// tile area); a live length longer than the bitmap is covered window by
// window, with the ranks carried from one window to the next.
#pragma once

#include "device_common.h"

namespace gqa {

// Index entries loaded per thread before their bitmap updates are issued
// (the loads of one batch are all in flight together).
constexpr int kSelectBatch = 16;

// Inclusive prefix sum of x over the 64 lanes of a wavefront, on DPP lane
// moves (no LDS round trips): Hillis-Steele within each 16-lane row (row
// shifts by 1, 2, 4, 8; lanes shifted in from outside the row read 0), then
// rows 1 and 3 add the last lane of rows 0 and 2 (row_bcast:15), and rows 2
// and 3 add lane 31 (row_bcast:31), the running total of rows 0 and 1.
__device__ __forceinline__ int wave_inclusive_sum(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, true);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, true);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, true);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, true);  // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);  // row_bcast:15
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);  // row_bcast:31
  return x;
}

// Exclusive prefix sum of v over the NT threads of the work-group; `total`
// receives the sum of all.  s_wave holds NT / 64 ints; the caller puts a
// barrier between two uses of the same s_wave.
template <int NT>
__device__ __forceinline__ int block_exclusive_sum(int v, int *s_wave,
                                                   int &total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int inc = wave_inclusive_sum(v);
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

// Words of the window's bitmap one thread holds in registers, at most.
constexpr int kSelectWordsPerThread = 16;

// Sequence b's selection (`row`: its `width` index entries; n: its live
// length): writes the selected slots of ascending rank lo, lo + 1, ...,
// below lo + cap to s_slot[0, 1, ...] and returns the selection's size.
// `lds` is LDS scratch of lds_words words (its contents are lost): the
// window's bitmap, the first rank of each of its words, and two words for
// the range below.  s_wave holds NT / 64 ints.  Every thread of the
// work-group calls it; when n > 0 it ends with a barrier, after which s_slot
// is complete.
//
// Each thread holds a contiguous run of the bitmap's words in registers; one
// prefix sum of their set bits gives every word its first rank.  Ranks grow
// with the word index, so the words holding ranks of the chunk form one
// contiguous range of words, which the work-group expands into slots: each
// wavefront reads 64 words of the range at a time and places the bits of
// the nonzero ones, a word per half-wavefront, lane j placing bit j, so a
// dense run of slots (a pool of consecutive tokens) costs no more than a
// sparse one and an empty word costs almost nothing.
template <int NT>
__device__ __forceinline__ int gather_select(const int32_t *row, int width,
                                             int n, int lo, int cap,
                                             int *s_slot, uint32_t *lds,
                                             int lds_words, int *s_wave) {
  constexpr int kPer = kSelectWordsPerThread;
  const int hi = lo + cap;
  // bitmap words per window: the bitmap and its first ranks fit the scratch,
  // and every thread's share fits its registers
  const int win = min((lds_words - 2) / 2, NT * kPer);
  uint32_t *bits = lds;
  int *wpos = reinterpret_cast<int *>(lds + win);
  int *range = reinterpret_cast<int *>(lds + lds_words - 2);  // [wa, wb]
  const int j = threadIdx.x & 31;  // the bit a lane places
  // the first batch of index entries is loaded before anything waits for
  // n (the caller's length load is then in flight with it) and again at each
  // later window, while the bitmap clears
  int v[kSelectBatch];
#pragma unroll
  for (int k = 0; k < kSelectBatch; ++k)
    v[k] = row[min(k * NT + (int)threadIdx.x, width - 1)];
  int base = 0;  // rank of the window's first selected slot
  for (int s0 = 0; s0 < n; s0 += win * 32) {
    const int s1 = min(s0 + win * 32, n);
    const int nw = (s1 - s0 + 31) >> 5;
    if (s0 > 0) {
#pragma unroll
      for (int k = 0; k < kSelectBatch; ++k)
        v[k] = row[min(k * NT + (int)threadIdx.x, width - 1)];
    }
    for (int w = threadIdx.x; w < nw; w += NT) bits[w] = 0u;
    if (threadIdx.x == 0) {
      range[0] = nw;
      range[1] = -1;
    }
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
    // this thread's words [w0, w1) (per <= kPer since nw <= NT * kPer)
    const int per = (nw + NT - 1) / NT;
    const int w0 = min((int)threadIdx.x * per, nw), w1 = min(w0 + per, nw);
    uint32_t m[kPer];
    int cnt = 0;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      m[i] = w0 + i < w1 ? bits[w0 + i] : 0u;
      cnt += __popc(m[i]);
    }
    int total;
    int pos = base + block_exclusive_sum<NT>(cnt, s_wave, total);
    int wa = nw, wb = -1;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      if (w0 + i < w1) {
        const int pc = __popc(m[i]);
        wpos[w0 + i] = pos;
        if (pc != 0 && pos < hi && pos + pc > lo) {
          wa = min(wa, w0 + i);
          wb = w0 + i;
        }
        pos += pc;
      }
    }
    if (wb >= 0) {
      atomicMin(&range[0], wa);
      atomicMax(&range[1], wb);
    }
    __syncthreads();
    // expansion: each wavefront reads 64 consecutive words of the range (and
    // their first ranks) at a time and places the bits of its nonzero words,
    // two words per pass (lanes 0-31 the first, 32-63 the second, lane j
    // placing bit j); empty words cost one coalesced read
    const int ra = __builtin_amdgcn_readfirstlane(range[0]);
    const int rb = __builtin_amdgcn_readfirstlane(range[1]);
    const int lane = threadIdx.x & 63;
    for (int wb0 = ra + (int)(threadIdx.x >> 6) * 64; wb0 <= rb; wb0 += NT) {
      const int w = wb0 + lane;
      const uint32_t mw = w <= rb ? bits[w] : 0u;
      const int pw = w <= rb ? wpos[w] : 0;
      unsigned long long nz = __ballot(mw != 0u);
      while (nz) {
        const int k1 = __builtin_ctzll(nz);
        nz &= nz - 1;
        const bool two = nz != 0;
        const int k2 = two ? __builtin_ctzll(nz) : k1;
        if (two) nz &= nz - 1;
        const bool second = lane >= 32;
        const int k = second ? k2 : k1;
        const uint32_t m1 = (uint32_t)__builtin_amdgcn_readlane((int)mw, k1);
        const uint32_t m2 = (uint32_t)__builtin_amdgcn_readlane((int)mw, k2);
        const int p1 = __builtin_amdgcn_readlane(pw, k1);
        const int p2 = __builtin_amdgcn_readlane(pw, k2);
        const uint32_t mk = second ? m2 : m1;
        const int pk = second ? p2 : p1;
        if ((!second || two) && ((mk >> j) & 1u)) {
          const int r = pk + __popc(mk & ((1u << j) - 1u));
          if (r >= lo && r < hi) s_slot[r - lo] = s0 + ((wb0 + k) << 5) + j;
        }
      }
    }
    base += total;
    __syncthreads();  // the bitmap, ranks, range and s_wave are reused next window
  }
  return base;
}

}  // namespace gqa
