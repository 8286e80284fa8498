// Device helpers shared by the partition kernels when they run a whole decode
// step in one launch: the append of the new token, the per-sequence length it
// implies, the arrival count of a KV group's work-groups, and the fold of the
// group's split-K partials that the last work-group to arrive performs.
#pragma once

#include "device_common.h"
#include "launch.h"

namespace gqa {

// s_waitcnt immediate (GFX9 encoding) waiting for vmcnt = 0 only: every
// vector memory access of the wavefront, stores included, has completed.
constexpr int kWaitVmcnt0 = 0x0F70;

// Points `a` at the branch that owns block `item` of a multi-branch launch
// (branches hold ascending block ranges) and makes `item` local to it.
__device__ __forceinline__ int select_branch(PartitionArgs &a, int &item) {
  // (a one-cache launch reads none of the further branches' fields)
  if (a.num_extra == 0) return 0;
  int base = 0, branch = 0;
#pragma unroll
  for (int e = 0; e < kMaxExtraBranches; ++e) {
    if (e < a.num_extra && item >= a.extra[e].item_base) {
      branch = e + 1;
      const ExtraBranch &x = a.extra[e];
      a.k = x.k;
      a.v = x.v;
      a.k_scale = x.k_scale;
      a.v_scale = x.v_scale;
      a.lens = x.lens;
      a.bias = x.bias;
      a.bias_stride = x.bias_stride;
      a.max_len = x.max_len;
      a.cache_len = x.max_len;
      a.chunk_tokens = x.chunk_tokens;
      a.num_chunks = x.num_chunks;
      a.col_base = x.col_base;
      base = x.item_base;
    }
  }
  item -= base;
  return branch;
}

// Keys attended by sequence b, and the slot a decode step appends to.
struct SeqLen {
  int n;      // keys attended: [0, n)
  int n_old;  // slot receiving the new token when `fresh`
  bool fresh;
};

// needle-core decode order: push_kv, then attend over the cache including the
// new token (`stepping`: this branch receives the token of a decode step).  A full cache (or a negative length) is left as it is: the step
// attends over what is there and the drop is counted.
__device__ __forceinline__ SeqLen seq_len(const PartitionArgs &a,
                                          const StepParams &sp, int b,
                                          bool stepping) {
  SeqLen s;
  if (stepping) {
    s.n_old = sp.lens_in[b];
    s.fresh = s.n_old >= 0 && s.n_old < a.max_len;
    s.n = s.fresh ? s.n_old + 1 : clamp_len(s.n_old, a.max_len);
  } else {
    s.n_old = -1;
    s.fresh = false;
    s.n = clamp_len(a.lens[b], a.max_len);
  }
  return s;
}

// The new lengths and the drop count, written once per sequence (by its first
// work-group).  lens_out never aliases lens_in, which every group still reads.
__device__ __forceinline__ void step_bookkeeping(const StepParams &sp, int b,
                                                 const SeqLen &s) {
  sp.lens_out[b] = s.fresh ? s.n_old + 1 : s.n_old;
  if (!s.fresh && sp.dropped) atomicAdd(sp.dropped, 1);
}

// Stores one KV group's rows of the new token (16-byte pieces) into the cache
// slot, spread over the threads first, first + stride, ...  Nothing in the same launch reads the slot, so the stores are not
// waited for; the launch's end makes them visible to later calls.
__device__ __forceinline__ void store_group_row(const u32x4 *kn, u32x4 *kd,
                                                int kpieces, const u32x4 *vn,
                                                u32x4 *vd, int vpieces,
                                                int first, int stride) {
  for (int e = first; e < kpieces + vpieces; e += stride) {
    if (e < kpieces)
      kd[e] = kn[e];
    else
      vd[e - kpieces] = vn[e - kpieces];
  }
}

// Stores and loads of split-K partials that another work-group of the same
// launch may read: device-coherent accesses (agent scope), which go to the
// coherence point instead of one XCD's L2.  This avoids the L2-wide write-back
// and invalidate that an agent-scope fence costs on a multi-XCD part.
__device__ __forceinline__ void coherent_store(float *p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float coherent_load(const float *p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Counts this work-group's arrival once its partial is published; true in the
// last of the `nc` work-groups of group (b, g), which then reads every partial
// with coherent loads.  Each wavefront first waits for its own coherent
// partial stores to complete (s_waitcnt vmcnt(0)), so every partial is at the
// coherence point before the counter moves.  The counter returns to zero for
// the next call.
__device__ __forceinline__ bool arrive_last(int *counter, int nc, int *flag) {
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  __syncthreads();
  if (threadIdx.x == 0) {
    const int prev = __hip_atomic_fetch_add(counter, 1, __ATOMIC_RELAXED,
                                            __HIP_MEMORY_SCOPE_AGENT);
    const int last = prev == nc - 1;
    if (last)
      __hip_atomic_store(counter, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *flag = last;
  }
  __syncthreads();
  return *flag != 0;
}

// carry_in's m (in base-2 units, -inf when empty) and l of the hpk query rows
// from row0 on, staged in LDS as s_in[h] and s_in[hpk + h].  Callers read them
// after a work-group barrier, and write carry_out only after that barrier, so
// carry_out may alias carry_in.
__device__ __forceinline__ void stage_carry_in(const StepParams &sp,
                                               size_t row0, int hpk,
                                               float *s_in) {
  for (int h = threadIdx.x; h < hpk; h += blockDim.x) {
    const float l = sp.in_l ? sp.in_l[row0 + h] : 0.0f;
    s_in[h] = l > 0.0f ? sp.in_m[row0 + h] * kLog2e : -INFINITY;
    s_in[hpk + h] = l;
  }
}

// Log-sum-exp merge of one column of a state (m in base-2 units, partition L,
// unnormalised acc) with another (usearch carry: both partial softmaxes are
// rescaled to the common maximum).  An empty state (l == 0) is the identity.
__device__ __forceinline__ void fold_state(float &m, float &L, float &acc,
                                           float m_b, float l_b, float acc_b) {
  if (l_b > 0.0f) {
    const float mn = fmaxf(m, m_b);
    const float fa = fast_exp2(m - mn), fb = fast_exp2(m_b - mn);
    L = L * fa + l_b * fb;
    acc = acc * fa + acc_b * fb;
    m = mn;
  }
}

// Writes column d of query row `row` from its final state: out = acc / L
// (usearch: the output rows come normalised by the partition) and carry_out;
// an empty state gives out 0 and carry (-inf, 0, 0).
__device__ __forceinline__ void write_final(const StepParams &sp, size_t row,
                                            int dv, int d, float m, float L,
                                            float acc) {
  const bool live = L > 0.0f;
  if (sp.out) sp.out[row * dv + d] = live ? acc / L : 0.0f;
  if (sp.out_acc) {
    sp.out_acc[row * dv + d] = live ? acc : 0.0f;
    if (d == 0) {
      sp.out_m[row] = live ? m * kLn2 : -INFINITY;
      sp.out_l[row] = live ? L : 0.0f;
    }
  }
}

// Folds the nc partials of the hpk query rows of group (b, g) and carry_in by
// log-sum-exp merge, then writes out and carry_out.  `lds` holds 2 * hpk
// floats.
__device__ __forceinline__ void fold_group(const PartitionArgs &a,
                                           const StepParams &sp, int b, int g,
                                           int nc, float *lds) {
  const int Hq = a.num_kv_heads * a.hpk;
  const size_t row0 = (size_t)b * Hq + (size_t)g * a.hpk;
  stage_carry_in(sp, row0, a.hpk, lds);
  __syncthreads();  // carry_in m/l are read before carry_out may overwrite them
  for (int e = threadIdx.x; e < a.hpk * a.dv; e += blockDim.x) {
    const int h = e / a.dv, d = e % a.dv;
    const size_t row = row0 + h;
    const float *pm = a.part_m + row * a.total_cols;
    const float *pl = a.part_l + row * a.total_cols;
    const float *pa = a.part_acc + row * a.total_cols * a.dv + d;
    float m = lds[h], L = 0.0f, acc = 0.0f;
    if (lds[a.hpk + h] > 0.0f) {
      L = lds[a.hpk + h];
      acc = sp.in_acc[row * a.dv + d];
    }
#pragma unroll 4
    for (int i = 0; i < nc; ++i) {
      const float mi = coherent_load(pm + i) * kLog2e;
      const float mn = fmaxf(m, mi), ref = exp_ref(mn);
      const float fo = fast_exp2(m - ref), fi = fast_exp2(mi - ref);
      acc = acc * fo + coherent_load(pa + (size_t)i * a.dv) * fi;
      L = L * fo + coherent_load(pl + i) * fi;
      m = mn;
    }
    write_final(sp, row, a.dv, d, m, L, acc);
  }
}

}  // namespace gqa
