// Split-K partition kernels for fp32 caches.
//
// Matrix-core family (head widths 64/64, 128/128, 192/128, 256/256): the same
// structure as the bf16 kernel, on the exact-fp32 MFMA 16x16x4.  A wavefront
// takes 16-token tiles (the bytes of a 32-token bf16 tile), stages K and V once
// per KV group in its own LDS slice, forms S^T[token][head] = K . q^T for all
// heads of the group at once, updates every head's maximum logit, sum of
// exponentials and value accumulator with the tile (usearch attend), and accumulates
// acc^T[dv][head] += V^T . P^T with P straight from the S^T registers.
//
// Vector-ALU family (any other head widths that are multiples of 4, up to
// 256): one wavefront per work-group, lane t scores token t of a 64-token tile
// against every head, then owns value columns t, t+64, ... for the P.V sum.
// Both read each K/V row of a KV group once and share it among the group's
// query heads (needle-core attn.rs: each KV head serves its query heads by
// broadcast).
#include "device_common.h"
#include "gather_common.h"
#include "launch.h"
#include "step_common.h"

namespace gqa {
namespace {

// ---- matrix-core family ---------------------------------------------------

constexpr int kF32Tile = 16;  // tokens per wavefront tile

template <int DK, int DV>
struct F32Geom {
  static_assert(DK % 16 == 0 && DV % 16 == 0, "head widths");
  static constexpr int kPieces = DK / 4;  // 16-byte pieces per K row
  static constexpr int vPieces = DV / 4;
  static constexpr int kLoads = kF32Tile * kPieces / 64;  // per lane
  static constexpr int vLoads = kF32Tile * vPieces / 64;
  static_assert(kF32Tile * kPieces % 64 == 0, "K tile split");
  static_assert(kF32Tile * vPieces % 64 == 0, "V tile split");
  static constexpr int kStride = DK + 4;  // LDS row stride in floats
  static constexpr int vStride = DV + 4;
  static constexpr int waveLdsFloats = kF32Tile * (kStride + vStride);
};

template <int DK, int DV, int NW, bool STEP, bool BIAS, bool GATHER>
__global__ __launch_bounds__(NW * 64) void partition_f32_mfma_kernel(
    PartitionArgs args, StepParams sp) {
  using G = F32Geom<DK, DV>;
  constexpr int kMergeFloats = NW * 16 * (DV + 2);
  constexpr int kTileFloats = NW * G::waveLdsFloats;
  constexpr int kLdsFloats = kTileFloats > kMergeFloats ? kTileFloats : kMergeFloats;
  __shared__ __attribute__((aligned(16))) float lds[kLdsFloats];
  __shared__ int s_flag;
  __shared__ float s_in[32];  // carry_in m, l of the group's rows (direct)
  __shared__ int s_slot[GATHER ? kGatherChunk : 1];  // gathered cache slots
  __shared__ int s_wave[2 * NW];  // the in-launch selection's prefix sums

  PartitionArgs a = args;
  int item, branch = 0;
  if (a.sched) {  // scheduled launch: the table entry, or nothing to do
    item = a.sched[blockIdx.x];
    if (item < 0) return;
  } else if (a.one_xcd) {
    // a small single-cache launch on one XCD: block i runs on XCD i % 8, so
    // only every eighth block works and the kernel's code is fetched into
    // one XCD's L2 instead of eight
    if (blockIdx.x % 8 != 0) return;
    item = blockIdx.x / 8;
  } else {
    // the block's branch (multi-branch launch: each branch owns a block
    // range starting at a multiple of 8), then its item within the branch
    item = blockIdx.x;
    branch = select_branch(a, item);
    const int nitems = a.batch * a.num_kv_heads * a.num_chunks;
    if (item >= nitems) return;  // padding up to the next branch
    item = xcd_local_item(item, nitems);
  }
  const int Hkv = a.num_kv_heads, hpk = a.hpk, nchunk = a.num_chunks;
  const int c = item % nchunk;
  const int bg = item / nchunk;
  const int g = bg % Hkv;
  const int b = bg / Hkv;
  // decode step: this branch takes the new token (the others attend as is)
  const bool stepping = STEP && branch == a.append_branch;
  const SeqLen sl = seq_len(a, sp, b, stepping);
  int n = sl.n;
  if (stepping && !a.sched && g == 0 && c == 0 && threadIdx.x == 0)
    step_bookkeeping(sp, b, sl);  // (a scheduled launch's schedule kernel does it)
  const int t0 = c * a.chunk_tokens;
  if (GATHER) {
    // the selection is attended as a cache of n keys, its t-th slot in
    // ascending order being token t; this chunk's slots go to s_slot (the
    // tile area is the selection's scratch until the tiles start)
    n = gather_select<NW * 64>(a.idx + (size_t)b * a.width, a.width,
                               clamp_len(a.lens[b], a.cache_len), t0,
                               a.chunk_tokens, s_slot,
                               reinterpret_cast<uint32_t *>(lds), kLdsFloats,
                               s_wave);
    if (g == 0 && c == 0 && threadIdx.x == 0) a.sel_count[b] = n;
  }
  if (t0 >= n && !(c == 0 && (sp.direct || (STEP && sp.fuse)))) return;
  const int t1 = min(t0 + a.chunk_tokens, n);
  const int ntiles = t1 > t0 ? (t1 - t0 + kF32Tile - 1) / kF32Tile : 0;

  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int hl = lane & 15;
  const int kg = lane >> 4;
  const int Hq = Hkv * hpk;

  // q as the B operand: for dim block blk and step j the lane holds
  // q[head hl][blk*16 + kg*4 + j]; K's A operand uses the same dims.
  // Padding columns (hl >= hpk) repeat the group's last head (never written).
  f32x4 qf[DK / 16];
  {
    const float *qrow = static_cast<const float *>(a.q) +
                        ((size_t)b * Hq + (size_t)g * hpk + min(hl, hpk - 1)) * DK;
#pragma unroll
    for (int blk = 0; blk < DK / 16; ++blk)
      qf[blk] = *reinterpret_cast<const f32x4 *>(qrow + blk * 16 + kg * 4);
  }

  float *Ks = lds + w * G::waveLdsFloats;
  float *Vs = Ks + kF32Tile * G::kStride;
  const size_t kTok = (size_t)Hkv * DK, vTok = (size_t)Hkv * DV;
  float *Kg = static_cast<float *>(const_cast<void *>(a.k)) +
              ((size_t)b * a.cache_len * Hkv + g) * DK;
  float *Vg = static_cast<float *>(const_cast<void *>(a.v)) +
              ((size_t)b * a.cache_len * Hkv + g) * DV;

  // STEP: the work-group whose chunk holds the new slot stores the token's
  // rows into the cache without waiting; this call reads them from
  // k_new/v_new in the one tile holding the slot (relative position `rel`,
  // the chunk's last live token).
  const float *knew = nullptr, *vnew = nullptr;
  int rel = -1;
  if (stepping && sl.fresh && sl.n_old / a.chunk_tokens == c) {
    rel = sl.n_old - t0;
    knew = static_cast<const float *>(sp.k_new) + ((size_t)b * Hkv + g) * DK;
    vnew = static_cast<const float *>(sp.v_new) + ((size_t)b * Hkv + g) * DV;
    store_group_row(reinterpret_cast<const u32x4 *>(knew),
                    reinterpret_cast<u32x4 *>(Kg + (size_t)sl.n_old * kTok), DK / 4,
                    reinterpret_cast<const u32x4 *>(vnew),
                    reinterpret_cast<u32x4 *>(Vg + (size_t)sl.n_old * vTok), DV / 4,
                    threadIdx.x, blockDim.x);
  }
  const int rel_tile = rel >= 0 ? rel / kF32Tile : -1;

  // Tokens past the chunk's last live token load that token again (finite,
  // masked to weight 0): no branches, and padding slots are never read.
  const int last = max(t1 - t0 - 1, 0);
  const __amdgpu_buffer_rsrc_t kview = buffer_view(
      Kg + (size_t)t0 * kTok, (uint32_t)(((size_t)last * kTok + DK) * 4));
  const __amdgpu_buffer_rsrc_t vview = buffer_view(
      Vg + (size_t)t0 * vTok, (uint32_t)(((size_t)last * vTok + DV) * 4));
  // Index-gathered: the chunk's cache slots are in s_slot; the views then
  // span the sequence's whole cache (slots are absolute)
  const __amdgpu_buffer_rsrc_t gkview = buffer_view(
      Kg, GATHER ? (uint32_t)(((size_t)(a.cache_len - 1) * kTok + DK) * 4) : 0u);
  const __amdgpu_buffer_rsrc_t gvview = buffer_view(
      Vg, GATHER ? (uint32_t)(((size_t)(a.cache_len - 1) * vTok + DV) * 4) : 0u);
  // additive bias of the chunk's live tokens (loads past the view return 0)
  const __amdgpu_buffer_rsrc_t bview =
      BIAS && a.bias ? buffer_view(a.bias + (size_t)b * a.bias_stride + t0,
                         (uint32_t)((t1 - t0) * 4))
           : buffer_view(nullptr, 0);
  u32x4 kr[G::kLoads], vr[G::vLoads];
  f32x4 br;  // bias of tokens kg*4 + i
  br = f32x4{0.f, 0.f, 0.f, 0.f};
  auto issue = [&](int tile) {
    if (BIAS) br = load4f(bview, (uint32_t)((tile * kF32Tile + kg * 4) * 4));
    if (STEP && tile == rel_tile) {
      const float *kb = Kg + (size_t)t0 * kTok, *vb = Vg + (size_t)t0 * vTok;
#pragma unroll
      for (int i = 0; i < G::kLoads; ++i) {
        const int idx = i * 64 + lane;
        const int t = min(tile * kF32Tile + idx / G::kPieces, last);
        const int pc = (idx % G::kPieces) * 4;
        kr[i] = stream_load16(t == rel ? knew + pc : kb + (size_t)t * kTok + pc);
      }
#pragma unroll
      for (int i = 0; i < G::vLoads; ++i) {
        const int idx = i * 64 + lane;
        const int t = min(tile * kF32Tile + idx / G::vPieces, last);
        const int pc = (idx % G::vPieces) * 4;
        vr[i] = stream_load16(t == rel ? vnew + pc : vb + (size_t)t * vTok + pc);
      }
      return;
    }
    if (GATHER) {
#pragma unroll
      for (int i = 0; i < G::kLoads; ++i) {
        const int idx = i * 64 + lane;
        const int s = s_slot[min(tile * kF32Tile + idx / G::kPieces, last)];
        kr[i] = stream_load16(gkview, (uint32_t)((s * kTok + (idx % G::kPieces) * 4) * 4));
      }
#pragma unroll
      for (int i = 0; i < G::vLoads; ++i) {
        const int idx = i * 64 + lane;
        const int s = s_slot[min(tile * kF32Tile + idx / G::vPieces, last)];
        vr[i] = stream_load16(gvview, (uint32_t)((s * vTok + (idx % G::vPieces) * 4) * 4));
      }
      return;
    }
#pragma unroll
    for (int i = 0; i < G::kLoads; ++i) {
      const int idx = i * 64 + lane;
      const int t = min(tile * kF32Tile + idx / G::kPieces, last);
      kr[i] = stream_load16(kview, (uint32_t)((t * kTok + (idx % G::kPieces) * 4) * 4));
    }
#pragma unroll
    for (int i = 0; i < G::vLoads; ++i) {
      const int idx = i * 64 + lane;
      const int t = min(tile * kF32Tile + idx / G::vPieces, last);
      vr[i] = stream_load16(vview, (uint32_t)((t * vTok + (idx % G::vPieces) * 4) * 4));
    }
  };

  float m_run = -INFINITY, l_run = 0.0f;
  f32x4 o[DV / 16];
#pragma unroll
  for (int blk = 0; blk < DV / 16; ++blk) o[blk] = f32x4{0.f, 0.f, 0.f, 0.f};

  int tile = w;
  if (tile < ntiles) issue(tile);
  for (; tile < ntiles; tile += NW) {
    const int tb = t0 + tile * kF32Tile;
    wave_lds_sync();
#pragma unroll
    for (int i = 0; i < G::kLoads; ++i) {
      const int idx = i * 64 + lane;
      const int pc = idx % G::kPieces;
      *reinterpret_cast<u32x4 *>(Ks + (idx / G::kPieces) * G::kStride + pc * 4) = kr[i];
    }
#pragma unroll
    for (int i = 0; i < G::vLoads; ++i) {
      const int idx = i * 64 + lane;
      const int pc = idx % G::vPieces;
      *reinterpret_cast<u32x4 *>(Vs + (idx / G::vPieces) * G::vStride + pc * 4) = vr[i];
    }
    const f32x4 bcur = br;
    if (tile + NW < ntiles) issue(tile + NW);
    wave_lds_sync();

    // S^T[token kg*4 + i][head hl]
    f32x4 sacc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int blk = 0; blk < DK / 16; ++blk) {
      const f32x4 av =
          *reinterpret_cast<const f32x4 *>(Ks + hl * G::kStride + blk * 16 + kg * 4);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        sacc = __builtin_amdgcn_mfma_f32_16x16x4f32(av[j], qf[blk][j], sacc, 0, 0, 0);
    }

    float x[4];
    float mt = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float v = sacc[i] * a.scale_log2;
      if (BIAS) v += bcur[i] * kLog2e;
      x[i] = (tb + kg * 4 + i < t1) ? v : -INFINITY;
      mt = fmaxf(mt, x[i]);
    }
    mt = fmaxf(mt, __shfl_xor(mt, 16, 64));
    mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
    const float m_new = fmaxf(m_run, mt);
    const float ref = exp_ref(m_new);  // -inf only while every key is removed
    const float alpha = fast_exp2(m_run - ref);
    m_run = m_new;
    float p[4], psum = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      p[i] = fast_exp2(x[i] - ref);
      psum += p[i];
    }
    l_run = l_run * alpha + psum;

    // acc^T += V^T P^T, one token per MFMA step: A = V[kg*4 + i][blk*16 + hl]
#pragma unroll
    for (int blk = 0; blk < DV / 16; ++blk) {
      o[blk] *= alpha;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        o[blk] = __builtin_amdgcn_mfma_f32_16x16x4f32(
            Vs[(kg * 4 + i) * G::vStride + blk * 16 + hl], p[i], o[blk], 0, 0, 0);
    }
  }

  float l_tot = l_run + __shfl_xor(l_run, 16, 64);
  l_tot += __shfl_xor(l_tot, 32, 64);

  __syncthreads();
  float *wm = lds;
  float *wl = wm + NW * 16;
  float *wacc = wl + NW * 16;
  if (ntiles > 0) {
    if (lane < 16) {
      wm[w * 16 + lane] = m_run;
      wl[w * 16 + lane] = l_tot;
    }
#pragma unroll
    for (int blk = 0; blk < DV / 16; ++blk)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        wacc[(w * 16 + hl) * DV + blk * 16 + kg * 4 + i] = o[blk][i];
  }
  if (sp.direct) stage_carry_in(sp, (size_t)b * Hq + (size_t)g * hpk, hpk, s_in);
  __syncthreads();

  if (ntiles > 0 || sp.direct) {
    for (int e = threadIdx.x; e < hpk * DV; e += NW * 64) {
      const int h = e / DV, d = e % DV;
      float M = -INFINITY, acc = 0.0f, L = 0.0f;
      if (ntiles > 0) {
#pragma unroll
        for (int ww = 0; ww < NW; ++ww) M = fmaxf(M, wm[ww * 16 + h]);
        const float ref = exp_ref(M);
#pragma unroll
        for (int ww = 0; ww < NW; ++ww) {
          const float f = fast_exp2(wm[ww * 16 + h] - ref);
          acc += f * wacc[(ww * 16 + h) * DV + d];
          L += f * wl[ww * 16 + h];
        }
      }
      const size_t row = (size_t)b * Hq + (size_t)g * hpk + h;
      if (sp.direct) {  // the only chunk: fold carry_in, write the results
        const float l_in = s_in[hpk + h];
        fold_state(M, L, acc, s_in[h], l_in,
                   l_in > 0.0f ? sp.in_acc[row * DV + d] : 0.0f);
        write_final(sp, row, DV, d, M, L, acc);
        continue;
      }
      const size_t col = row * a.total_cols + a.col_base + c;
      float *pa = a.part_acc + col * DV + d;
      float *pm = a.part_m + col;
      float *pl = a.part_l + col;
      if (STEP && sp.fuse) {  // read back by this launch's last work-group
        coherent_store(pa, acc);
        if (d == 0) {
          coherent_store(pm, M * kLn2);
          coherent_store(pl, L);
        }
      } else {
        *pa = acc;
        if (d == 0) {
          *pm = M * kLn2;
          *pl = L;
        }
      }
    }
  }

  if (STEP && sp.fuse) {
    const int nc = (n + a.chunk_tokens - 1) / a.chunk_tokens;
    const bool last = nc == 0 || arrive_last(sp.counters + (size_t)b * Hkv + g,
                                             nc, &s_flag);
    if (last) {
      __syncthreads();
      fold_group(a, sp, b, g, nc, lds);
    }
  }
}

// Launches of at most this many work-groups run on one XCD (one_xcd).
constexpr int kOneXcdItems = 32;

template <int DK, int DV, bool STEP>
hipError_t launch_mfma(const PartitionArgs &args, const StepParams &sp,
                       hipStream_t s) {
  PartitionArgs a = args;
  a.one_xcd = !a.sched && a.num_extra == 0 && a.total_items <= kOneXcdItems;
  const int nwork = a.sched ? a.sched_len : a.one_xcd ? 8 * a.total_items
                                                      : a.total_items;
  if (a.idx) {  // index-gathered: attend only, no bias, never scheduled
    if (STEP || a.has_bias || a.sched) return hipErrorInvalidValue;
    hipLaunchKernelGGL(
        (partition_f32_mfma_kernel<DK, DV, kPartitionWaves, false, false, true>),
        dim3(nwork), dim3(kPartitionWaves * 64), 0, s, a, sp);
  } else if (a.has_bias) {
    hipLaunchKernelGGL(
        (partition_f32_mfma_kernel<DK, DV, kPartitionWaves, STEP, true, false>),
        dim3(nwork), dim3(kPartitionWaves * 64), 0, s, a, sp);
  } else {
    hipLaunchKernelGGL(
        (partition_f32_mfma_kernel<DK, DV, kPartitionWaves, STEP, false, false>),
        dim3(nwork), dim3(kPartitionWaves * 64), 0, s, a, sp);
  }
  return hipGetLastError();
}

template <bool STEP>
hipError_t dispatch_mfma(const PartitionArgs &a, const StepParams &sp,
                         hipStream_t s) {
  if (a.dk == 64 && a.dv == 64) return launch_mfma<64, 64, STEP>(a, sp, s);
  if (a.dk == 128 && a.dv == 128) return launch_mfma<128, 128, STEP>(a, sp, s);
  if (a.dk == 192 && a.dv == 128) return launch_mfma<192, 128, STEP>(a, sp, s);
  if (a.dk == 256 && a.dv == 256) return launch_mfma<256, 256, STEP>(a, sp, s);
  return hipErrorInvalidValue;
}

bool mfma_shape(int dk, int dv) {
  return (dk == 64 && dv == 64) || (dk == 128 && dv == 128) ||
         (dk == 192 && dv == 128) || (dk == 256 && dv == 256);
}

// ---- vector-ALU family ----------------------------------------------------

constexpr int kTok = 64;       // tokens per tile (one per lane)
constexpr int kMaxHeads = 16;  // heads per KV group
constexpr int kMaxCols = 4;    // value columns per lane (dv <= 256)

constexpr int kBatch = 16;     // 16-byte loads in flight per lane

// Stages tokens [tb, tb + kTok) of one group (row stride `gstride` floats,
// width d) into LDS rows of `lstride` floats; tokens at or past t1 read as 0.
// Loads are issued kBatch at a time before any of them is stored.
__device__ __forceinline__ void load_tile(const float *src, size_t gstride,
                                          int d, int tb, int t1, int lane,
                                          float *dst, int lstride,
                                          bool vec_store) {
  const int d4 = d >> 2;
  const int total = kTok * d4;
  for (int e0 = 0; e0 < total; e0 += kBatch * 64) {
    float4 x[kBatch];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const int e = e0 + j * 64 + lane;
      const int tok = e / d4, col = (e % d4) * 4;
      x[j] = (e < total && tb + tok < t1)
                 ? *reinterpret_cast<const float4 *>(src + (tb + tok) * gstride + col)
                 : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const int e = e0 + j * 64 + lane;
      if (e < total) {
        const int tok = e / d4, col = (e % d4) * 4;
        float *p = dst + tok * lstride + col;
        if (vec_store) {
          *reinterpret_cast<float4 *>(p) = x[j];
        } else {
          p[0] = x[j].x; p[1] = x[j].y; p[2] = x[j].z; p[3] = x[j].w;
        }
      }
    }
  }
}

__global__ __launch_bounds__(64) void partition_f32_kernel(
    const float *__restrict__ q, const float *__restrict__ K,
    const float *__restrict__ V, const int32_t *__restrict__ lens, int batch,
    int max_len, int Hkv, int hpk, int dk, int dv, int chunk, int nchunk,
    float scale_log2, const float *__restrict__ bias, long long bias_stride,
    float *__restrict__ part_m, float *__restrict__ part_l,
    float *__restrict__ part_acc) {
  extern __shared__ __attribute__((aligned(16))) float smem[];
  const int ks = dk + 1;           // odd stride: column reads hit 64 banks
  float *Ks = smem;                // [kTok][dk + 1]
  float *Vs = Ks + kTok * ks;      // [kTok][dv]
  float *Ps = Vs + kTok * dv;      // [hpk][kTok]
  float *Qs = Ps + hpk * kTok;     // [hpk][dk]

  const int item = xcd_local_item(blockIdx.x, batch * Hkv * nchunk);
  const int c = item % nchunk;
  const int bg = item / nchunk;
  const int g = bg % Hkv;
  const int b = bg / Hkv;
  const int n = clamp_len(lens[b], max_len);
  const int t0 = c * chunk;
  if (t0 >= n) return;
  const int t1 = min(t0 + chunk, n);
  const int lane = threadIdx.x;
  const int Hq = Hkv * hpk;

  const float *qg = q + ((size_t)b * Hq + (size_t)g * hpk) * dk;
  for (int e = lane; e < hpk * dk; e += 64) Qs[e] = qg[e];

  const size_t kT = (size_t)Hkv * dk, vT = (size_t)Hkv * dv;
  const float *Kg = K + ((size_t)b * max_len * Hkv + g) * dk;
  const float *Vg = V + ((size_t)b * max_len * Hkv + g) * dv;

  float m[kMaxHeads], l[kMaxHeads], acc[kMaxHeads][kMaxCols];
#pragma unroll
  for (int h = 0; h < kMaxHeads; ++h) {
    m[h] = -INFINITY;
    l[h] = 0.0f;
#pragma unroll
    for (int k = 0; k < kMaxCols; ++k) acc[h][k] = 0.0f;
  }

  for (int tb = t0; tb < t1; tb += kTok) {
    wave_lds_sync();
    load_tile(Kg, kT, dk, tb, t1, lane, Ks, ks, false);
    load_tile(Vg, vT, dv, tb, t1, lane, Vs, dv, true);
    wave_lds_sync();

    float s[kMaxHeads];
#pragma unroll
    for (int h = 0; h < kMaxHeads; ++h) s[h] = 0.0f;
    for (int cc = 0; cc < dk; ++cc) {
      const float kv = Ks[lane * ks + cc];
#pragma unroll
      for (int h = 0; h < kMaxHeads; ++h)
        if (h < hpk) s[h] = fmaf(Qs[h * dk + cc], kv, s[h]);
    }
    const bool live = tb + lane < t1;
    const float bl =
        (live && bias) ? bias[(size_t)b * bias_stride + tb + lane] * kLog2e : 0.0f;
#pragma unroll
    for (int h = 0; h < kMaxHeads; ++h) {
      if (h < hpk) {
        const float x = live ? s[h] * scale_log2 + bl : -INFINITY;
        const float m_new = fmaxf(m[h], wave_max(x));
        const float ref = exp_ref(m_new);
        const float alpha = fast_exp2(m[h] - ref);
        const float p = fast_exp2(x - ref);
        l[h] = l[h] * alpha + wave_sum(p);
        m[h] = m_new;
        Ps[h * kTok + lane] = p;
#pragma unroll
        for (int k = 0; k < kMaxCols; ++k) acc[h][k] *= alpha;
      }
    }
    wave_lds_sync();
    for (int t = 0; t < kTok; ++t) {
#pragma unroll
      for (int k = 0; k < kMaxCols; ++k) {
        const int col = lane + 64 * k;
        if (col < dv) {
          const float vv = Vs[t * dv + col];
#pragma unroll
          for (int h = 0; h < kMaxHeads; ++h)
            if (h < hpk) acc[h][k] = fmaf(Ps[h * kTok + t], vv, acc[h][k]);
        }
      }
    }
  }

#pragma unroll
  for (int h = 0; h < kMaxHeads; ++h) {
    if (h < hpk) {
      const size_t row = (size_t)b * Hq + (size_t)g * hpk + h;
#pragma unroll
      for (int k = 0; k < kMaxCols; ++k) {
        const int col = lane + 64 * k;
        if (col < dv) part_acc[(row * nchunk + c) * dv + col] = acc[h][k];
      }
      if (lane == 0) {
        part_m[row * nchunk + c] = m[h] * kLn2;
        part_l[row * nchunk + c] = l[h];
      }
    }
  }
}

}  // namespace

size_t partition_f32_lds_bytes(int dk, int dv, int hpk) {
  return sizeof(float) *
         ((size_t)kTok * (dk + 1) + (size_t)kTok * dv + (size_t)hpk * kTok +
          (size_t)hpk * dk);
}

// LDS of one gfx950 work-group.
constexpr size_t kMaxLds = 160 * 1024;

// Shapes with a kernel: the matrix-core shapes (1..16 heads per KV head),
// or a vector-ALU tile that fits the LDS of a work-group.
bool partition_f32_supported(int dk, int dv, int hpk) {
  if (hpk < 1 || hpk > kMaxHeads) return false;
  if (mfma_shape(dk, dv)) return true;
  return dk >= 4 && dk <= 256 && dk % 4 == 0 && dv >= 4 &&
         dv <= 64 * kMaxCols && dv % 4 == 0 &&
         partition_f32_lds_bytes(dk, dv, hpk) <= kMaxLds;
}

bool partition_f32_uses_mfma(int dk, int dv) { return mfma_shape(dk, dv); }

hipError_t launch_partition_f32(const PartitionArgs &a, const StepParams &ep,
                                hipStream_t s) {
  if (mfma_shape(a.dk, a.dv)) return dispatch_mfma<false>(a, ep, s);
  if (ep.direct || ep.fuse || a.sched || a.idx) return hipErrorInvalidValue;
  const int nwork = a.batch * a.num_kv_heads * a.num_chunks;
  const size_t lds = partition_f32_lds_bytes(a.dk, a.dv, a.hpk);
  if (lds > 65536) {
    const hipError_t e = hipFuncSetAttribute(
        reinterpret_cast<const void *>(partition_f32_kernel),
        hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(partition_f32_kernel, dim3(nwork), dim3(64), lds, s,
                     static_cast<const float *>(a.q),
                     static_cast<const float *>(a.k),
                     static_cast<const float *>(a.v), a.lens, a.batch,
                     a.max_len, a.num_kv_heads, a.hpk, a.dk, a.dv,
                     a.chunk_tokens, a.num_chunks, a.scale_log2, a.bias,
                     a.bias_stride, a.part_m,
                     a.part_l, a.part_acc);
  return hipGetLastError();
}

hipError_t launch_step_f32(const PartitionArgs &a, const StepParams &sp,
                           hipStream_t s) {
  if (!mfma_shape(a.dk, a.dv)) return hipErrorInvalidValue;
  return dispatch_mfma<true>(a, sp, s);
}

}  // namespace gqa
