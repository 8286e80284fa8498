// Split-K partition kernel for bf16 and fp8 (E4M3) caches on gfx950
// (MFMA 16x16x32 bf16).  Template body shared by partition_bf16.hip and
// partition_fp8.hip, each instantiating one storage type.
//
// One work-group handles one (sequence b, KV group g, chunk c) and all
// heads_per_kv query heads of the group.  Every K/V row of the chunk is read
// from HBM once, with 16-byte coalesced nontemporal loads, staged in the
// wavefront's own LDS slice, and shared by all heads of the group through the
// MFMA N dimension (needle-core attn.rs module doc: a KV head serves several
// query heads directly, without copying its K/V per head; cortiq-engine
// NystromState: the rows of a group are identical for all its heads, so they
// are held once per group).
//
// Per 32-token tile a wavefront computes
//   S^T[token][head] = K_tile[token][:] . q[head][:]         (MFMA, A = K)
// then folds the tile into the per-head state: maximum logit m, partition l and
// weighted value sum acc (usearch attend: each scored key updates these three
// per-head quantities), in base-2 units:
//   m' = max(m, max_j s_j), alpha = 2^(m - m'), p_j = 2^(s_j - m'),
//   l = alpha l + sum_j p_j,  acc = alpha acc + sum_j p_j V_j
// with acc^T[dv][head] += V_tile^T[dv][token] . P^T[token][head] on MFMA.
// The S^T accumulator layout (lane = head column, 4 consecutive tokens per
// lane group) is exactly the B-operand layout the P.V product needs, so P never
// leaves registers.  P is split as p = hi + lo with hi, lo bf16 so that the
// product keeps ~16 bits of each weight (two MFMAs instead of one; the matrix
// cores are far from busy on this HBM-bound loop).
//
// Heads are padded to 16 (the MFMA N width); padded columns repeat the
// group's last head and are never written.  Token offsets of a tile past the
// chunk's last live token are clamped to that token and their logits masked
// to -inf, so slots at or past the length are never read.
//
// In STEP mode the same launch is a whole decode step (needle-core
// self_attn_incremental: push_kv, then attend over the cache including the new
// token).  The work-group whose chunk holds the new slot stores the token's
// rows into the cache without waiting for the stores; its tile loop reads only
// the cache tokens before the slot, and its first wavefront folds the new
// token in from k_new/v_new afterwards, so the append never stalls the stream
// and the tile loop carries no special case.  The group's partials are folded
// by the last work-group to finish when `fuse` is set.
//
// With fp8 storage (FP8) a 16-byte load brings sixteen codes, which go to
// LDS as they are (half the LDS bytes); each MFMA operand is decoded to bf16
// as it is read (exact: every E4M3 value is a bf16 value), the V operand
// with one byte-transpose load per block.  The group's K scale multiplies
// the logit scale and its V scale the weighted value sum; a decode step
// quantises the new token's rows with the same scales.
#pragma once

#include "device_common.h"
#include "fp8_common.h"
#include "gather_common.h"
#include "launch.h"
#include "step_common.h"

namespace gqa {
namespace {

constexpr int kTileTokens = 32;

template <int DK, int DV, bool FP8>
struct Mfma16Geom {
  static_assert(DK % 32 == 0 && DV % 32 == 0, "head widths");
  static constexpr int kEsize = FP8 ? 1 : 2;       // bytes per stored element
  static constexpr int kPerPiece = 16 / kEsize;    // elements per 16-byte load
  static constexpr int kPieces = DK / kPerPiece;   // 16-byte pieces per K row
  static constexpr int vPieces = DV / kPerPiece;
  static constexpr int kLoads = kTileTokens * kPieces / 64;  // per lane
  static constexpr int vLoads = kTileTokens * vPieces / 64;
  static_assert(kTileTokens * kPieces % 64 == 0, "K tile split");
  static_assert(kTileTokens * vPieces % 64 == 0, "V tile split");
  // LDS rows: bf16 values for bf16 storage (stride in elements, +16 B pad);
  // the codes themselves for fp8 storage (+16 B pad), decoded when read.
  static constexpr int kStride = DK + 8;
  static constexpr int vStride = DV + 8;
  static constexpr int kRowBytes = FP8 ? DK + 16 : kStride * 2;
  static constexpr int vRowBytes = FP8 ? DV + 16 : vStride * 2;
  static constexpr int waveLdsBytes = kTileTokens * (kRowBytes + vRowBytes);
};

// The work-group's main LDS area: the wavefronts' tile slices, reused for the
// merge of their states (NW * 16 rows of dv + 2 floats).
template <int DK, int DV, int NW, bool FP8>
constexpr int partition_lds_bytes() {
  constexpr int tiles = NW * Mfma16Geom<DK, DV, FP8>::waveLdsBytes;
  constexpr int merge = NW * 16 * (DV + 2) * 4;
  return tiles > merge ? tiles : merge;
}

// One segment of one (sequence b, KV group g): cache tokens [t0, t1) streamed
// tile by tile by the work-group's wavefronts (wavefront w takes tiles w,
// w + NW, ...), plus, when `has_new`, the decode step's new token (stored
// into slot n_old and folded in from k_new / v_new).  Every wavefront's state
// (base-2 m, partition, acc^T) is left in the LDS merge area for the
// epilogue (`merged_state`), after a work-group barrier; with `stage_in` the
// group's carry_in m / l are staged in s_in before that barrier.  Returns
// whether the segment saw any key.  Index-gathered (GATHER): token t0 + e of
// the segment is cache slot s_slot[e].  Group split (SPLIT): wavefront w
// takes KV group g + w and every tile of the segment, so its state is that
// group's alone (no stage_in).
template <int DK, int DV, int NW, bool STEP, bool BIAS, bool GATHER, bool FP8,
          bool SPLIT = false>
__device__ __forceinline__ bool stream_segment(const PartitionArgs &a,
                                               const StepParams &sp, int b,
                                               int g, int t0, int t1,
                                               bool has_new, int n_old,
                                               bool stage_in,
                                               unsigned char *lds,
                                               int *s_slot, float *s_in) {
  using G = Mfma16Geom<DK, DV, FP8>;
  constexpr int ES = G::kEsize;
  const int Hkv = a.num_kv_heads, hpk = a.hpk;
  const int ntiles = t1 > t0 ? (t1 - t0 + kTileTokens - 1) / kTileTokens : 0;

  const int lane = threadIdx.x & 63;
  // the wavefront's index, known to the compiler as uniform across its lanes
  // (the tile loop is then scalar)
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int hl = lane & 15;  // head column of this lane
  const int kg = lane >> 4;  // lane group: k-slice of MFMA operands
  const int Hq = Hkv * hpk;
  const int gw = SPLIT ? g + w : g;  // this wavefront's KV group

  // q as the B operand of S^T = K q^T: lane holds head hl, dims s*32+kg*8..+8.
  // Padding columns (hl >= hpk) repeat the group's last head; they are never
  // written, and loading them unconditionally keeps the load off the critical
  // path (no partial-lane write to wait for).
  bf16x8 qf[DK / 32];
  {
    const uint16_t *qrow = static_cast<const uint16_t *>(a.q) +
                           ((size_t)b * Hq + (size_t)gw * hpk + min(hl, hpk - 1)) * DK;
#pragma unroll
    for (int s = 0; s < DK / 32; ++s)
      qf[s] = *reinterpret_cast<const bf16x8 *>(qrow + s * 32 + kg * 8);
  }

  unsigned char *Ks8 = lds + w * G::waveLdsBytes;  // this wavefront's tiles
  unsigned char *Vs8 = Ks8 + kTileTokens * G::kRowBytes;
  uint16_t *Ks = reinterpret_cast<uint16_t *>(Ks8);  // bf16 storage
  uint16_t *Vs = reinterpret_cast<uint16_t *>(Vs8);
  // this lane's fetch address for the transpose loads of V (see below): bf16
  // lane u = lane % 16 of group kg fetches V[kg*4 + u/4][4(u%4) ..+4]; fp8
  // lane u fetches codes V[token(kg, u/2)][8(u%2) ..+8]
  const uint16_t *vsrc = Vs + (kg * 4 + (lane & 15) / 4) * G::vStride + 4 * (lane & 3);
  const int vk8 = (lane & 15) >> 1;
  const unsigned char *vsrc8 =
      Vs8 + (vk8 < 4 ? kg * 4 + vk8 : 16 + kg * 4 + (vk8 - 4)) * G::vRowBytes +
      8 * (lane & 1);

  const size_t kTok = (size_t)Hkv * DK * ES;  // bytes between tokens
  const size_t vTok = (size_t)Hkv * DV * ES;
  unsigned char *Kg = static_cast<unsigned char *>(const_cast<void *>(a.k)) +
                      ((size_t)b * a.cache_len * Hkv + gw) * DK * ES;
  unsigned char *Vg = static_cast<unsigned char *>(const_cast<void *>(a.v)) +
                      ((size_t)b * a.cache_len * Hkv + gw) * DV * ES;
  // fp8: the group's scales (K into the logit scale, V into acc at the end)
  const float kscale = FP8 ? a.k_scale[(size_t)b * Hkv + gw] : 1.0f;
  const float vscale = FP8 ? a.v_scale[(size_t)b * Hkv + gw] : 1.0f;
  const float scale_log2 = a.scale_log2 * kscale;
  // fp8 decode step: the new rows are multiplied by these before encoding
  const float kinv = FP8 && STEP ? e4m3_inv_scale(kscale) : 1.0f;
  const float vinv = FP8 && STEP ? e4m3_inv_scale(vscale) : 1.0f;

  // STEP: the work-group whose segment holds the new slot stores the token's
  // rows of this group (of each wavefront's group when split) into the cache.
  // The stores are not waited for: later calls read the slot, while this call
  // takes the rows from k_new/v_new.
  const uint16_t *knew = nullptr, *vnew = nullptr;
  if (STEP && has_new) {
    knew = static_cast<const uint16_t *>(sp.k_new) + ((size_t)b * Hkv + gw) * DK;
    vnew = static_cast<const uint16_t *>(sp.v_new) + ((size_t)b * Hkv + gw) * DV;
    const int first = SPLIT ? lane : (int)threadIdx.x;
    const int stride = SPLIT ? 64 : NW * 64;
    if (FP8)
      store_group_row_e4m3(knew, reinterpret_cast<u32x4 *>(Kg + (size_t)n_old * kTok),
                           DK / 16, kinv, vnew,
                           reinterpret_cast<u32x4 *>(Vg + (size_t)n_old * vTok),
                           DV / 16, vinv, first, stride);
    else
      store_group_row(reinterpret_cast<const u32x4 *>(knew),
                      reinterpret_cast<u32x4 *>(Kg + (size_t)n_old * kTok), DK / 8,
                      reinterpret_cast<const u32x4 *>(vnew),
                      reinterpret_cast<u32x4 *>(Vg + (size_t)n_old * vTok), DV / 8,
                      first, stride);
  }

  // K/V are read exactly once per call, so the loads are nontemporal: they
  // stream through without displacing cached lines.  Tokens of a tile past
  // the segment's last live token load that last token again (a finite row
  // whose logit is masked, so its weight is exactly 0): no branches, and no
  // slot at or past the length is ever read.
  const int last = max(t1 - t0 - 1, 0);  // last live token, relative to t0
  const __amdgpu_buffer_rsrc_t kview = buffer_view(
      Kg + (size_t)t0 * kTok, (uint32_t)((size_t)last * kTok + DK * ES));
  const __amdgpu_buffer_rsrc_t vview = buffer_view(
      Vg + (size_t)t0 * vTok, (uint32_t)((size_t)last * vTok + DV * ES));
  // Index-gathered: the chunk's cache slots are in s_slot (staged by the
  // caller); the views then span the sequence's whole cache (slots are
  // absolute)
  const __amdgpu_buffer_rsrc_t gkview = buffer_view(
      Kg, GATHER ? (uint32_t)((size_t)(a.cache_len - 1) * kTok + DK * ES) : 0u);
  const __amdgpu_buffer_rsrc_t gvview = buffer_view(
      Vg, GATHER ? (uint32_t)((size_t)(a.cache_len - 1) * vTok + DV * ES) : 0u);
  // The additive bias of the segment's live tokens (needle-core attn_bias:
  // one term per position, shared by the heads); loads past the view return 0.
  const __amdgpu_buffer_rsrc_t bview =
      BIAS && a.bias ? buffer_view(a.bias + (size_t)b * a.bias_stride + t0,
                         (uint32_t)((t1 - t0) * 4))
                     : buffer_view(nullptr, 0);
  u32x4 kr[G::kLoads], vr[G::vLoads];
  f32x4 br[2];  // bias of tokens rb*16 + kg*4 + i, i < 4
  br[0] = br[1] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto issue = [&](int tile) {
    if (BIAS) {
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
        br[rb] = load4f(bview, (uint32_t)((tile * kTileTokens + rb * 16 + kg * 4) * 4));
    }
    if (GATHER) {
#pragma unroll
      for (int i = 0; i < G::kLoads; ++i) {
        const int idx = i * 64 + lane;
        const int s = s_slot[min(tile * kTileTokens + idx / G::kPieces, last)];
        kr[i] = stream_load16(gkview, (uint32_t)(s * kTok + (idx % G::kPieces) * 16));
      }
#pragma unroll
      for (int i = 0; i < G::vLoads; ++i) {
        const int idx = i * 64 + lane;
        const int s = s_slot[min(tile * kTileTokens + idx / G::vPieces, last)];
        vr[i] = stream_load16(gvview, (uint32_t)(s * vTok + (idx % G::vPieces) * 16));
      }
      return;
    }
#pragma unroll
    for (int i = 0; i < G::kLoads; ++i) {
      const int idx = i * 64 + lane;
      const int t = min(tile * kTileTokens + idx / G::kPieces, last);
      kr[i] = stream_load16(kview, (uint32_t)(t * kTok + (idx % G::kPieces) * 16));
    }
#pragma unroll
    for (int i = 0; i < G::vLoads; ++i) {
      const int idx = i * 64 + lane;
      const int t = min(tile * kTileTokens + idx / G::vPieces, last);
      vr[i] = stream_load16(vview, (uint32_t)(t * vTok + (idx % G::vPieces) * 16));
    }
  };

  float m_run = -INFINITY;  // base-2 running max of head hl
  float l_run = 0.0f;       // this lane's share of the partition
  f32x4 o[DV / 16];         // acc^T: head hl, dv rows blk*16 + kg*4 + i
#pragma unroll
  for (int blk = 0; blk < DV / 16; ++blk) o[blk] = f32x4{0.f, 0.f, 0.f, 0.f};

  // wavefront w takes tiles w, w + NW, ... of the group, or all of them when
  // the wavefronts hold different groups
  constexpr int kStep = SPLIT ? 1 : NW;
  int tile = SPLIT ? 0 : w;
  if (tile < ntiles) issue(tile);
  for (; tile < ntiles; tile += kStep) {
    const int tb = t0 + tile * kTileTokens;
    wave_lds_sync();  // previous tile's LDS reads are done
#pragma unroll
    for (int i = 0; i < G::kLoads; ++i) {
      const int idx = i * 64 + lane;
      *reinterpret_cast<u32x4 *>(Ks8 + (idx / G::kPieces) * G::kRowBytes +
                                 (idx % G::kPieces) * 16) = kr[i];
    }
#pragma unroll
    for (int i = 0; i < G::vLoads; ++i) {
      const int idx = i * 64 + lane;
      *reinterpret_cast<u32x4 *>(Vs8 + (idx / G::vPieces) * G::vRowBytes +
                                 (idx % G::vPieces) * 16) = vr[i];
    }
    const f32x4 bcur[2] = {br[0], br[1]};
    if (tile + kStep < ntiles) issue(tile + kStep);  // next tile in flight meanwhile
    wave_lds_sync();

    // S^T for tokens rb*16 + kg*4 + i (i < 4), head hl
    f32x4 sacc[2];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      sacc[rb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < DK / 32; ++s) {
        bf16x8 av;
        if constexpr (FP8) {  // eight codes of token rb*16 + hl, decoded
          const uint2 c = *reinterpret_cast<const uint2 *>(
              Ks8 + (rb * 16 + hl) * G::kRowBytes + s * 32 + kg * 8);
          av = e4m3x8_to_bf16x8(c.x, c.y);
        } else {
          av = *reinterpret_cast<const bf16x8 *>(
              Ks + (rb * 16 + hl) * G::kStride + s * 32 + kg * 8);
        }
        sacc[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, qf[s], sacc[rb],
                                                           0, 0, 0);
      }
    }

    float x[8];
    float mt = -INFINITY;
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = tb + rb * 16 + kg * 4 + i;
        float v = sacc[rb][i] * scale_log2;
        if (BIAS) v += bcur[rb][i] * kLog2e;
        v = (t < t1) ? v : -INFINITY;
        x[rb * 4 + i] = v;
        mt = fmaxf(mt, v);
      }
    }
    mt = rows_max(mt);
    const float m_new = fmaxf(m_run, mt);
    const float ref = exp_ref(m_new);  // -inf only while every key is removed
    const float alpha = fast_exp2(m_run - ref);
    m_run = m_new;

    bf16x8 phi, plo;
    float psum = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float p = fast_exp2(x[j] - ref);
      psum += p;
      const __bf16 h = (__bf16)p;
      phi[j] = h;
      plo[j] = (__bf16)(p - (float)h);
    }
    l_run = l_run * alpha + psum;

    // acc^T += V^T P^T; the A operand holds V[token(kg, j)][blk*16 + hl]
    // with token(kg, j) = j < 4 ? kg*4 + j : 16 + kg*4 + (j - 4), the token
    // order of this lane's P values.  Two transpose loads bring it: lane
    // u = lane % 16 of group kg fetches V[kg*4 + u/4][blk*16 + 4(u%4) ..+4]
    // (and the same 16 tokens further), so that lane hl receives column
    // blk*16 + hl of tokens kg*4 + 0..3.
#pragma unroll
    for (int blk = 0; blk < DV / 16; ++blk) {
      bf16x8 av;
      if constexpr (FP8) {  // one byte-transpose load: all eight tokens
        const i32x2 c = lds_read_tr8(vsrc8 + blk * 16);
        av = e4m3x8_to_bf16x8(c.x, c.y);
      } else {
        const i16x4 lo = lds_read_tr16(vsrc + blk * 16);
        const i16x4 hi = lds_read_tr16(vsrc + 16 * G::vStride + blk * 16);
        av = __builtin_bit_cast(
            bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      }
      o[blk] *= alpha;
      o[blk] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, phi, o[blk], 0, 0, 0);
      o[blk] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, plo, o[blk], 0, 0, 0);
    }
  }

  // The new token of a decode step, folded into wavefront 0's state (every
  // wavefront's, for its own group, when split): its logit from q and k_new
  // (for fp8 caches, the decoded codes it is stored as), then the usual online
  // update with its value row.
  if (STEP && has_new && (SPLIT || w == 0)) {
    float dot = 0.0f;
#pragma unroll
    for (int s = 0; s < DK / 32; ++s) {
      const u32x4 raw = stream_load16(knew + s * 32 + kg * 8);
      bf16x8 kv;
      if constexpr (FP8) {
        const uint2 code = e4m3_quantize8(raw, kinv);
        kv = e4m3x8_to_bf16x8(code.x, code.y);
      } else {
        kv = __builtin_bit_cast(bf16x8, raw);
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) dot += (float)qf[s][j] * (float)kv[j];
    }
    float sn = rows_sum(dot) * scale_log2;
    if (BIAS && a.bias) sn += a.bias[(size_t)b * a.bias_stride + n_old] * kLog2e;
    const float m_new = fmaxf(m_run, sn);
    const float ref = exp_ref(m_new);
    const float alpha = fast_exp2(m_run - ref);
    const float p = fast_exp2(sn - ref);
    m_run = m_new;
    l_run = l_run * alpha + (kg == 0 ? p : 0.0f);  // once per head column
#pragma unroll
    for (int blk = 0; blk < DV / 16; ++blk) {
      // value rows blk*16 + kg*4 + i of this lane's acc^T entries
      const uint2 raw = *reinterpret_cast<const uint2 *>(vnew + blk * 16 + kg * 4);
      uint2 vb = raw;
      if constexpr (FP8) {
        vb = e4m3x4_to_bf16(e4m3_pack4(
            __uint_as_float(raw.x << 16) * vinv, __uint_as_float(raw.x & 0xFFFF0000u) * vinv,
            __uint_as_float(raw.y << 16) * vinv, __uint_as_float(raw.y & 0xFFFF0000u) * vinv));
      }
      const float vv[4] = {__uint_as_float(vb.x << 16), __uint_as_float(vb.x & 0xFFFF0000u),
                           __uint_as_float(vb.y << 16), __uint_as_float(vb.y & 0xFFFF0000u)};
#pragma unroll
      for (int i = 0; i < 4; ++i) o[blk][i] = o[blk][i] * alpha + p * vv[i];
    }
  }

  if (FP8) {
#pragma unroll
    for (int blk = 0; blk < DV / 16; ++blk) o[blk] *= vscale;
  }

  // Partition of head hl over the whole wavefront.
  const float l_tot = rows_sum(l_run);

  // Each wavefront's state into the merge area (the tile slices are free).
  __syncthreads();
  float *wm = reinterpret_cast<float *>(lds);
  float *wl = wm + NW * 16;
  float *wacc = wl + NW * 16;
  const bool live = ntiles > 0 || has_new;  // the segment saw keys
  if (live) {
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
  if (stage_in) stage_carry_in(sp, (size_t)b * Hq + (size_t)g * hpk, hpk, s_in);
  __syncthreads();
  return live;
}

// The work-group's merged state of head h, column d, from the wavefronts'
// states `stream_segment` left in the LDS merge area (m in base-2 units;
// -inf / 0 / 0 when the segment saw no key).
template <int DV, int NW>
__device__ __forceinline__ void merged_state(const unsigned char *lds, bool live,
                                             int h, int d, float &M, float &L,
                                             float &acc) {
  const float *wm = reinterpret_cast<const float *>(lds);
  const float *wl = wm + NW * 16;
  const float *wacc = wl + NW * 16;
  M = -INFINITY;
  acc = 0.0f;
  L = 0.0f;
  if (!live) return;
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

// Final results of a group whose keys one work-group saw in full: carry_in
// (staged in s_in) folded in, then out and carry_out.
template <int DV, int NW>
__device__ __forceinline__ void write_group_direct(const StepParams &sp,
                                                   size_t row0, int hpk,
                                                   bool live,
                                                   const unsigned char *lds,
                                                   const float *s_in) {
  for (int e = threadIdx.x; e < hpk * DV; e += NW * 64) {
    const int h = e / DV, d = e % DV;
    float M, L, acc;
    merged_state<DV, NW>(lds, live, h, d, M, L, acc);
    const size_t row = row0 + h;
    const float l_in = s_in[hpk + h];
    fold_state(M, L, acc, s_in[h], l_in,
               l_in > 0.0f ? sp.in_acc[row * DV + d] : 0.0f);
    write_final(sp, row, DV, d, M, L, acc);
  }
}

template <int DK, int DV, int NW, bool STEP, bool BIAS, bool GATHER, bool FP8>
__global__ __launch_bounds__(NW * 64) void partition_bf16_kernel(
    PartitionArgs args, StepParams sp) {
  constexpr int kLdsBytes = partition_lds_bytes<DK, DV, NW, FP8>();
  __shared__ __attribute__((aligned(16))) unsigned char lds[kLdsBytes];
  __shared__ int s_flag;
  __shared__ float s_in[32];  // carry_in m, l of the group's rows (direct)
  __shared__ int s_slot[GATHER ? kGatherChunk : 1];  // gathered cache slots
  __shared__ int s_wave[2 * NW];  // the in-launch selection's prefix sums

  PartitionArgs a = args;
  int item, branch = 0;
  if (!GATHER && a.sched) {  // scheduled launch: the table entry, or nothing to do
    item = a.sched[blockIdx.x];
    if (item < 0) return;
  } else {
    // the block's branch (multi-branch launch: each branch owns a block
    // range starting at a multiple of 8), then its item within the branch
    // (a gathered launch has one branch and no schedule)
    item = blockIdx.x;
    if (!GATHER) branch = select_branch(a, item);
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
                               reinterpret_cast<uint32_t *>(lds), kLdsBytes / 4,
                               s_wave);
    if (g == 0 && c == 0 && threadIdx.x == 0) a.sel_count[b] = n;
  }
  // A work-group with nothing live exits, except the first of an empty
  // sequence when final results are written in this launch: it still writes
  // the group's outputs.
  if (t0 >= n && !(c == 0 && (sp.direct || (STEP && sp.fuse)))) return;
  // Decode step: the work-group whose chunk holds the new slot (always the
  // chunk's last live token) reads only the cache tokens before it in its
  // tile loop and folds the new token in from k_new / v_new afterwards.
  const bool has_new = stepping && sl.fresh && sl.n_old / a.chunk_tokens == c;
  const int t1 = has_new ? sl.n_old : min(t0 + a.chunk_tokens, n);  // tiles: [t0, t1)

  const bool live = stream_segment<DK, DV, NW, STEP, BIAS, GATHER, FP8>(
      a, sp, b, g, t0, t1, has_new, sl.n_old, sp.direct != 0, lds, s_slot, s_in);

  const int Hq = Hkv * hpk;
  const size_t row0 = (size_t)b * Hq + (size_t)g * hpk;
  if (sp.direct) {  // the only chunk: fold carry_in, write the results
    write_group_direct<DV, NW>(sp, row0, hpk, live, lds, s_in);
  } else if (live) {  // one partial per (query row, chunk)
    for (int e = threadIdx.x; e < hpk * DV; e += NW * 64) {
      const int h = e / DV;
      const int d = e % DV;
      float M, L, acc;
      merged_state<DV, NW>(lds, live, h, d, M, L, acc);
      const size_t col = (row0 + h) * a.total_cols + a.col_base + c;
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
    // an empty sequence has no partials: its first work-group folds alone
    const bool last = nc == 0 || arrive_last(sp.counters + (size_t)b * Hkv + g,
                                             nc, &s_flag);
    if (last) {
      __syncthreads();  // the LDS merge area is reused below
      fold_group(a, sp, b, g, nc, reinterpret_cast<float *>(lds));
    }
  }
}

// Group-split chunked launch (fp8 caches with 64-wide heads, plain chunked
// plans: no schedule, queue, further branch or gathered index, and a combine
// launch after it; launch.h group_split).
// Work-group (b, q, c) holds the NW consecutive KV groups q NW .. q NW + NW - 1
// of sequence b over chunk c, and wavefront w streams group q NW + w over the
// whole chunk.  The KV heads of one token lie side by side in the cache, so
// the work-group's loads of a tile cover NW groups' rows of the same tokens at
// the same time, where NW work-groups would read them at different times
// (for E4M3 rows of 128 bytes at a 1 KiB token stride, the batched shape, a
// load-only probe read the cache in 22.0 us this way against 24.9 us).  Each
// wavefront's state is its group's partial for the chunk; nothing is merged.
template <int DK, int DV, int NW, bool STEP, bool BIAS, bool FP8>
__global__ __launch_bounds__(NW * 64) void partition_split_kernel(
    PartitionArgs a, StepParams sp) {
  constexpr int kLdsBytes = partition_lds_bytes<DK, DV, NW, FP8>();
  __shared__ __attribute__((aligned(16))) unsigned char lds[kLdsBytes];

  const int Hkv = a.num_kv_heads, hpk = a.hpk, nchunk = a.num_chunks;
  const int nq = Hkv / NW;  // work-groups per (sequence, chunk)
  const int nitems = a.batch * nq * nchunk;  // the grid (launch_one)
  if ((int)blockIdx.x >= nitems) return;
  const int item = xcd_local_item(blockIdx.x, nitems);
  const int c = item % nchunk;
  const int bq = item / nchunk;
  const int g = (bq % nq) * NW;  // the work-group's first KV group
  const int b = bq / nq;

  const SeqLen sl = seq_len(a, sp, b, STEP);
  const int n = sl.n;
  if (STEP && g == 0 && c == 0 && threadIdx.x == 0) step_bookkeeping(sp, b, sl);
  const int t0 = c * a.chunk_tokens;
  if (t0 >= n) return;  // the combine takes only live chunks
  // decode step: the chunk holding the new slot (the last live token) reads
  // the cache tokens before it and folds the new token in afterwards
  const bool has_new = STEP && sl.fresh && sl.n_old / a.chunk_tokens == c;
  const int t1 = has_new ? sl.n_old : min(t0 + a.chunk_tokens, n);
  stream_segment<DK, DV, NW, STEP, BIAS, false, FP8, true>(
      a, sp, b, g, t0, t1, has_new, sl.n_old, false, lds, nullptr, nullptr);

  // every wavefront's state, as stream_segment left it in the merge area, is
  // one partial: wavefront wv's head h is query row (g + wv) hpk + h
  const float *wm = reinterpret_cast<const float *>(lds);
  const float *wl = wm + NW * 16;
  const float *wacc = wl + NW * 16;
  const size_t row0 = (size_t)b * Hkv * hpk + (size_t)g * hpk;
  for (int e = threadIdx.x; e < NW * hpk * DV; e += NW * 64) {
    const int wh = e / DV;  // wv * hpk + h
    const int d = e - wh * DV;
    const int wv = wh / hpk, h = wh - wv * hpk;
    const size_t col = (row0 + wh) * a.total_cols + a.col_base + c;
    a.part_acc[col * DV + d] = wacc[(wv * 16 + h) * DV + d];
    if (d == 0) {
      a.part_m[col] = wm[wv * 16 + h] * kLn2;
      a.part_l[col] = wl[wv * 16 + h];
    }
  }
}

// Balanced launch (a plan with many items over several rounds of
// work-groups, where fixed chunks leave a ragged last round, and where the
// work-groups' read rates differ by tens of percent from one CU or XCD to
// another): a work queue.  The balance kernel cuts every sequence into runs
// of 32-token tiles in three phases of shrinking run length (kQueueRun0/1/2
// tiles) and lists them phase by phase, sequence by sequence; item i of the
// queue is run i / num_kv_heads for KV group i % num_kv_heads, so the groups
// of one run, which share its cache rows, are taken one after the other.
// a.balanced persistent work-groups take items from one counter until the
// queue is empty (the next index is fetched while the current item streams),
// so faster work-groups simply take more items and the last ones are short.
// Every item leaves its partial state in piece slot i; the balanced combine
// folds each query row's pieces.  A decode step's new token is stored and
// folded by the item whose run holds the sequence's last tile.
template <int DK, int DV, int NW, bool STEP, bool BIAS, bool FP8>
__global__ __launch_bounds__(NW * 64) void partition_balanced_kernel(
    PartitionArgs a, StepParams sp) {
  constexpr int kLdsBytes = partition_lds_bytes<DK, DV, NW, FP8>();
  __shared__ __attribute__((aligned(16))) unsigned char lds[kLdsBytes];
  __shared__ int s_item;

  const int Hkv = a.num_kv_heads, hpk = a.hpk;
  int *queue = a.queue;
  const int total = queue[kQueueItems];
  const int *runs = queue + queue_runs_offset(a.batch);
  if (threadIdx.x == 0) s_item = atomicAdd(queue + kQueueCounter, 1);
  __syncthreads();
  int item = s_item;
  while (item < total) {
    const int run = item / Hkv, g = item - run * Hkv;
    const int b = runs[3 * run], t0t = runs[3 * run + 1], t1t = runs[3 * run + 2];
    int next = 0;
    if (threadIdx.x == 0) next = atomicAdd(queue + kQueueCounter, 1);
    const SeqLen sl = seq_len(a, sp, b, STEP);
    const int n = sl.n;
    const int t0 = t0t * kTileTokens;
    const int tend = min(t1t * kTileTokens, n);
    // decode step: the run holding the sequence's last tile holds the slot
    const bool has_new = STEP && sl.fresh && tend == n;
    const int t1 = has_new ? sl.n_old : tend;
    const bool live = stream_segment<DK, DV, NW, STEP, BIAS, false, FP8>(
        a, sp, b, g, t0, t1, has_new, sl.n_old, false, lds, nullptr, nullptr);
    for (int e = threadIdx.x; e < hpk * DV; e += NW * 64) {
      const int h = e / DV, d = e % DV;
      float M, L, acc;
      merged_state<DV, NW>(lds, live, h, d, M, L, acc);
      const size_t pr = (size_t)item * hpk + h;  // piece row
      a.part_acc[pr * DV + d] = acc;
      if (d == 0) {
        a.part_m[pr] = M * kLn2;
        a.part_l[pr] = L;
      }
    }
    if (threadIdx.x == 0) s_item = next;
    __syncthreads();  // the next index is visible; the merge area is free
    item = s_item;
  }
}

// A scheduled launch runs its work-groups in several rounds.  There the read
// stream ran fastest with at most two work-groups resident per CU (ragged
// workload: 749 -> 738 us per launch against up to four by LDS; 771 us with
// one), so such a launch reserves unused dynamic LDS that keeps a third out
// of a CU's 160 KB.  The reservation is sized against the main LDS area
// alone, a lower bound of the static LDS, so three never fit; two always do
// (the total stays within 55 KB).
constexpr int kCuLdsBytes = 160 * 1024;

template <int DK, int DV, int NW, bool FP8>
int residency_lds_bytes(const PartitionArgs &a) {
  constexpr int kThird = kCuLdsBytes / 3 + 1;
  constexpr int kMain = partition_lds_bytes<DK, DV, NW, FP8>();
  return a.sched && kMain < kThird ? kThird - kMain : 0;
}

// A balanced launch has exactly kBalancedPerCu work-groups per CU, all
// resident at once: unused dynamic LDS keeps one more out of a CU, so the
// ranges spread evenly over the CUs.
constexpr int kBalancedPerCu = 2;

template <int DK, int DV, int NW, bool FP8>
constexpr int balanced_lds_bytes() {
  constexpr int kShare = kCuLdsBytes / (kBalancedPerCu + 1) + 1;
  constexpr int kMain = partition_lds_bytes<DK, DV, NW, FP8>();
  return kMain < kShare ? kShare - kMain : 0;
}

template <int DK, int DV, int NW, bool STEP, bool FP8>
hipError_t launch_one(const PartitionArgs &a, const StepParams &sp,
                      hipStream_t s) {
  if (a.balanced) {  // one resident work-group per range, two per CU
    if (a.idx || a.num_extra || a.sched || (sp.fuse && STEP) ||
        a.balanced % 8)
      return hipErrorInvalidValue;
    const int dyn = balanced_lds_bytes<DK, DV, NW, FP8>();
    if (a.has_bias)
      hipLaunchKernelGGL((partition_balanced_kernel<DK, DV, NW, STEP, true, FP8>),
                         dim3(a.balanced), dim3(NW * 64), dyn, s, a, sp);
    else
      hipLaunchKernelGGL((partition_balanced_kernel<DK, DV, NW, STEP, false, FP8>),
                         dim3(a.balanced), dim3(NW * 64), dyn, s, a, sp);
    return hipGetLastError();
  }
  if constexpr (FP8 && DK + DV <= 128) {
    constexpr int SW = split_waves(DK, DV);
    const int nwork = a.total_items / SW;
    if (group_split(DK, DV, FP8, a.num_kv_heads) == SW &&
        a.total_items == a.batch * a.num_kv_heads * a.num_chunks &&
        nwork >= kSplitMinGroups && nwork < kSplitMaxGroups && !a.sched &&
        a.num_extra == 0 && !a.idx && !sp.direct && !(STEP && sp.fuse)) {
      if (a.has_bias)
        hipLaunchKernelGGL((partition_split_kernel<DK, DV, SW, STEP, true, FP8>),
                           dim3(nwork), dim3(SW * 64), 0, s, a, sp);
      else
        hipLaunchKernelGGL((partition_split_kernel<DK, DV, SW, STEP, false, FP8>),
                           dim3(nwork), dim3(SW * 64), 0, s, a, sp);
      return hipGetLastError();
    }
  }
  const int nwork = a.sched ? a.sched_len : a.total_items;
  const int dyn = residency_lds_bytes<DK, DV, NW, FP8>(a);
  if (a.idx) {  // index-gathered: attend only, one branch, no bias or schedule
    if (STEP || a.has_bias || a.sched || a.num_extra) return hipErrorInvalidValue;
    hipLaunchKernelGGL((partition_bf16_kernel<DK, DV, NW, false, false, true, FP8>),
                       dim3(nwork), dim3(NW * 64), 0, s, a, sp);
  } else if (a.has_bias) {
    hipLaunchKernelGGL((partition_bf16_kernel<DK, DV, NW, STEP, true, false, FP8>),
                       dim3(nwork), dim3(NW * 64), dyn, s, a, sp);
  } else {
    hipLaunchKernelGGL((partition_bf16_kernel<DK, DV, NW, STEP, false, false, FP8>),
                       dim3(nwork), dim3(NW * 64), dyn, s, a, sp);
  }
  return hipGetLastError();
}

template <int DK, int DV, bool STEP, bool FP8>
hipError_t launch_shape(const PartitionArgs &a, const StepParams &sp,
                        hipStream_t s) {
  return launch_one<DK, DV, partition_waves(DK, DV, FP8), STEP, FP8>(a, sp, s);
}

// Launches the kernel of the plan's head widths; fp8 storage must match
// the instantiating file's FP8.
template <bool STEP, bool FP8>
hipError_t dispatch(const PartitionArgs &a, const StepParams &sp,
                    hipStream_t s) {
  if ((a.fp8 != 0) != FP8) return hipErrorInvalidValue;
  if (a.dk == 64 && a.dv == 64) return launch_shape<64, 64, STEP, FP8>(a, sp, s);
  if (a.dk == 128 && a.dv == 128) return launch_shape<128, 128, STEP, FP8>(a, sp, s);
  if (a.dk == 192 && a.dv == 128) return launch_shape<192, 128, STEP, FP8>(a, sp, s);
  if (a.dk == 256 && a.dv == 256) return launch_shape<256, 256, STEP, FP8>(a, sp, s);
  return hipErrorInvalidValue;
}

}  // namespace
}  // namespace gqa
