// Split-K partition kernel for bf16 caches on gfx950 (MFMA 16x16x32 bf16).
//
// One work-group handles one (sequence b, KV group g, chunk c) and all
// heads_per_kv query heads of the group.  Every K/V row of the chunk is read
// from HBM once, with 16-byte coalesced loads, staged in the wavefront's own
// LDS slice, and shared by all heads of the group through the MFMA N dimension
// (needle-core attn.rs module doc: each KV head serves its query heads by
// broadcast, not repeat-copy; cortiq-engine NystromState: the rows of a group
// are identical for all its heads, so they are held once per group).
//
// Per 32-token tile a wavefront computes
//   S^T[token][head] = K_tile[token][:] . q[head][:]         (MFMA, A = K)
// then folds the tile into each head's running maximum m, partition l and
// weighted value sum acc (usearch attend: every key folds into each head's
// running maximum, partition and weighted value sum), in base-2 units:
//   m' = max(m, max_j s_j), alpha = 2^(m - m'), p_j = 2^(s_j - m'),
//   l = alpha l + sum_j p_j,  acc = alpha acc + sum_j p_j V_j
// with acc^T[dv][head] += V_tile^T[dv][token] . P^T[token][head] on MFMA.
// The S^T accumulator layout (lane = head column, 4 consecutive tokens per
// lane group) is exactly the B-operand layout the P.V product needs, so P never
// leaves registers.  P is split as p = hi + lo with hi, lo bf16 so that the
// product keeps ~16 bits of each weight (two MFMAs instead of one; the matrix
// cores are far from busy on this HBM-bound loop).
//
// Heads are padded to 16 (the MFMA N width); padded heads see q = 0 and are
// never written.  Tokens of a tile past the chunk end are loaded as zeros and
// masked to -inf logits, so padding slots of the cache are never read.
#include "device_common.h"
#include "launch.h"

namespace gqa {
namespace {

constexpr int kTileTokens = 32;

template <int DK, int DV>
struct Bf16Geom {
  static_assert(DK % 32 == 0 && DV % 16 == 0, "head widths");
  static constexpr int kPieces = DK / 8;  // 16-byte pieces per K row
  static constexpr int vPieces = DV / 8;
  static constexpr int kLoads = kTileTokens * kPieces / 64;  // per lane
  static constexpr int vLoads = kTileTokens * vPieces / 64;
  static_assert(kTileTokens * kPieces % 64 == 0, "K tile split");
  static_assert(kTileTokens * vPieces % 64 == 0, "V tile split");
  static constexpr int kStride = DK + 8;  // LDS row stride in bf16 (+16 B pad)
  static constexpr int vStride = DV + 8;
  static constexpr int waveLdsElems = kTileTokens * (kStride + vStride);
};

template <int DK, int DV, int NW>
__global__ __launch_bounds__(NW * 64) void partition_bf16_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ K,
    const uint16_t *__restrict__ V, const int32_t *__restrict__ lens,
    int batch, int max_len, int Hkv, int hpk, int chunk, int nchunk,
    float scale_log2, float *__restrict__ part_m, float *__restrict__ part_l,
    float *__restrict__ part_acc) {
  using G = Bf16Geom<DK, DV>;
  constexpr int kMergeFloats = NW * 16 * (DV + 2);
  constexpr int kTileBytes = NW * G::waveLdsElems * 2;
  constexpr int kLdsBytes =
      kTileBytes > kMergeFloats * 4 ? kTileBytes : kMergeFloats * 4;
  __shared__ __attribute__((aligned(16))) unsigned char lds[kLdsBytes];

  const int nwork = batch * Hkv * nchunk;
  const int item = xcd_local_item(blockIdx.x, nwork);
  const int c = item % nchunk;
  const int bg = item / nchunk;
  const int g = bg % Hkv;
  const int b = bg / Hkv;

  const int n = clamp_len(lens[b], max_len);
  const int t0 = c * chunk;
  if (t0 >= n) return;  // whole work-group: nothing of this chunk is live
  const int t1 = min(t0 + chunk, n);
  const int ntiles = (t1 - t0 + kTileTokens - 1) / kTileTokens;

  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int hl = lane & 15;  // head column of this lane
  const int kg = lane >> 4;  // lane group: k-slice of MFMA operands
  const int Hq = Hkv * hpk;

  // q as the B operand of S^T = K q^T: lane holds head hl, dims s*32+kg*8..+8
  bf16x8 qf[DK / 32];
  {
    const bool live = hl < hpk;
    const uint16_t *qrow = q + ((size_t)b * Hq + (size_t)g * hpk + hl) * DK;
#pragma unroll
    for (int s = 0; s < DK / 32; ++s) {
      if (live) {
        qf[s] = *reinterpret_cast<const bf16x8 *>(qrow + s * 32 + kg * 8);
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) qf[s][j] = (__bf16)0.0f;
      }
    }
  }

  uint16_t *Ks = reinterpret_cast<uint16_t *>(lds) + w * G::waveLdsElems;
  uint16_t *Vs = Ks + kTileTokens * G::kStride;

  const size_t kTok = (size_t)Hkv * DK;  // elements between tokens
  const size_t vTok = (size_t)Hkv * DV;
  const uint16_t *Kg = K + ((size_t)b * max_len * Hkv + g) * DK;
  const uint16_t *Vg = V + ((size_t)b * max_len * Hkv + g) * DV;

  // K/V are read exactly once per call, so the loads are nontemporal: they
  // stream through without displacing cached lines.
  u32x4 kr[G::kLoads], vr[G::vLoads];
  auto issue = [&](int tile) {
    const int tb = t0 + tile * kTileTokens;
#pragma unroll
    for (int i = 0; i < G::kLoads; ++i) {
      const int idx = i * 64 + lane;
      const int t = tb + idx / G::kPieces;
      const int pc = idx % G::kPieces;
      kr[i] = (t < t1) ? stream_load16(Kg + t * kTok + pc * 8) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int i = 0; i < G::vLoads; ++i) {
      const int idx = i * 64 + lane;
      const int t = tb + idx / G::vPieces;
      const int pc = idx % G::vPieces;
      vr[i] = (t < t1) ? stream_load16(Vg + t * vTok + pc * 8) : u32x4{0, 0, 0, 0};
    }
  };

  float m_run = -INFINITY;  // base-2 running max of head hl
  float l_run = 0.0f;       // this lane's share of the partition
  f32x4 o[DV / 16];         // acc^T: head hl, dv rows blk*16 + kg*4 + i
#pragma unroll
  for (int blk = 0; blk < DV / 16; ++blk) o[blk] = f32x4{0.f, 0.f, 0.f, 0.f};

  int tile = w;
  if (tile < ntiles) issue(tile);
  for (; tile < ntiles; tile += NW) {
    wave_lds_sync();  // previous tile's LDS reads are done
#pragma unroll
    for (int i = 0; i < G::kLoads; ++i) {
      const int idx = i * 64 + lane;
      *reinterpret_cast<u32x4 *>(Ks + (idx / G::kPieces) * G::kStride +
                                 (idx % G::kPieces) * 8) = kr[i];
    }
#pragma unroll
    for (int i = 0; i < G::vLoads; ++i) {
      const int idx = i * 64 + lane;
      *reinterpret_cast<u32x4 *>(Vs + (idx / G::vPieces) * G::vStride +
                                 (idx % G::vPieces) * 8) = vr[i];
    }
    if (tile + NW < ntiles) issue(tile + NW);  // next tile in flight meanwhile
    wave_lds_sync();

    // S^T for tokens rb*16 + kg*4 + i (i < 4), head hl
    f32x4 sacc[2];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      sacc[rb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < DK / 32; ++s) {
        const bf16x8 a = *reinterpret_cast<const bf16x8 *>(
            Ks + (rb * 16 + hl) * G::kStride + s * 32 + kg * 8);
        sacc[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[s], sacc[rb],
                                                           0, 0, 0);
      }
    }

    const int tb = t0 + tile * kTileTokens;
    float x[8];
    float mt = -INFINITY;
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = tb + rb * 16 + kg * 4 + i;
        const float v = (t < t1) ? sacc[rb][i] * scale_log2 : -INFINITY;
        x[rb * 4 + i] = v;
        mt = fmaxf(mt, v);
      }
    }
    mt = fmaxf(mt, __shfl_xor(mt, 16, 64));
    mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
    const float m_new = fmaxf(m_run, mt);
    const float alpha = fast_exp2(m_run - m_new);
    m_run = m_new;

    bf16x8 phi, plo;
    float psum = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float p = fast_exp2(x[j] - m_new);
      psum += p;
      const __bf16 h = (__bf16)p;
      phi[j] = h;
      plo[j] = (__bf16)(p - (float)h);
    }
    l_run = l_run * alpha + psum;

    // acc^T += V^T P^T; the A operand gathers V[token(kg, j)][blk*16 + hl]
    // with token(kg, j) = j < 4 ? kg*4 + j : 16 + kg*4 + (j - 4), the token
    // order of this lane's P values.
#pragma unroll
    for (int blk = 0; blk < DV / 16; ++blk) {
      bf16x8 a;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int tok = (j < 4) ? (kg * 4 + j) : (16 + kg * 4 + (j - 4));
        a[j] = __builtin_bit_cast(__bf16, Vs[tok * G::vStride + blk * 16 + hl]);
      }
      o[blk] *= alpha;
      o[blk] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, phi, o[blk], 0, 0, 0);
      o[blk] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, plo, o[blk], 0, 0, 0);
    }
  }

  // Partition of head hl over the whole wavefront.
  float l_tot = l_run + __shfl_xor(l_run, 16, 64);
  l_tot += __shfl_xor(l_tot, 32, 64);

  // Merge the wavefronts' states through LDS and write one partial per head.
  __syncthreads();
  float *wm = reinterpret_cast<float *>(lds);
  float *wl = wm + NW * 16;
  float *wacc = wl + NW * 16;
  if (lane < 16) {
    wm[w * 16 + lane] = m_run;
    wl[w * 16 + lane] = l_tot;
  }
#pragma unroll
  for (int blk = 0; blk < DV / 16; ++blk)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      wacc[(w * 16 + hl) * DV + blk * 16 + kg * 4 + i] = o[blk][i];
  __syncthreads();

  for (int e = threadIdx.x; e < hpk * DV; e += NW * 64) {
    const int h = e / DV;
    const int d = e % DV;
    float M = -INFINITY;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) M = fmaxf(M, wm[ww * 16 + h]);
    float acc = 0.0f, L = 0.0f;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) {
      const float f = fast_exp2(wm[ww * 16 + h] - M);
      acc += f * wacc[(ww * 16 + h) * DV + d];
      L += f * wl[ww * 16 + h];
    }
    const size_t row = (size_t)b * Hq + (size_t)g * hpk + h;
    part_acc[(row * nchunk + c) * DV + d] = acc;
    if (d == 0) {
      part_m[row * nchunk + c] = M * kLn2;
      part_l[row * nchunk + c] = L;
    }
  }
}

template <int DK, int DV, int NW>
hipError_t launch_one(const PartitionArgs &a, hipStream_t s) {
  const int nwork = a.batch * a.num_kv_heads * a.num_chunks;
  hipLaunchKernelGGL((partition_bf16_kernel<DK, DV, NW>), dim3(nwork),
                     dim3(NW * 64), 0, s,
                     static_cast<const uint16_t *>(a.q),
                     static_cast<const uint16_t *>(a.k),
                     static_cast<const uint16_t *>(a.v), a.lens, a.batch,
                     a.max_len, a.num_kv_heads, a.hpk, a.chunk_tokens,
                     a.num_chunks, a.scale_log2, a.part_m, a.part_l,
                     a.part_acc);
  return hipGetLastError();
}

}  // namespace

bool partition_bf16_supported(int dk, int dv, int hpk) {
  if (hpk < 1 || hpk > 16) return false;
  return (dk == 64 && dv == 64) || (dk == 128 && dv == 128) ||
         (dk == 192 && dv == 128) || (dk == 256 && dv == 256);
}

// Two wavefronts per work-group: the split-K plan sizes chunks so that the
// launch holds about a thousand wavefronts, each streaming a long run of
// tiles, which measured best across the workload shapes on MI355X.
hipError_t launch_partition_bf16(const PartitionArgs &a, hipStream_t s) {
  if (a.dk == 64 && a.dv == 64) return launch_one<64, 64, kPartitionWaves>(a, s);
  if (a.dk == 128 && a.dv == 128) return launch_one<128, 128, kPartitionWaves>(a, s);
  if (a.dk == 192 && a.dv == 128) return launch_one<192, 128, kPartitionWaves>(a, s);
  if (a.dk == 256 && a.dv == 256) return launch_one<256, 256, kPartitionWaves>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace gqa
