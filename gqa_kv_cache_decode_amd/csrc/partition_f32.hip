// Split-K partition kernel for fp32 caches (VALU, any dk/dv up to 256).
//
// fp32 keeps full-precision products, so this family runs on the vector ALUs
// rather than on bf16 matrix cores.  One wavefront per work-group handles one
// (sequence b, KV group g, chunk c) for all heads_per_kv query heads: each
// 64-token tile of K and V is read once with coalesced loads into LDS and
// shared by the group's heads (needle-core attn.rs: each KV head serves its
// query heads by broadcast).  Lane t scores token t against every head,
// the wavefront folds the tile into each head's running maximum, partition and
// weighted value sum (usearch attend), and lane t then owns value columns
// t, t+64, ... of every head for the P.V sum.
#include "device_common.h"
#include "launch.h"

namespace gqa {
namespace {

constexpr int kTok = 64;       // tokens per tile (one per lane)
constexpr int kMaxHeads = 16;  // heads per KV group
constexpr int kMaxCols = 4;    // value columns per lane (dv <= 256)

__global__ __launch_bounds__(64) void partition_f32_kernel(
    const float *__restrict__ q, const float *__restrict__ K,
    const float *__restrict__ V, const int32_t *__restrict__ lens, int batch,
    int max_len, int Hkv, int hpk, int dk, int dv, int chunk, int nchunk,
    float scale_log2, float *__restrict__ part_m, float *__restrict__ part_l,
    float *__restrict__ part_acc) {
  extern __shared__ __attribute__((aligned(16))) float smem[];
  const int ks = dk + 1;           // odd stride: column reads hit 64 banks
  float *Ks = smem;                // [kTok][dk + 1]
  float *Vs = Ks + kTok * ks;      // [kTok][dv]
  float *Ps = Vs + kTok * dv;      // [hpk][kTok]
  float *Qs = Ps + hpk * kTok;     // [hpk][dk]

  const int nwork = batch * Hkv * nchunk;
  const int item = xcd_local_item(blockIdx.x, nwork);
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
    const int d4 = dk >> 2, v4 = dv >> 2;
    for (int e = lane; e < kTok * d4; e += 64) {
      const int tok = e / d4, col = (e % d4) * 4;
      float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
      if (tb + tok < t1)
        x = *reinterpret_cast<const float4 *>(Kg + (tb + tok) * kT + col);
      float *dst = Ks + tok * ks + col;
      dst[0] = x.x; dst[1] = x.y; dst[2] = x.z; dst[3] = x.w;
    }
    for (int e = lane; e < kTok * v4; e += 64) {
      const int tok = e / v4, col = (e % v4) * 4;
      float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
      if (tb + tok < t1)
        x = *reinterpret_cast<const float4 *>(Vg + (tb + tok) * vT + col);
      *reinterpret_cast<float4 *>(Vs + tok * dv + col) = x;
    }
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
#pragma unroll
    for (int h = 0; h < kMaxHeads; ++h) {
      if (h < hpk) {
        const float x = live ? s[h] * scale_log2 : -INFINITY;
        const float m_new = fmaxf(m[h], wave_max(x));
        const float alpha = fast_exp2(m[h] - m_new);
        const float p = fast_exp2(x - m_new);
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

// Shapes whose tile fits the LDS of a work-group.
bool partition_f32_supported(int dk, int dv, int hpk) {
  return hpk >= 1 && hpk <= kMaxHeads && dk >= 4 && dk <= 256 &&
         dk % 4 == 0 && dv >= 4 && dv <= 64 * kMaxCols && dv % 4 == 0 &&
         partition_f32_lds_bytes(dk, dv, hpk) <= kMaxLds;
}

hipError_t launch_partition_f32(const PartitionArgs &a, hipStream_t s) {
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
                     a.chunk_tokens, a.num_chunks, a.scale_log2, a.part_m,
                     a.part_l, a.part_acc);
  return hipGetLastError();
}

}  // namespace gqa
