// kv_append: needle-core KvCache::push_kv, one work-group per sequence.
//
// With n = lens_in[b]: if 0 <= n < max_len the token's rows for every KV head
// ([num_kv_heads][d], contiguous in the [max_len][num_kv_heads][d] layout)
// are copied to slot n and lens_out[b] = n + 1.  Otherwise nothing is written
// and the drop is counted: the page warns that the cache is full and returns
// without writing.
#include "device_common.h"
#include "fp8_common.h"
#include "launch.h"

namespace gqa {
namespace {

constexpr int kThreads = 256;
constexpr int kPieces = 4;  // 16-byte pieces per thread held in registers

// Copies one row; pieces of 16 bytes when everything is 16-byte aligned.
// The source pieces are loaded before the destination slot is known, so the
// loads overlap the read of the length.
__device__ __forceinline__ void copy_rows(unsigned char *kd, const unsigned char *ks,
                                          int kbytes, unsigned char *vd,
                                          const unsigned char *vs, int vbytes,
                                          bool aligned, bool ok) {
  if (aligned) {
    const int nk = kbytes / 16, nv = vbytes / 16;
    const u32x4 *k16 = reinterpret_cast<const u32x4 *>(ks);
    const u32x4 *v16 = reinterpret_cast<const u32x4 *>(vs);
    u32x4 kb[kPieces], vb[kPieces];
#pragma unroll
    for (int p = 0; p < kPieces; ++p) {
      const int i = threadIdx.x + p * kThreads;
      if (i < nk) kb[p] = k16[i];
      if (i < nv) vb[p] = v16[i];
    }
    if (!ok) return;
#pragma unroll
    for (int p = 0; p < kPieces; ++p) {
      const int i = threadIdx.x + p * kThreads;
      if (i < nk) reinterpret_cast<u32x4 *>(kd)[i] = kb[p];
      if (i < nv) reinterpret_cast<u32x4 *>(vd)[i] = vb[p];
    }
    for (int i = threadIdx.x + kPieces * kThreads; i < nk; i += kThreads)
      reinterpret_cast<u32x4 *>(kd)[i] = k16[i];
    for (int i = threadIdx.x + kPieces * kThreads; i < nv; i += kThreads)
      reinterpret_cast<u32x4 *>(vd)[i] = v16[i];
  } else if (ok) {
    for (int i = threadIdx.x; i < kbytes / 2; i += kThreads)
      reinterpret_cast<uint16_t *>(kd)[i] = reinterpret_cast<const uint16_t *>(ks)[i];
    for (int i = threadIdx.x; i < vbytes / 2; i += kThreads)
      reinterpret_cast<uint16_t *>(vd)[i] = reinterpret_cast<const uint16_t *>(vs)[i];
  }
}

__global__ __launch_bounds__(kThreads) void append_kernel(AppendArgs a) {
  const int b = blockIdx.x;
  const int n = a.lens_in[b];
  const bool ok = n >= 0 && n < a.max_len;
  const size_t slot = (size_t)b * a.max_len + (ok ? n : 0);
  unsigned char *kd = static_cast<unsigned char *>(a.k) + slot * a.row_bytes_k;
  unsigned char *vd = static_cast<unsigned char *>(a.v) + slot * a.row_bytes_v;
  const unsigned char *ks =
      static_cast<const unsigned char *>(a.k_new) + (size_t)b * a.row_bytes_k;
  const unsigned char *vs =
      static_cast<const unsigned char *>(a.v_new) + (size_t)b * a.row_bytes_v;
  const bool aligned = ((reinterpret_cast<uintptr_t>(a.k) |
                         reinterpret_cast<uintptr_t>(a.v) |
                         reinterpret_cast<uintptr_t>(a.k_new) |
                         reinterpret_cast<uintptr_t>(a.v_new) |
                         (uintptr_t)a.row_bytes_k | (uintptr_t)a.row_bytes_v) &
                        15) == 0;
  copy_rows(kd, ks, a.row_bytes_k, vd, vs, a.row_bytes_v, aligned, ok);
  __syncthreads();  // lens_in is read by every thread before lens_out is set
  if (threadIdx.x == 0) {
    a.lens_out[b] = ok ? n + 1 : n;
    if (!ok && a.dropped) atomicAdd(a.dropped, 1);
  }
}

// kv_append into fp8 caches: the new bf16 rows are quantised (times the fp32
// reciprocal of the sequence's scale of that KV head, nearest E4M3 code, ties
// to even, saturating at 448) into slot n, sixteen codes per thread and piece.
__global__ __launch_bounds__(kThreads) void append_e4m3_kernel(AppendArgs a) {
  const int b = blockIdx.x;
  const int n = a.lens_in[b];
  const bool ok = n >= 0 && n < a.max_len;
  if (ok) {
    const size_t slot = (size_t)b * a.max_len + n;
    const size_t sb = (size_t)b * a.num_kv_heads;
    const int dk = a.row_bytes_k / a.num_kv_heads;
    const int dv = a.row_bytes_v / a.num_kv_heads;
    u32x4 *kd = reinterpret_cast<u32x4 *>(static_cast<unsigned char *>(a.k) +
                                          slot * a.row_bytes_k);
    u32x4 *vd = reinterpret_cast<u32x4 *>(static_cast<unsigned char *>(a.v) +
                                          slot * a.row_bytes_v);
    const uint16_t *kn = static_cast<const uint16_t *>(a.k_new) +
                         (size_t)b * a.row_bytes_k;
    const uint16_t *vn = static_cast<const uint16_t *>(a.v_new) +
                         (size_t)b * a.row_bytes_v;
    for (int e = threadIdx.x; e < a.row_bytes_k / 16; e += kThreads)
      kd[e] = e4m3_quantize16(kn + e * 16,
                              e4m3_inv_scale(a.k_scale[sb + e * 16 / dk]));
    for (int e = threadIdx.x; e < a.row_bytes_v / 16; e += kThreads)
      vd[e] = e4m3_quantize16(vn + e * 16,
                              e4m3_inv_scale(a.v_scale[sb + e * 16 / dv]));
  }
  __syncthreads();  // lens_in is read by every thread before lens_out is set
  if (threadIdx.x == 0) {
    a.lens_out[b] = ok ? n + 1 : n;
    if (!ok && a.dropped) atomicAdd(a.dropped, 1);
  }
}

// Streaming layout (cortiq-engine NystromState: permanent exact sink keys and
// an exact window ring per KV group; the key a full ring evicts moves into
// the exact main cache here, where the page feeds an approximate far field).
// With t = count_in[b]:
//   t < 0: nothing changes, the drop is counted;
//   t < S: the token goes to sink slot t;
//   else:  ring slot r = (t - S) % W; when the ring is full (t - S >= W) its
//          token there (position t - W) first moves to main slot t - S - W
//          (a full main cache drops the new token instead; without a main
//          cache the old token simply leaves), then the new token takes r.
// count_out = t + 1 unless dropped; lens_* = the live keys of each part.
// One work-group per sequence; each thread copies its own 4-byte words, so
// the old ring word is read before the same thread overwrites it.  With fp8
// caches a word holds four codes of one KV head, quantised from the four
// bf16 values of the new row with that head's scale of the sequence.
__device__ __forceinline__ uint32_t stream_word(const StreamAppendArgs &a,
                                                const void *row, int i,
                                                const float *scale, int b,
                                                int d) {
  if (!a.fp8) return static_cast<const uint32_t *>(row)[i];
  const uint2 x = static_cast<const uint2 *>(row)[i];  // bf16 values 4i..4i+3
  const float inv =
      e4m3_inv_scale(scale[(size_t)b * a.num_kv_heads + 4 * i / d]);
  return e4m3_pack4(__uint_as_float(x.x << 16) * inv,
                    __uint_as_float(x.x & 0xFFFF0000u) * inv,
                    __uint_as_float(x.y << 16) * inv,
                    __uint_as_float(x.y & 0xFFFF0000u) * inv);
}

__global__ __launch_bounds__(kThreads) void stream_append_kernel(
    StreamAppendArgs a) {
  const int b = blockIdx.x;
  const int t = a.count_in[b];
  const int S = a.sink, W = a.window, M = a.main_len;
  bool ok = t >= 0;
  uint32_t *kd = nullptr, *vd = nullptr;   // destination of the new token
  uint32_t *ek = nullptr, *ev = nullptr;   // main slot of the evicted token
  if (ok && t < S) {
    kd = static_cast<uint32_t *>(a.sink_k) + ((size_t)b * S + t) * (a.row_bytes_k / 4);
    vd = static_cast<uint32_t *>(a.sink_v) + ((size_t)b * S + t) * (a.row_bytes_v / 4);
  } else if (ok) {
    const int r = (t - S) % W;
    if (t - S >= W && a.main_k) {
      const int j = t - S - W;
      if (j >= M) {
        ok = false;
      } else {
        ek = static_cast<uint32_t *>(a.main_k) + ((size_t)b * M + j) * (a.row_bytes_k / 4);
        ev = static_cast<uint32_t *>(a.main_v) + ((size_t)b * M + j) * (a.row_bytes_v / 4);
      }
    }
    kd = static_cast<uint32_t *>(a.ring_k) + ((size_t)b * W + r) * (a.row_bytes_k / 4);
    vd = static_cast<uint32_t *>(a.ring_v) + ((size_t)b * W + r) * (a.row_bytes_v / 4);
  }
  if (ok) {
    // the new rows: as stored (4-byte words), or bf16 for fp8 caches
    const int in_esize = a.fp8 ? 2 : 1;  // input bytes per stored byte
    const void *kn = static_cast<const unsigned char *>(a.k_new) +
                     (size_t)b * a.row_bytes_k * in_esize;
    const void *vn = static_cast<const unsigned char *>(a.v_new) +
                     (size_t)b * a.row_bytes_v * in_esize;
    const int dk = a.fp8 ? a.row_bytes_k / a.num_kv_heads : 0;
    const int dv = a.fp8 ? a.row_bytes_v / a.num_kv_heads : 0;
    for (int i = threadIdx.x; i < a.row_bytes_k / 4; i += kThreads) {
      if (ek) ek[i] = kd[i];
      kd[i] = stream_word(a, kn, i, a.k_scale, b, dk);
    }
    for (int i = threadIdx.x; i < a.row_bytes_v / 4; i += kThreads) {
      if (ev) ev[i] = vd[i];
      vd[i] = stream_word(a, vn, i, a.v_scale, b, dv);
    }
  }
  __syncthreads();  // count_in is read by every thread before count_out is set
  if (threadIdx.x == 0) {
    const int t1 = ok ? t + 1 : t;
    const int tc = t1 < 0 ? 0 : t1;
    a.count_out[b] = t1;
    if (a.lens_sink) a.lens_sink[b] = min(tc, S);
    a.lens_ring[b] = min(max(tc - S, 0), W);
    if (a.lens_main) a.lens_main[b] = min(max(tc - S - W, 0), M);
    if (!ok && a.dropped) atomicAdd(a.dropped, 1);
  }
}

}  // namespace

hipError_t launch_append(const AppendArgs &a, hipStream_t s) {
  if (a.fp8)
    hipLaunchKernelGGL(append_e4m3_kernel, dim3(a.batch), dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL(append_kernel, dim3(a.batch), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_stream_append(const StreamAppendArgs &a, hipStream_t s) {
  hipLaunchKernelGGL(stream_append_kernel, dim3(a.batch), dim3(kThreads), 0, s,
                     a);
  return hipGetLastError();
}

}  // namespace gqa
