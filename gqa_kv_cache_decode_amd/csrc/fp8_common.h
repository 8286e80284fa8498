// E4M3 (OCP 8-bit floating point, "E4M3FN") codes on gfx950: decode to
// bf16 for the matrix cores, and the quantisation of new rows.
//
// A cache of codes carries one fp32 scale per (sequence, KV head) for K and
// one for V; code c stands for decode(c) * scale.  Every E4M3 value has at
// most four significant bits and an exponent within bf16's range, so it is
// exact in bf16: the kernels stage codes in LDS and decode each MFMA operand
// to bf16 as they read it, folding the K scale into the logit scale and the
// V scale into the weighted value sum.
#pragma once

#include "device_common.h"

namespace gqa {

typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr float kE4m3Max = 448.0f;

// Four codes (the bytes of w, lowest first) as four bf16 values in two
// words: gfx950's packed E4M3 -> bf16 conversion, two codes per instruction,
// with a unit scale (the conversion multiplies by the scale; 1 leaves every
// decoded value as it is, and each is exact in bf16).
__device__ __forceinline__ uint2 e4m3x4_to_bf16(uint32_t w) {
  uint2 r;
  r.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(
                                         w, 1.0f, false));  // bytes 0, 1
  r.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(
                                         w, 1.0f, true));   // bytes 2, 3
  return r;
}

// Eight codes (w0 holds codes 0..3, w1 codes 4..7, lowest byte first) as an
// MFMA operand of eight bf16 values, in order.
__device__ __forceinline__ bf16x8 e4m3x8_to_bf16x8(uint32_t w0, uint32_t w1) {
  const uint2 a = e4m3x4_to_bf16(w0), b = e4m3x4_to_bf16(w1);
  return __builtin_bit_cast(bf16x8, u32x4{a.x, a.y, b.x, b.y});
}

// The code of x: nearest E4M3 value, ties to the even mantissa, magnitudes
// above 448 saturated.  The hardware conversion rounds to nearest even but
// does not saturate (it gives NaN from 480 up), hence the clamp first; the
// clamp keeps the sign of zero.
__device__ __forceinline__ float e4m3_clamp(float x) {
  return fminf(fmaxf(x, -kE4m3Max), kE4m3Max);
}

// Codes of four fp32 values packed into a word (element 0 in the low byte).
__device__ __forceinline__ uint32_t e4m3_pack4(float x0, float x1, float x2,
                                               float x3) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(e4m3_clamp(x0), e4m3_clamp(x1), 0,
                                          false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(e4m3_clamp(x2), e4m3_clamp(x3), w, true);
  return (uint32_t)w;
}

// The factor a value is multiplied by before encoding: the correctly
// rounded fp32 reciprocal of its scale.
__device__ __forceinline__ float e4m3_inv_scale(float scale) {
  return 1.0f / scale;
}

// Codes of eight bf16 values (one 16-byte piece) times `inv_scale`, each
// product rounded to fp32.
__device__ __forceinline__ uint2 e4m3_quantize8(u32x4 x, float inv_scale) {
  float f[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(x[i] << 16) * inv_scale;
    f[2 * i + 1] = __uint_as_float(x[i] & 0xFFFF0000u) * inv_scale;
  }
  uint2 r;
  r.x = e4m3_pack4(f[0], f[1], f[2], f[3]);
  r.y = e4m3_pack4(f[4], f[5], f[6], f[7]);
  return r;
}

// Codes of sixteen bf16 values at `src` (two 16-byte pieces), times
// `inv_scale`.
__device__ __forceinline__ u32x4 e4m3_quantize16(const uint16_t *src,
                                                 float inv_scale) {
  const uint2 a = e4m3_quantize8(stream_load16(src), inv_scale);
  const uint2 b = e4m3_quantize8(stream_load16(src + 8), inv_scale);
  return u32x4{a.x, a.y, b.x, b.y};
}

// Stores one KV group's rows of the new token (bf16 [d] each) into the cache
// slot as codes (kinv, vinv: e4m3_inv_scale of the group's scales), 16 codes
// per 16-byte piece, spread over the threads first, first + stride, ...  As
// for bf16 rows, nothing in the same launch reads the slot, so the stores are
// not waited for.
__device__ __forceinline__ void store_group_row_e4m3(
    const uint16_t *kn, u32x4 *kd, int kpieces, float kinv,
    const uint16_t *vn, u32x4 *vd, int vpieces, float vinv, int first,
    int stride) {
  for (int e = first; e < kpieces + vpieces; e += stride) {
    if (e < kpieces)
      kd[e] = e4m3_quantize16(kn + e * 16, kinv);
    else
      vd[e - kpieces] = e4m3_quantize16(vn + (e - kpieces) * 16, vinv);
  }
}

}  // namespace gqa
