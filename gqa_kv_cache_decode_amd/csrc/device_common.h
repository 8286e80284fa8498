// Device-side helpers shared by the decode kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gqa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kLog2e = 1.44269504088896340736f;

// 2^x on the hardware exp unit (v_exp_f32): exact 0 for -inf.
__device__ __forceinline__ float fast_exp2(float x) {
  return __builtin_amdgcn_exp2f(x);
}

// 16-byte load marked nontemporal (data read once per call).
__device__ __forceinline__ u32x4 stream_load16(const void *p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
}

// Raw buffer view of `bytes` bytes at `base` (the gfx9 descriptor word for
// untyped 32-bit data).  Loads past `bytes` return zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_view(const void *base,
                                                              uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, bytes,
                                           0x00020000);
}

// 16-byte nontemporal load at byte offset `off` of a buffer view.
__device__ __forceinline__ u32x4 stream_load16(__amdgpu_buffer_rsrc_t v,
                                               uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(v, off, 0, /*nt*/ 2);
}

// 16-byte (four fp32) load at byte offset `off` of a buffer view; zeros past
// the view's end.
__device__ __forceinline__ f32x4 load4f(__amdgpu_buffer_rsrc_t v, uint32_t off) {
  return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(v, off, 0, 0));
}

// The running maximum used as the exponent reference: a state that has seen
// no finite logit yet (m = -inf) takes 0, so exp2(x - ref) is 0, not NaN.
__device__ __forceinline__ float exp_ref(float m) {
  return m == -INFINITY ? 0.0f : m;
}

__device__ __forceinline__ float bf16_bits_to_float(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Maximum / sum over the four 16-lane rows of a wavefront (lanes i, i ^ 16,
// i ^ 32, i ^ 48).  gfx950's row-swap permutes are VALU operations: the
// 32-lane swap of x with itself yields the lower half of x in one result and
// the upper half in the other (each repeated twice), the 16-lane swap the
// even and the odd rows likewise, so two steps cover the four rows without a
// round trip through LDS.
__device__ __forceinline__ float rows_max(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x),
                                                  __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x),
                                                  __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ __forceinline__ float rows_sum(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x),
                                                  __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x),
                                                  __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// LDS transpose load (ds_read_b64_tr_b16) from a generic pointer into LDS.
// Each of the 16 lanes of a row fetches four consecutive 16-bit values at its
// own address; lane j of the row then receives value j % 4 of the fetches of
// lanes j / 4, j / 4 + 4, j / 4 + 8 and j / 4 + 12 (in that order).
__device__ __forceinline__ i16x4 lds_read_tr16(const uint16_t *p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_i16x4 *)(const_cast<uint16_t *>(p)));
}

typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;

// LDS transpose load of bytes (ds_read_b64_tr_b8).  Each of the 16 lanes of a
// row fetches eight consecutive bytes at its own address; lane j of the row
// then receives byte j % 8 of the fetches of lanes j / 8, j / 8 + 2, ...,
// j / 8 + 14 (in that order, lowest byte first).
__device__ __forceinline__ i32x2 lds_read_tr8(const unsigned char *p) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32(
      (lds_i32x2 *)(const_cast<unsigned char *>(p)));
}

// Butterfly reductions across the 64 lanes of a wavefront.
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x = fmaxf(x, __shfl_xor(x, off, 64));
  return x;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, 64);
  return x;
}

__device__ __forceinline__ int wave_sum_int(int x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, 64);
  return x;
}

// Makes this wavefront's own LDS writes visible to its other lanes and keeps
// the compiler from moving LDS accesses across the point.  Only valid for LDS
// regions private to one wavefront.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ int clamp_len(int n, int max_len) {
  return n < 0 ? 0 : (n > max_len ? max_len : n);
}

// Spreads consecutive work items over the same XCD: hardware hands block i to
// XCD i % 8, so item w = (i % 8) * (N / 8) + i / 8 gives each XCD a contiguous
// run of items (the N % 8 tail keeps the identity map).  Consecutive items are
// the chunks of one (sequence, KV group), whose rows then stream through one
// XCD's path to memory.  (A chunk-major order, which balances ragged lengths
// over the XCDs exactly, measured slower on every workload shape.)
__device__ __forceinline__ int xcd_local_item(int i, int n) {
  const int per = n >> 3;
  return (i < (per << 3)) ? (i & 7) * per + (i >> 3) : i;
}

}  // namespace gqa
