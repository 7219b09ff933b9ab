// Shared device helpers for the atlasmem kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

namespace am {

constexpr int kWave = 64;

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Two fp32 -> packed bf16 pair (round to nearest even, one hardware conversion).
__device__ __forceinline__ uint32_t cvt_pk_bf16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}
// Round-to-nearest-even fp32 -> bf16 bit pattern.
__device__ __forceinline__ uint32_t bf16_bits(float x) { return cvt_pk_bf16(x, 0.0f) & 0xFFFFu; }
__device__ __forceinline__ float bf16_value(uint32_t bits) { return __uint_as_float(bits << 16); }

// Split a pair into hi = bf16(x), lo = bf16(x - hi), both packed; hi + lo carries ~16
// significant bits of each value.
__device__ __forceinline__ void split2(float a, float b, uint32_t& hi, uint32_t& lo) {
  hi = cvt_pk_bf16(a, b);
  lo = cvt_pk_bf16(a - __uint_as_float(hi << 16), b - __uint_as_float(hi & 0xFFFF0000u));
}
// Single-value split (bit patterns in the low half).
__device__ __forceinline__ void split_bf16(float x, uint32_t& hi, uint32_t& lo) {
  const uint32_t h = cvt_pk_bf16(x, 0.0f) & 0xFFFFu;
  hi = h;
  lo = cvt_pk_bf16(x - __uint_as_float(h << 16), 0.0f) & 0xFFFFu;
}

// Pack eight fp32 values into bf16x8 hi / lo operand words (little-endian pairs).
__device__ __forceinline__ void pack8(const float* v, u32x4& hi, u32x4& lo) {
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    uint32_t h, l;
    split2(v[2 * p], v[2 * p + 1], h, l);
    hi[p] = h;
    lo[p] = l;
  }
}
__device__ __forceinline__ void pack8_hi(const float* v, u32x4& hi) {
#pragma unroll
  for (int p = 0; p < 4; ++p) hi[p] = cvt_pk_bf16(v[2 * p], v[2 * p + 1]);
}

__device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                 0, 0, 0);
}

// sigma(z) with the hardware exponential and reciprocal (about 1 ulp each)
__device__ __forceinline__ float sigmoidf_(float z) { return __builtin_amdgcn_rcpf(1.0f + __expf(-z)); }
__device__ __forceinline__ float siluf_(float z) { return z * sigmoidf_(z); }
__device__ __forceinline__ float silu_primef_(float z) {
  float s = sigmoidf_(z);
  return s * (1.0f + z * (1.0f - s));
}

// Raw buffer access: a uniform base in a buffer resource plus a 32-bit per-lane byte offset and
// a uniform byte offset, so that per-element addresses cost no 64-bit vector arithmetic.
// Accesses at or beyond `bytes` read 0 / are dropped by the hardware range check.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ float buf_ld(rsrc_t r, int voff, int soff) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0));
}
__device__ __forceinline__ float4 buf_ld4(rsrc_t r, int voff, int soff) {
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
  return float4{__uint_as_float(v[0]), __uint_as_float(v[1]), __uint_as_float(v[2]), __uint_as_float(v[3])};
}
__device__ __forceinline__ uint2 buf_ld8(rsrc_t r, int voff, int soff) {
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0);
  return uint2{v[0], v[1]};
}
__device__ __forceinline__ u32x4 buf_ld16(rsrc_t r, int voff, int soff) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
}
__device__ __forceinline__ uint32_t buf_ld_u16(rsrc_t r, int voff, int soff) {
  return (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, 0);
}
__device__ __forceinline__ void buf_st_u16(rsrc_t r, int voff, int soff, uint32_t x) {
  __builtin_amdgcn_raw_buffer_store_b16((unsigned short)x, r, voff, soff, 0);
}
__device__ __forceinline__ void buf_st(rsrc_t r, int voff, int soff, float x) {
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(x), r, voff, soff, 0);
}
__device__ __forceinline__ void buf_st4(rsrc_t r, int voff, int soff, float4 x) {
  __builtin_amdgcn_raw_buffer_store_b128(
      u32x4{__float_as_uint(x.x), __float_as_uint(x.y), __float_as_uint(x.z), __float_as_uint(x.w)}, r, voff, soff, 0);
}

// Load one input element (bf16 bits or fp32) as float.
__device__ __forceinline__ float load_in(const void* p, int64_t idx, int is_bf16) {
  if (is_bf16) return bf16_value(((const uint16_t*)p)[idx]);
  return ((const float*)p)[idx];
}

}  // namespace am

// Host-side launch helpers
#define AM_LAUNCH_CHECK()                                   \
  do {                                                      \
    hipError_t e_ = hipGetLastError();                      \
    if (e_ != hipSuccess) return ATLASMEM_E_DEVICE;         \
  } while (0)

namespace am {

// Degree-2 feature map phi(x) = [1, x_0..x_{d-1}, x_i x_j / 2 (i <= j, row-major upper
// triangle = combinations_with_replacement order)], C(d+2, 2) features.  The pair index p of
// (i, j) is start(i) + (j - i) with start(i) = i d - i (i - 1) / 2.
__device__ __forceinline__ int pair_start(int i, int d) { return i * d - (i * (i - 1)) / 2; }
__device__ __forceinline__ void pair_of(int p, int d, int& i, int& j) {
  const float fd = 2.0f * d + 1.0f;
  int ii = (int)((fd - sqrtf(fmaxf(fd * fd - 8.0f * (float)p, 0.0f))) * 0.5f);
  ii = ii < 0 ? 0 : (ii > d - 1 ? d - 1 : ii);
  while (ii > 0 && pair_start(ii, d) > p) --ii;
  while (ii + 1 < d && pair_start(ii + 1, d) <= p) ++ii;
  i = ii;
  j = ii + (p - pair_start(ii, d));
}
__device__ __forceinline__ int poly_count(int d) { return 1 + d + (d * (d + 1)) / 2; }

}  // namespace am
