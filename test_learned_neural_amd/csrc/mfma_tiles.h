// 32 x 32 matrix-core tiles shared by the fused kernels (gfx950, v_mfma_f32_32x32x16_bf16): operand
// assembly from LDS, split-bf16 products and tile stores.
//
// A 32 x 32 output tile leaves lane l with rows 8q + 4(l/32) + u (q, u = 0..3) of column l % 32.
// Every fp32 operand is split into bf16 hi + lo and multiplied as hi*hi + hi*lo + lo*hi.
#pragma once

#include "common.h"

namespace am {

__device__ __forceinline__ u32x4 cat2(uint2 a, uint2 b) { return u32x4{a.x, a.y, b.x, b.y}; }
__device__ __forceinline__ uint2 lds8(const uint16_t* s, int off) { return *(const uint2*)(s + off); }
__device__ __forceinline__ u32x4 lds16(const uint16_t* s, int off) { return *(const u32x4*)(s + off); }

// 8 consecutive fp32 of a tile (k-step kl) -> hi / lo operand words
__device__ __forceinline__ void tile_op(const f32x16& t, int kl, u32x4& hi, u32x4& lo) {
  float v[8];
#pragma unroll
  for (int s = 0; s < 8; ++s) v[s] = t[8 * kl + s];
  pack8(v, hi, lo);
}

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.0f;
  return z;
}

__device__ __forceinline__ f32x16 mma3(u32x4 ah, u32x4 al, u32x4 bh, u32x4 bl, f32x16 c) {
  c = mfma32(ah, bh, c);
  c = mfma32(ah, bl, c);
  c = mfma32(al, bh, c);
  return c;
}
__device__ __forceinline__ f32x4 mma3_16(u32x4 ah, u32x4 al, u32x4 bh, u32x4 bl, f32x4 c) {
  c = mfma16(ah, bh, c);
  c = mfma16(ah, bl, c);
  c = mfma16(al, bh, c);
  return c;
}
// PL (the plain bf16 precision): every operand is its bf16 rounding (hi) alone, one product per
// term; the lo words are neither formed nor stored.  Otherwise the three split products.
template <bool PL>
__device__ __forceinline__ f32x16 mmp(u32x4 ah, u32x4 al, u32x4 bh, u32x4 bl, f32x16 c) {
  if constexpr (PL) return mfma32(ah, bh, c);
  else return mma3(ah, al, bh, bl, c);
}
template <bool PL>
__device__ __forceinline__ f32x4 mmp16(u32x4 ah, u32x4 al, u32x4 bh, u32x4 bl, f32x4 c) {
  if constexpr (PL) return mfma16(ah, bh, c);
  else return mma3_16(ah, al, bh, bl, c);
}

// Write a 32x32 fp32 tile (rows r0.., cols c0..) transposed into an LDS matrix [col][row] as
// hi/lo: four consecutive rows of a column are one 8-byte store.
template <bool PL = false>
__device__ __forceinline__ void store_tile_T(uint16_t* sm, int offh, int offl, int ld, const f32x16& t, int r0, int c0,
                                             int lane) {
  const int hf = lane >> 5, col = c0 + (lane & 31);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    uint32_t h0, l0, h1, l1;
    split2(t[4 * q], t[4 * q + 1], h0, l0);
    split2(t[4 * q + 2], t[4 * q + 3], h1, l1);
    const int o = col * ld + r0 + 8 * q + 4 * hf;
    *(uint2*)(sm + offh + o) = uint2{h0, h1};
    if constexpr (!PL) *(uint2*)(sm + offl + o) = uint2{l0, l1};
  }
}

// X^T element (c, r) of the Newton-Schulz buffer lives at c * 64 + (r ^ swz(c)): the XOR moves
// whole 8-byte chunks so that the 8-byte stores and reads along c and the transposing reads
// across four consecutive c all land on distinct banks.
__device__ __forceinline__ int swz(int c) {
  const int x = (c >> 1) & 15;
  return 4 * (((x & 1) << 3) | (x >> 1));
}
typedef short v4i16 __attribute__((ext_vector_type(4)));
// ds_read_b64_tr_b16: within each 16-lane group, lane 4e + q names an 8-byte chunk (row e, four
// consecutive columns 4q..4q+3 of a 4 x 16 block); lane i receives column i of the four rows.
__device__ __forceinline__ uint2 lds_tr16(const uint16_t* p) {
  const v4i16 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)(p));
  return __builtin_bit_cast(uint2, v);
}

}  // namespace am
