// Batched small-GEMM engine on CDNA4 matrix cores (v_mfma_f32_16x16x32_bf16).
//
// out[z](i, j) = sum_k A[z](i, k) * B[z](k, j) for every batch index z, with
//  - A and B produced element-wise by loader functors (so transposes, feature maps,
//    SiLU and per-row coefficients are applied while staging, never materialised),
//  - each fp32 operand split into bf16 hi + lo in LDS and the product formed as
//    hi*hi (+ hi*lo + lo*hi in the split precision; a side known to be an exact bf16
//    input contributes no lo term),
//  - fp32 accumulation in the matrix cores and a functor epilogue per output element.
//
// Tile 64 x 64 x 32, 256 threads = 4 waves in a 2 x 2 grid, each wave 32 x 32 = 2 x 2
// MFMA blocks of 16 x 16.  Grid: (ceil(N/64), ceil(M/64), batch).
#pragma once

#include <type_traits>

#include "common.h"

namespace am {

// Loader contract: load8(z, outer, k0, v) fills v[u] = Op(outer, k0 + u) for u = 0..7, zero
// outside [0, outer_dim) x [0, K).  For A, outer = row i; for B, outer = column j.

constexpr int GT = 64;       // output tile
constexpr int GK = 32;       // k step
constexpr int GLD = GK + 8;  // LDS row stride in bf16 (80 bytes: 16-byte aligned, staggers banks)

// An epilogue that reads memory declares `Pre` (what one element reads), `Pre load(z, row, col)`
// and `store(z, row, col, acc, pre)`; one that only writes has just operator()(z, row, col, acc).
template <class EP, class = void>
struct EpiTwoPhase : std::false_type {};
template <class EP>
struct EpiTwoPhase<EP, std::void_t<typename EP::Pre>> : std::true_type {};

// LDS staging of one 64 x 64 x 32 tile step: hi (and, for split operands, lo) words of A and B.
template <bool SPLIT, bool A_EXACT, bool B_EXACT>
struct TileSmem {
  uint16_t Ah[GT * GLD];
  uint16_t Bh[GT * GLD];
  uint16_t Al[SPLIT && !A_EXACT ? GT * GLD : 8];
  uint16_t Bl[SPLIT && !B_EXACT ? GT * GLD : 8];
};

// One output tile (rows m0.., columns n0.. of batch z) by the 256 threads t = 0..255 of a tile
// group.  Every thread of the workgroup executes the same barriers: a group with no tile in a
// round passes active = false and only takes part in them (barriers are workgroup-wide).
template <bool SPLIT, bool A_EXACT, bool B_EXACT, class LA, class LB, class EP>
__device__ __forceinline__ void gemm_tile(int M, int N, int K, const LA& la, const LB& lb, const EP& ep, int z, int m0,
                                          int n0, int t, TileSmem<SPLIT, A_EXACT, B_EXACT>& sm, bool active,
                                          int kbeg = 0, int kend = -1) {
  if (kend < 0) kend = K;
  const int lane = t & 63, w = t >> 6;
  const int wm = w >> 1, wn = w & 1;
  const int lr = lane & 15, lk = (lane >> 4) * 8;

  f32x4 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int srow = t >> 2, sk = (t & 3) * 8;
  for (int k0 = kbeg; k0 < kend; k0 += GK) {
    if (active) {
      {
        float v[8];
        la.load8(z, m0 + srow, k0 + sk, v);
        u32x4 hi, lo;
        if (SPLIT && !A_EXACT) {
          pack8(v, hi, lo);
          *(u32x4*)&sm.Al[srow * GLD + sk] = lo;
        } else {
          pack8_hi(v, hi);
        }
        *(u32x4*)&sm.Ah[srow * GLD + sk] = hi;
      }
      {
        float v[8];
        lb.load8(z, n0 + srow, k0 + sk, v);
        u32x4 hi, lo;
        if (SPLIT && !B_EXACT) {
          pack8(v, hi, lo);
          *(u32x4*)&sm.Bl[srow * GLD + sk] = lo;
        } else {
          pack8_hi(v, hi);
        }
        *(u32x4*)&sm.Bh[srow * GLD + sk] = hi;
      }
    }
    __syncthreads();
    if (active) {
      u32x4 ah[2], bh[2], al[2], bl[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int r = (wm * 32 + i * 16 + lr) * GLD + lk;
        ah[i] = *(const u32x4*)&sm.Ah[r];
        if (SPLIT && !A_EXACT) al[i] = *(const u32x4*)&sm.Al[r];
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int r = (wn * 32 + j * 16 + lr) * GLD + lk;
        bh[j] = *(const u32x4*)&sm.Bh[r];
        if (SPLIT && !B_EXACT) bl[j] = *(const u32x4*)&sm.Bl[r];
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          acc[i][j] = mfma16(ah[i], bh[j], acc[i][j]);
          if (SPLIT && !B_EXACT) acc[i][j] = mfma16(ah[i], bl[j], acc[i][j]);
          if (SPLIT && !A_EXACT) acc[i][j] = mfma16(al[i], bh[j], acc[i][j]);
        }
    }
    __syncthreads();
  }
  if (!active) return;
  if constexpr (EpiTwoPhase<EP>::value) {
    // every element's loads first, then every element's stores: the compiler may not move
    // element r + 1's loads above element r's stores (it cannot rule out aliasing), so this is
    // what lets a lane's sixteen loads be in flight together
    typename EP::Pre pre[2][2][4];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = m0 + wm * 32 + i * 16 + (lane >> 4) * 4 + r;
          const int col = n0 + wn * 32 + j * 16 + lr;
          if (row < M && col < N) pre[i][j][r] = ep.load(z, row, col);
        }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = m0 + wm * 32 + i * 16 + (lane >> 4) * 4 + r;
          const int col = n0 + wn * 32 + j * 16 + lr;
          if (row < M && col < N) ep.store(z, row, col, acc[i][j][r], pre[i][j][r]);
        }
  } else {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = m0 + wm * 32 + i * 16 + (lane >> 4) * 4 + r;
          const int col = n0 + wn * 32 + j * 16 + lr;
          if (row < M && col < N) ep(z, row, col, acc[i][j][r]);
        }
  }
}

template <bool SPLIT, bool A_EXACT, bool B_EXACT, class LA, class LB, class EP>
__global__ void __launch_bounds__(256) gemm_tile_kernel(int M, int N, int K, LA la, LB lb, EP ep) {
  __shared__ __attribute__((aligned(16))) TileSmem<SPLIT, A_EXACT, B_EXACT> sm;
  gemm_tile<SPLIT, A_EXACT, B_EXACT>(M, N, K, la, lb, ep, blockIdx.z, blockIdx.y * GT, blockIdx.x * GT, threadIdx.x,
                                     sm, true);
}

// Split-K: a product with few output tiles and a long k range (each k-step is a dependent
// global-load round trip) runs as nsplit k-slices, slice sp of batch z writing its partial tile
// to part[((sp * batch + z) * M + row) * N + col]; the reduction sums the slices in slice order
// (deterministic) and applies the product's epilogue.
struct EpiPart {
  float* part;
  int64_t mn;
  int N, batch, sp;
  __device__ __forceinline__ void operator()(int z, int row, int col, float v) const {
    part[((int64_t)sp * batch + z) * mn + (int64_t)row * N + col] = v;
  }
};

template <bool SPLIT, bool A_EXACT, bool B_EXACT, class LA, class LB>
__global__ void __launch_bounds__(256) gemm_part_kernel(int M, int N, int K, int batch, int kslice, LA la, LB lb,
                                                        float* part) {
  __shared__ __attribute__((aligned(16))) TileSmem<SPLIT, A_EXACT, B_EXACT> sm;
  const int z = blockIdx.z % batch, sp = blockIdx.z / batch;
  const int kb = sp * kslice, ke = kb + kslice < K ? kb + kslice : K;
  const EpiPart ep{part, (int64_t)M * N, N, batch, sp};
  gemm_tile<SPLIT, A_EXACT, B_EXACT>(M, N, K, la, lb, ep, z, blockIdx.y * GT, blockIdx.x * GT, threadIdx.x, sm, true,
                                     kb, ke);
}

// Split-K inside one workgroup, for products of at most KGROUPS k-steps: group g (256 threads)
// forms the partial tile of k-step g, writes it over its own LDS operand buffers, and after a
// barrier the workgroup sums the groups' partials in group order (the order of the launched
// slices' reduction) and applies the product's epilogue.  No partial tiles in global memory and
// no reduction launch.  Taken, where split products are allowed, for every product of 2..KGROUPS
// k-steps with at least KGROUP_MIN_TILES output tiles, also those too wide for launched slices
// (128 memories of the 64 -> 128 -> 64 memory on MI355X: per-chunk path 4.79 -> 4.08 ms, its
// outer backward 17.9 -> 15.9 ms; the 384 -> 768 -> 384 memory 1.34 -> 1.24 ms); with fewer tiles,
// one workgroup per k-step spreads a tile's loads over more CUs, which eight memories' products
// (8-16 tiles) need (per-token retrieval 8.1 -> 9.1 ms this way).
constexpr int KGROUPS = 4;
constexpr int KGROUP_MIN_TILES = 128;
template <bool SPLIT, bool A_EXACT, bool B_EXACT>
union KGroupSmem {  // a group's operand buffers, then its partial tile
  TileSmem<SPLIT, A_EXACT, B_EXACT> tile;
  float red[GT * GT];
};

struct EpiLdsTile {  // element (row, col) of the tile at (m0, n0) into red[(row - m0) * GT + col - n0]
  float* red;
  int m0, n0;
  __device__ __forceinline__ void operator()(int, int row, int col, float v) const {
    red[(row - m0) * GT + (col - n0)] = v;
  }
};

template <bool SPLIT, bool A_EXACT, bool B_EXACT, class LA, class LB, class EP>
__global__ void __launch_bounds__(256 * KGROUPS) gemm_kgroup_kernel(int M, int N, int K, LA la, LB lb, EP ep) {
  __shared__ __attribute__((aligned(16))) KGroupSmem<SPLIT, A_EXACT, B_EXACT> sm[KGROUPS];
  const int ng = blockDim.x >> 8;  // groups: the product's k-steps (2 .. KGROUPS)
  const int g = threadIdx.x >> 8, t = threadIdx.x & 255;
  const int z = blockIdx.z, m0 = blockIdx.y * GT, n0 = blockIdx.x * GT;
  // gemm_tile's last k-step ends at a barrier, after which its epilogue may overwrite the
  // group's operand buffers
  gemm_tile<SPLIT, A_EXACT, B_EXACT>(M, N, K, la, lb, EpiLdsTile{sm[g].red, m0, n0}, z, m0, n0, t, sm[g].tile, true,
                                     g * GK, g * GK + GK);
  __syncthreads();
  for (int e = threadIdx.x; e < GT * GT; e += blockDim.x) {
    const int row = m0 + e / GT, col = n0 + e % GT;
    if (row >= M || col >= N) continue;
    float v = 0.0f;
    for (int q = 0; q < ng; ++q) v += sm[q].red[e];
    if constexpr (EpiTwoPhase<EP>::value) ep.store(z, row, col, v, ep.load(z, row, col));
    else ep(z, row, col, v);
  }
}

template <class EP>
__global__ void splitk_reduce_kernel(int M, int N, int batch, int nsplit, const float* __restrict__ part, EP ep) {
  const int64_t mn = (int64_t)M * N;
  const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= mn * batch) return;
  const int z = (int)(e / mn);
  const int64_t rem = e - z * mn;
  const int row = (int)(rem / N), col = (int)(rem - (int64_t)row * N);
  float v = 0.0f;
  for (int sp = 0; sp < nsplit; ++sp) v += part[((int64_t)sp * batch + z) * mn + rem];
  if constexpr (EpiTwoPhase<EP>::value) ep.store(z, row, col, v, ep.load(z, row, col));
  else ep(z, row, col, v);
}

// Slices for a product of `tiles` output tiles and nk >= 2 k-steps: enough workgroups to spread
// over the chip (about four per CU) and partials that fit the scratch.  Up to 12 k-steps a slice
// may be a single step (the short products of eight memories' chunks, 8-16 tiles each, are
// latency-bound chains); longer k ranges keep at least two steps per slice, where more slices
// only add partial-sum traffic.
inline int splitk_slices(int M, int N, int K, int batch, int64_t scratch_floats) {
  const int64_t tiles = (int64_t)((N + GT - 1) / GT) * ((M + GT - 1) / GT) * batch;
  const int nk = (K + GK - 1) / GK;
  if (scratch_floats <= 0 || tiles > 256 || nk < 2) return 1;
  int ns = (int)((1024 + tiles - 1) / tiles);
  const int cap = nk <= 12 ? nk : nk / 2;
  if (ns > cap) ns = cap;
  while (ns > 1 && (int64_t)ns * batch * M * N > scratch_floats) --ns;
  return ns < 1 ? 1 : ns;
}

template <bool A_EXACT, bool B_EXACT, class LA, class LB, class EP>
inline void launch_gemm(bool split, int M, int N, int K, int batch, const LA& la, const LB& lb, const EP& ep,
                        hipStream_t st, float* scratch = nullptr, int64_t scratch_floats = 0) {
  if (M <= 0 || N <= 0 || batch <= 0) return;
  const int ns = splitk_slices(M, N, K, batch, scratch ? scratch_floats : 0);
  const int nk = (K + GK - 1) / GK;
  const int64_t tiles = (int64_t)((N + GT - 1) / GT) * ((M + GT - 1) / GT) * batch;
  if (scratch && scratch_floats > 0 && nk >= 2 && nk <= KGROUPS && tiles >= KGROUP_MIN_TILES) {
    dim3 grid((N + GT - 1) / GT, (M + GT - 1) / GT, batch);
    if (split)
      hipLaunchKernelGGL((gemm_kgroup_kernel<true, A_EXACT, B_EXACT, LA, LB, EP>), grid, dim3(256 * nk), 0, st, M, N,
                         K, la, lb, ep);
    else
      hipLaunchKernelGGL((gemm_kgroup_kernel<false, A_EXACT, B_EXACT, LA, LB, EP>), grid, dim3(256 * nk), 0, st, M,
                         N, K, la, lb, ep);
    return;
  }
  if (ns > 1) {
    const int kslice = ((nk + ns - 1) / ns) * GK;
    const int nsl = (K + kslice - 1) / kslice;
    dim3 grid((N + GT - 1) / GT, (M + GT - 1) / GT, batch * nsl);
    if (split)
      hipLaunchKernelGGL((gemm_part_kernel<true, A_EXACT, B_EXACT, LA, LB>), grid, dim3(256), 0, st, M, N, K, batch,
                         kslice, la, lb, scratch);
    else
      hipLaunchKernelGGL((gemm_part_kernel<false, A_EXACT, B_EXACT, LA, LB>), grid, dim3(256), 0, st, M, N, K, batch,
                         kslice, la, lb, scratch);
    const int64_t n = (int64_t)M * N * batch;
    hipLaunchKernelGGL((splitk_reduce_kernel<EP>), dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, M, N, batch,
                       nsl, (const float*)scratch, ep);
    return;
  }
  dim3 grid((N + GT - 1) / GT, (M + GT - 1) / GT, batch);
  if (split)
    hipLaunchKernelGGL((gemm_tile_kernel<true, A_EXACT, B_EXACT, LA, LB, EP>), grid, dim3(256), 0, st, M, N, K, la,
                       lb, ep);
  else
    hipLaunchKernelGGL((gemm_tile_kernel<false, A_EXACT, B_EXACT, LA, LB, EP>), grid, dim3(256), 0, st, M, N, K, la,
                       lb, ep);
}

// ---------------------------------------------------------------------------- fp32 operands
//
// The F32 precision: operands kept in fp32 and multiplied on the matrix cores' fp32 path
// (v_mfma_f32_16x16x4_f32, fp32 products and accumulation), for configurations whose rounding
// the split bf16 products amplify too much.  Same 64 x 64 x 32 tiles, loaders, epilogues and
// output layout as gemm_tile (lane l of a 16 x 16 block holds rows 4(l/16) + r of column l % 16);
// a k-step of 32 is eight k = 4 products, lane l supplying k = 4s + l/16 of its row (A) or column
// (B).  No split-K: this path is for accuracy, not speed.
constexpr int GLDF = GK + 4;  // fp32 row stride: rows 36 words apart put 16 rows x 4 k on 64 banks

template <class LA, class LB, class EP>
__global__ void __launch_bounds__(256) gemm_f32_kernel(int M, int N, int K, LA la, LB lb, EP ep) {
  __shared__ __attribute__((aligned(16))) float As[GT * GLDF];
  __shared__ __attribute__((aligned(16))) float Bs[GT * GLDF];
  const int z = blockIdx.z, m0 = blockIdx.y * GT, n0 = blockIdx.x * GT;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int wm = w >> 1, wn = w & 1;
  const int lr = lane & 15, lq = lane >> 4;
  f32x4 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int srow = t >> 2, sk = (t & 3) * 8;
  for (int k0 = 0; k0 < K; k0 += GK) {
    {
      float v[8];
      la.load8(z, m0 + srow, k0 + sk, v);
      *(float4*)&As[srow * GLDF + sk] = float4{v[0], v[1], v[2], v[3]};
      *(float4*)&As[srow * GLDF + sk + 4] = float4{v[4], v[5], v[6], v[7]};
      lb.load8(z, n0 + srow, k0 + sk, v);
      *(float4*)&Bs[srow * GLDF + sk] = float4{v[0], v[1], v[2], v[3]};
      *(float4*)&Bs[srow * GLDF + sk + 4] = float4{v[4], v[5], v[6], v[7]};
    }
    __syncthreads();
#pragma unroll
    for (int s4 = 0; s4 < GK / 4; ++s4) {
      float a[2], b[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) a[i] = As[(wm * 32 + i * 16 + lr) * GLDF + 4 * s4 + lq];
#pragma unroll
      for (int j = 0; j < 2; ++j) b[j] = Bs[(wn * 32 + j * 16 + lr) * GLDF + 4 * s4 + lq];
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[i], b[j], acc[i][j], 0, 0, 0);
    }
    __syncthreads();
  }
  if constexpr (EpiTwoPhase<EP>::value) {
    typename EP::Pre pre[2][2][4];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = m0 + wm * 32 + i * 16 + lq * 4 + r, col = n0 + wn * 32 + j * 16 + lr;
          if (row < M && col < N) pre[i][j][r] = ep.load(z, row, col);
        }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = m0 + wm * 32 + i * 16 + lq * 4 + r, col = n0 + wn * 32 + j * 16 + lr;
          if (row < M && col < N) ep.store(z, row, col, acc[i][j][r], pre[i][j][r]);
        }
  } else {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = m0 + wm * 32 + i * 16 + lq * 4 + r, col = n0 + wn * 32 + j * 16 + lr;
          if (row < M && col < N) ep(z, row, col, acc[i][j][r]);
        }
  }
}

template <class LA, class LB, class EP>
inline void launch_gemm_f32(int M, int N, int K, int batch, const LA& la, const LB& lb, const EP& ep, hipStream_t st) {
  if (M <= 0 || N <= 0 || batch <= 0) return;
  dim3 grid((N + GT - 1) / GT, (M + GT - 1) / GT, batch);
  hipLaunchKernelGGL((gemm_f32_kernel<LA, LB, EP>), grid, dim3(256), 0, st, M, N, K, la, lb, ep);
}

// ---------------------------------------------------------------------------- generic loaders

enum Xform { XF_NONE = 0, XF_SILU = 1, XF_COEF = 2, XF_SCALE = 3, XF_GATED = 4, XF_MAT = 5 };

// Element (outer, k) = xf(base[zoff(z) + outer * so + k * sk]); zoff(z) = (z / zdiv) * sz.
// XF_COEF multiplies by coef[(z / zdiv) * cz + csel(z) + k]  (per-k coefficient; csel picks
// one of two coefficient arrays by z % 2 when `pair` is set).
// XF_SCALE multiplies by scale[z].
// XF_GATED is silu(x) times the element `gofs` further on (the gated memory's activation
// silu(Z1) * Z3, with Z3 stored beside Z1).
// XF_MAT multiplies element (outer, k) by coef0[(z / zdiv) * cz + outer * cld + k] (a per-element
// coefficient matrix).
struct StridedLoader {
  const float* base;
  int64_t sz, so, sk;
  int zdiv;
  int outer_dim, K;
  int xf;
  const float* coef0;
  const float* coef1;
  int64_t cz;
  const float* scale;
  int64_t gofs;
  int64_t cld;
  __device__ __forceinline__ void load8(int z, int outer, int k0, float* v) const {
    const int zz = z / zdiv;
    const float* p = base + zz * sz + (int64_t)outer * so;
    const float* cf = nullptr;
    if (xf == XF_COEF) cf = ((zdiv == 2 && (z & 1)) ? coef1 : coef0) + zz * cz;
    if (xf == XF_MAT) cf = coef0 + zz * cz + (int64_t)outer * cld;
    const float sc = (xf == XF_SCALE) ? scale[z] : 1.0f;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int k = k0 + u;
      float x = 0.0f;
      if (outer < outer_dim && k < K) {
        x = p[(int64_t)k * sk];
        if (xf == XF_SILU) x = siluf_(x);
        else if (xf == XF_GATED) x = siluf_(x) * p[(int64_t)k * sk + gofs];
        else if (xf == XF_COEF || xf == XF_MAT) x *= cf[k];
        else if (xf == XF_SCALE) x *= sc;
      }
      v[u] = x;
    }
  }
};
// The same loader with clamped indices and every load of a call issued before any is used: fewer
// instructions per element where the whole call is in range.  Used by the chunk-loop kernel, one
// workgroup per memory, where the loaders' instruction count sets the chunk's time (the
// per-product launches, with many workgroups per product, run the plain loader).
struct StridedLoaderC : StridedLoader {
  __device__ __forceinline__ void load8(int z, int outer, int k0, float* v) const {
    const int zz = z / zdiv;
    const bool orow = outer < outer_dim;
    const int oc = orow ? outer : 0;
    const float* p = base + zz * sz + (int64_t)oc * so;
    const float* cf = nullptr;
    if (xf == XF_COEF) cf = ((zdiv == 2 && (z & 1)) ? coef1 : coef0) + zz * cz;
    if (xf == XF_MAT) cf = coef0 + zz * cz + (int64_t)oc * cld;
    float x[8], g[8];
    if (k0 + 8 <= K) {
      // all eight in range: one base address, 32-bit strides (immediate offsets when sk == 1)
      const float* q = p + (int64_t)k0 * sk;
      const int s32 = (int)sk;
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        x[u] = sk == 1 ? q[u] : q[u * s32];
        g[u] = 1.0f;
        if (xf == XF_GATED) g[u] = sk == 1 ? q[u + gofs] : q[u * s32 + gofs];
        else if (xf == XF_COEF || xf == XF_MAT) g[u] = cf[k0 + u];
        else if (xf == XF_SCALE) g[u] = scale[z];
      }
    } else {
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int k = k0 + u;
        const int kc = k < K ? k : K - 1;
        x[u] = p[(int64_t)kc * sk];
        g[u] = 1.0f;
        if (xf == XF_GATED) g[u] = p[(int64_t)kc * sk + gofs];
        else if (xf == XF_COEF || xf == XF_MAT) g[u] = cf[kc];
        else if (xf == XF_SCALE) g[u] = scale[z];
      }
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      float y = x[u];
      if (xf == XF_SILU) y = siluf_(y);
      else if (xf == XF_GATED) y = siluf_(y) * g[u];
      else if (xf == XF_COEF || xf == XF_MAT || xf == XF_SCALE) y *= g[u];
      v[u] = (orow && k0 + u < K) ? y : 0.0f;
    }
  }
};
__host__ __device__ inline StridedLoaderC clamped(const StridedLoader& l) {
  StridedLoaderC c;
  static_cast<StridedLoader&>(c) = l;
  return c;
}


}  // namespace am
