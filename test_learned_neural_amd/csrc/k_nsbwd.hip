// Newton-Schulz forward recomputation and reverse of the outer-loop backward through per-chunk
// gates, one workgroup per matrix (slab) for the 64 x 128 working shape: every step of a slab runs
// in one launch, its operands staged in LDS, its products on the matrix cores in split bf16.
//
// The iteration (ATLAS summary, section 5, the Newton-Schulz orthogonalisation of the memory's
// update; Atlas-Torch README, Atlas Extensions table, row "Muon / Newton-Schulz"):
//   X_0 = G / (|G| + eps),  A_i = X_i X_i^T,  B_i = b A_i + c A_i^2,  X_{i+1} = a X_i + B_i X_i.
// Its reverse (the outer loop differentiates through the inner updates: Atlas-Torch README, "How
// the memory works"), from Xa = dL/dX_{i+1}, with A_i and B_i symmetric:
//   Ba = Xa X_i^T,  Aa = b Ba + c (Ba A_i + A_i Ba),
//   dL/dX_i = a Xa + B_i Xa + (Aa + Aa^T) X_i,
// where Aa + Aa^T = b Bs + c (Q + Q^T) with Bs = Ba + Ba^T and Q = Bs A_i (A_i Bs = Q^T), so a
// step takes four products: Xa X_i^T, B_i Xa, Bs A_i, S X_i with S = b Bs + c (Q + Q^T).  Last,
// dL/dG = Xa_0 / n - (<Xa_0, X_0> / (n |G|)) G with n = |G| + eps.
//
// Layout: the working matrix is G, or G^T when G has more rows than columns (64 x 128 either
// way).  Wave w of the four holds columns [32w, 32w + 32) as two 32 x 32 register tiles (rows
// 0..31, 32..63); every 64 x 64 matrix of the iteration is symmetric, so it is stored and read in
// either orientation.  The forward keeps X_i^T ([128][64] per step), A_i and B_i ([64][64]) in the
// caller's workspace for the reverse.  Every global access goes through a buffer resource sized to
// its slab, so no access leaves it.
#include "common.h"
#include "internal.h"
#include "mfma_tiles.h"

namespace am {
namespace nsb {

constexpr int R = 64;     // working rows
constexpr int CW = 128;   // working columns
constexpr int NT = 256;   // four waves
constexpr int LD = R + 8;  // [64][64] matrices read 16 bytes per lane along k (A_i, Bs)
constexpr int LE = R + 4;  // [64][64] matrices read 8 bytes per lane (B_i, S)
constexpr int LF = R + 1;  // fp32 [64][64] scratch for tile transposes
// LDS map (uint16 units)
constexpr int XT = 0;             // X_i^T [128][64] hi, then lo (rows of 128 bytes, 8-byte chunks swizzled)
constexpr int XTS = CW * R;
constexpr int YT = XT + 2 * XTS;  // Xa^T hi, lo; later Bs [64][LD] hi, lo
constexpr int AI = YT + 2 * XTS;  // A_i [64][LD] hi, lo
constexpr int SB = AI + 2 * R * LD;  // B_i, later S, [64][LE] hi, lo
constexpr int FT = SB + 2 * R * LE;  // fp32 [64][LF]
constexpr int LDS_U16 = FT + 2 * R * LF;
constexpr int LDS_BYTES = LDS_U16 * 2 + 8 * 4;  // + four partial sums
static_assert(2 * R * LD <= 2 * XTS, "Bs lies in the Xa^T region");
static_assert(LDS_BYTES <= 160 * 1024, "LDS");

struct Args {
  NsSlabGeo g;
  const float* G;   // [M][P]: matrix z / M of memory z % M at goff
  const float* Na;  // reverse: the adjoint of N, G's layout
  float* N;         // forward: the result, G's layout
  float* Ga;        // reverse: the adjoint of G, G's layout
  float* X;         // per slab [steps][128][64]: X_i^T
  float* A;         // per slab [steps][64][64]
  float* B;
  float* sq;        // per slab |G|^2
  int steps;
  float a, b, c, eps;
};

// The working matrix (this lane's column cx, rows 32t + 8q + 4hf + u in register 4q + u of tile t)
// from a matrix in G's layout, and back.
__device__ __forceinline__ void load_work(rsrc_t rm, int tr, int cx, int hf, f32x16 (&x)[2]) {
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int r0 = 32 * t + 8 * q + 4 * hf;
      if (tr) {  // stored [128][64]: row cx holds working column cx
        const float4 v = buf_ld4(rm, (cx * R + r0) * 4, 0);
        x[t][4 * q] = v.x; x[t][4 * q + 1] = v.y; x[t][4 * q + 2] = v.z; x[t][4 * q + 3] = v.w;
      } else {   // stored [64][128]
#pragma unroll
        for (int u = 0; u < 4; ++u) x[t][4 * q + u] = buf_ld(rm, ((r0 + u) * CW + cx) * 4, 0);
      }
    }
}
__device__ __forceinline__ void store_work(rsrc_t rm, int tr, int cx, int hf, const f32x16 (&x)[2]) {
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int r0 = 32 * t + 8 * q + 4 * hf;
      if (tr) {
        buf_st4(rm, (cx * R + r0) * 4, 0, float4{x[t][4 * q], x[t][4 * q + 1], x[t][4 * q + 2], x[t][4 * q + 3]});
      } else {
#pragma unroll
        for (int u = 0; u < 4; ++u) buf_st(rm, ((r0 + u) * CW + cx) * 4, 0, x[t][4 * q + u]);
      }
    }
}

// X_i^T of step i in the workspace slab (this lane's column, as register tiles) and back.
__device__ __forceinline__ void load_xt(rsrc_t rx, int i, int cx, int hf, f32x16 (&x)[2]) {
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float4 v = buf_ld4(rx, ((i * CW + cx) * R + 32 * t + 8 * q + 4 * hf) * 4, 0);
      x[t][4 * q] = v.x; x[t][4 * q + 1] = v.y; x[t][4 * q + 2] = v.z; x[t][4 * q + 3] = v.w;
    }
}
__device__ __forceinline__ void store_xt(rsrc_t rx, int i, int cx, int hf, const f32x16 (&x)[2]) {
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int q = 0; q < 4; ++q)
      buf_st4(rx, ((i * CW + cx) * R + 32 * t + 8 * q + 4 * hf) * 4, 0,
              float4{x[t][4 * q], x[t][4 * q + 1], x[t][4 * q + 2], x[t][4 * q + 3]});
}
// Tile (rt, ct) of a symmetric [64][64] matrix of step i (lane: column 32ct + l32, rows 32rt + 8q
// + 4hf + u), stored as [column][row].
__device__ __forceinline__ void load_sym(rsrc_t rm, int i, int rt, int ct, int lane, f32x16& t) {
  const int hf = lane >> 5, col = 32 * ct + (lane & 31);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float4 v = buf_ld4(rm, ((i * R + col) * R + 32 * rt + 8 * q + 4 * hf) * 4, 0);
    t[4 * q] = v.x; t[4 * q + 1] = v.y; t[4 * q + 2] = v.z; t[4 * q + 3] = v.w;
  }
}
__device__ __forceinline__ void store_sym(rsrc_t rm, int i, int rt, int ct, int lane, const f32x16& t) {
  const int hf = lane >> 5, col = 32 * ct + (lane & 31);
#pragma unroll
  for (int q = 0; q < 4; ++q)
    buf_st4(rm, ((i * R + col) * R + 32 * rt + 8 * q + 4 * hf) * 4, 0,
            float4{t[4 * q], t[4 * q + 1], t[4 * q + 2], t[4 * q + 3]});
}

// X^T of the register tiles into an LDS buffer (split, rows of this lane's column cx).
__device__ __forceinline__ void stage_xt(uint16_t* sm, int bh, int cx, int hf, const f32x16 (&x)[2]) {
  const int xrow = cx * R, xsw = swz(cx) ^ (4 * hf);
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      uint32_t h0, l0, h1, l1;
      split2(x[t][4 * q], x[t][4 * q + 1], h0, l0);
      split2(x[t][4 * q + 2], x[t][4 * q + 3], h1, l1);
      const int o = xrow + ((32 * t + 8 * q) ^ xsw);
      *(uint2*)(sm + bh + o) = uint2{h0, h1};
      *(uint2*)(sm + bh + XTS + o) = uint2{l0, l1};
    }
}

// Tile (rt, ct) of P Q^T for two 64 x 128 matrices staged as transposes (pa: P^T, pb: Q^T), by
// transposing LDS reads: lane (g, e, q) of 16-lane group g reads the chunk of row c = 16ks + 8(g/2)
// + e (+4 for the second half of the k-step) at rows 32rt + 16(g%2) + 4q.
__device__ __forceinline__ f32x16 prod_t(const uint16_t* sm, int pa, int pb, int rt, int ct, int lane) {
  const int g = lane >> 4, e = (lane >> 2) & 3, q4 = 4 * (lane & 3);
  const int c1 = 8 * (g >> 1) + e, c2 = c1 + 4;
  const int ra = 32 * rt + 16 * (g & 1) + q4, rb = 32 * ct + 16 * (g & 1) + q4;
  const int ta1 = c1 * R + (ra ^ swz(c1)), ta2 = c2 * R + (ra ^ swz(c2));
  const int tb1 = c1 * R + (rb ^ swz(c1)), tb2 = c2 * R + (rb ^ swz(c2));
  f32x16 acc = zero16();
#pragma unroll
  for (int ks = 0; ks < CW / 16; ++ks) {
    const int f = (ks & 1) ? 16 : 0, kb = ks * 16 * R;
    const u32x4 ah = cat2(lds_tr16(sm + pa + kb + (ta1 ^ f)), lds_tr16(sm + pa + kb + (ta2 ^ f)));
    const u32x4 al = cat2(lds_tr16(sm + pa + XTS + kb + (ta1 ^ f)), lds_tr16(sm + pa + XTS + kb + (ta2 ^ f)));
    const u32x4 bh = cat2(lds_tr16(sm + pb + kb + (tb1 ^ f)), lds_tr16(sm + pb + kb + (tb2 ^ f)));
    const u32x4 bl = cat2(lds_tr16(sm + pb + XTS + kb + (tb1 ^ f)), lds_tr16(sm + pb + XTS + kb + (tb2 ^ f)));
    acc = mma3(ah, al, bh, bl, acc);
  }
  return acc;
}

// Tile (rt, ct) of P Q for two symmetric 64 x 64 matrices in LDS ([64][LD] hi, then lo).
__device__ __forceinline__ f32x16 prod_sym(const uint16_t* sm, int pa, int pb, int rt, int ct, int lane) {
  const int hf = lane >> 5, l32 = lane & 31;
  const int ara = (32 * rt + l32) * LD + 8 * hf, arb = (32 * ct + l32) * LD + 8 * hf;
  f32x16 acc = zero16();
#pragma unroll
  for (int ks = 0; ks < R / 16; ++ks) {
    const int oa = ara + 16 * ks, ob = arb + 16 * ks;
    acc = mma3(lds16(sm, pa + oa), lds16(sm, pa + R * LD + oa), lds16(sm, pb + ob), lds16(sm, pb + R * LD + ob), acc);
  }
  return acc;
}

// acc[t] += M V for a symmetric 64 x 64 matrix M in LDS ([64][LE] hi, then lo) and the 64 x 128
// matrix V staged as V^T (this lane's column cx, the k operand read back from its own row).
__device__ __forceinline__ void prod_mv(const uint16_t* sm, int pm, int pv, int cx, int lane, f32x16 (&acc)[2]) {
  const int hf = lane >> 5, l32 = lane & 31;
  const int xrow = cx * R, xsw = swz(cx) ^ (4 * hf);
  const int brow = l32 * LE + 4 * hf;
#pragma unroll
  for (int ks = 0; ks < R / 16; ++ks) {
    const int o1 = xrow + ((16 * ks) ^ xsw), o2 = xrow + ((16 * ks + 8) ^ xsw);
    const u32x4 xh = cat2(lds8(sm, pv + o1), lds8(sm, pv + o2));
    const u32x4 xl = cat2(lds8(sm, pv + XTS + o1), lds8(sm, pv + XTS + o2));
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int o0 = brow + 32 * t * LE + 16 * ks;
      const u32x4 ah = cat2(lds8(sm, pm + o0), lds8(sm, pm + o0 + 8));
      const u32x4 al = cat2(lds8(sm, pm + R * LE + o0), lds8(sm, pm + R * LE + o0 + 8));
      acc[t] = mma3(ah, al, xh, xl, acc[t]);
    }
  }
}

// Sum over the workgroup of one value per lane.
__device__ __forceinline__ float block_sum(float v, float* red, int w, int lane) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  if (lane == 0) red[w] = v;
  __syncthreads();
  const float s = red[0] + red[1] + red[2] + red[3];
  __syncthreads();
  return s;
}

struct Slab {
  int z, tr, w, lane, hf, cx, rt, ct;
  rsrc_t rg, rx, ra, rb;
};
__device__ __forceinline__ Slab slab_of(const Args& a) {
  Slab s;
  s.z = blockIdx.x;
  const int mi = s.z / a.g.M, zm = s.z - mi * a.g.M;
  s.tr = a.g.tr[mi];
  s.w = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  s.lane = threadIdx.x & 63;
  s.hf = s.lane >> 5;
  s.cx = 32 * s.w + (s.lane & 31);
  s.rt = s.w >> 1;
  s.ct = s.w & 1;
  const int64_t moff = (int64_t)zm * a.g.P + a.g.goff[mi];
  s.rg = make_rsrc(a.G + moff, (uint32_t)(R * CW * 4));
  s.rx = make_rsrc(a.X + (int64_t)s.z * a.steps * R * CW, (uint32_t)(a.steps * R * CW * 4));
  s.ra = make_rsrc(a.A + (int64_t)s.z * a.steps * R * R, (uint32_t)(a.steps * R * R * 4));
  s.rb = make_rsrc(a.B + (int64_t)s.z * a.steps * R * R, (uint32_t)(a.steps * R * R * 4));
  return s;
}

__global__ void __launch_bounds__(NT) forward_kernel(Args a) {
  extern __shared__ __attribute__((aligned(16))) uint16_t sm[];
  float* red = (float*)(sm + LDS_U16);
  const Slab s = slab_of(a);
  const int64_t moff = (int64_t)(s.z % a.g.M) * a.g.P + a.g.goff[s.z / a.g.M];
  f32x16 x[2];
  load_work(s.rg, s.tr, s.cx, s.hf, x);
  float ss = 0.0f;
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) ss = fmaf(x[t][r], x[t][r], ss);
  const float sq = block_sum(ss, red, s.w, s.lane);
  if (threadIdx.x == 0) a.sq[s.z] = sq;
  const float inv = 1.0f / (sqrtf(sq) + a.eps);
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) x[t][r] *= inv;
  for (int i = 0; i < a.steps; ++i) {
    store_xt(s.rx, i, s.cx, s.hf, x);
    stage_xt(sm, XT, s.cx, s.hf, x);
    __syncthreads();
    // A_i = X X^T
    const f32x16 A = prod_t(sm, XT, XT, s.rt, s.ct, s.lane);
    store_sym(s.ra, i, s.rt, s.ct, s.lane, A);
    store_tile_T(sm, AI, AI + R * LD, LD, A, 32 * s.rt, 32 * s.ct, s.lane);
    __syncthreads();
    // B_i = b A_i + c A_i^2
    const f32x16 A2 = prod_sym(sm, AI, AI, s.rt, s.ct, s.lane);
    f32x16 Bt;
#pragma unroll
    for (int r = 0; r < 16; ++r) Bt[r] = a.b * A[r] + a.c * A2[r];
    store_sym(s.rb, i, s.rt, s.ct, s.lane, Bt);
    store_tile_T(sm, SB, SB + R * LE, LE, Bt, 32 * s.rt, 32 * s.ct, s.lane);
    __syncthreads();
    // X_{i+1} = a X_i + B_i X_i (the k operand X_i from this lane's own row of X^T)
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) x[t][r] *= a.a;
    prod_mv(sm, SB, XT, s.cx, s.lane, x);
    __syncthreads();  // every read of this step's LDS operands before the next step's stores
  }
  store_work(make_rsrc(a.N + moff, (uint32_t)(R * CW * 4)), s.tr, s.cx, s.hf, x);
}

__global__ void __launch_bounds__(NT) reverse_kernel(Args a) {
  extern __shared__ __attribute__((aligned(16))) uint16_t sm[];
  float* red = (float*)(sm + LDS_U16);
  float* ft = (float*)(sm + FT);
  const Slab s = slab_of(a);
  const int64_t moff = (int64_t)(s.z % a.g.M) * a.g.P + a.g.goff[s.z / a.g.M];
  const int l32 = s.lane & 31;
  f32x16 xa[2];
  load_work(make_rsrc(a.Na + moff, (uint32_t)(R * CW * 4)), s.tr, s.cx, s.hf, xa);
  for (int i = a.steps - 1; i >= 0; --i) {
    {  // stage X_i^T, Xa^T, A_i and B_i
      f32x16 xi[2];
      load_xt(s.rx, i, s.cx, s.hf, xi);
      f32x16 at, bt;
      load_sym(s.ra, i, s.rt, s.ct, s.lane, at);
      load_sym(s.rb, i, s.rt, s.ct, s.lane, bt);
      stage_xt(sm, XT, s.cx, s.hf, xi);
      stage_xt(sm, YT, s.cx, s.hf, xa);
      store_tile_T(sm, AI, AI + R * LD, LD, at, 32 * s.rt, 32 * s.ct, s.lane);
      store_tile_T(sm, SB, SB + R * LE, LE, bt, 32 * s.rt, 32 * s.ct, s.lane);
    }
    __syncthreads();
    // Ba = Xa X_i^T (tile rt, ct); Xn = a Xa + B_i Xa
    const f32x16 ba = prod_t(sm, YT, XT, s.rt, s.ct, s.lane);
    f32x16 xn[2];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) xn[t][r] = a.a * xa[t][r];
    prod_mv(sm, SB, YT, s.cx, s.lane, xn);
    // tile element r: row 32rt + 8(r/4) + 4hf + r%4, column 32ct + l32
    const int col = 32 * s.ct + l32, row0 = 32 * s.rt + 4 * s.hf;
#pragma unroll
    for (int r = 0; r < 16; ++r) ft[(row0 + 8 * (r >> 2) + (r & 3)) * LF + col] = ba[r];
    __syncthreads();
    // Bs = Ba + Ba^T over the Xa^T region (read last above)
    f32x16 bs;
#pragma unroll
    for (int r = 0; r < 16; ++r) bs[r] = ba[r] + ft[col * LF + row0 + 8 * (r >> 2) + (r & 3)];
    store_tile_T(sm, YT, YT + R * LD, LD, bs, 32 * s.rt, 32 * s.ct, s.lane);
    __syncthreads();
    // Q = Bs A_i, into the scratch (its Ba^T reads are behind the barrier above)
    const f32x16 q = prod_sym(sm, YT, AI, s.rt, s.ct, s.lane);
#pragma unroll
    for (int r = 0; r < 16; ++r) ft[(row0 + 8 * (r >> 2) + (r & 3)) * LF + col] = q[r];
    __syncthreads();
    // S = b Bs + c (Q + Q^T) over B_i (read last in B_i Xa)
    f32x16 sv;
#pragma unroll
    for (int r = 0; r < 16; ++r) sv[r] = a.b * bs[r] + a.c * (q[r] + ft[col * LF + row0 + 8 * (r >> 2) + (r & 3)]);
    store_tile_T(sm, SB, SB + R * LE, LE, sv, 32 * s.rt, 32 * s.ct, s.lane);
    __syncthreads();
    // Xn += S X_i
    prod_mv(sm, SB, XT, s.cx, s.lane, xn);
#pragma unroll
    for (int t = 0; t < 2; ++t) xa[t] = xn[t];
    __syncthreads();  // every read of this step's LDS operands before the next step's stores
  }
  // dL/dG = Xa_0 / n - (<Xa_0, X_0> / (n |G|)) G
  f32x16 x0[2], g[2];
  load_xt(s.rx, 0, s.cx, s.hf, x0);
  load_work(s.rg, s.tr, s.cx, s.hf, g);
  float dp = 0.0f;
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) dp = fmaf(xa[t][r], x0[t][r], dp);
  const float dot = block_sum(dp, red, s.w, s.lane);
  const float gn = sqrtf(a.sq[s.z]), nn = gn + a.eps;
  const float corr = gn > 0.0f ? dot / (nn * gn) : 0.0f;
  const float inv = 1.0f / nn;
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) g[t][r] = xa[t][r] * inv - corr * g[t][r];
  store_work(make_rsrc(a.Ga + moff, (uint32_t)(R * CW * 4)), s.tr, s.cx, s.hf, g);
}

}  // namespace nsb

bool ns_slab_supported(int rows, int cols, int steps) {
  return rows == nsb::R && cols == nsb::CW && steps >= 1 && steps <= 64;
}

static atlasmem_status ns_slab_launch(void (*kern)(nsb::Args), const nsb::Args& a, hipStream_t st) {
  if (hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, nsb::LDS_BYTES) != hipSuccess)
    return ATLASMEM_E_DEVICE;
  const unsigned nslab = (unsigned)(a.g.nm * a.g.M);
  if (nslab == 0) return ATLASMEM_OK;
  hipLaunchKernelGGL(kern, dim3(nslab), dim3(nsb::NT), nsb::LDS_BYTES, st, a);
  AM_LAUNCH_CHECK();
  return ATLASMEM_OK;
}

atlasmem_status launch_ns_slab_forward(const NsSlabGeo& g, const float* G, float* X, float* A, float* B, float* sq,
                                       float* N, int steps, float ca, float cb, float cc, float eps, hipStream_t st) {
  nsb::Args a{};
  a.g = g;
  a.G = G;
  a.N = N;
  a.X = X;
  a.A = A;
  a.B = B;
  a.sq = sq;
  a.steps = steps;
  a.a = ca;
  a.b = cb;
  a.c = cc;
  a.eps = eps;
  return ns_slab_launch(nsb::forward_kernel, a, st);
}

atlasmem_status launch_ns_slab_reverse(const NsSlabGeo& g, const float* G, const float* Na, const float* X,
                                       const float* A, const float* B, const float* sq, float* Ga, int steps, float ca,
                                       float cb, float cc, float eps, hipStream_t st) {
  nsb::Args a{};
  a.g = g;
  a.G = G;
  a.Na = Na;
  a.Ga = Ga;
  a.X = const_cast<float*>(X);
  a.A = const_cast<float*>(A);
  a.B = const_cast<float*>(B);
  a.sq = const_cast<float*>(sq);
  a.steps = steps;
  a.a = ca;
  a.b = cb;
  a.c = cc;
  a.eps = eps;
  return ns_slab_launch(nsb::reverse_kernel, a, st);
}

}  // namespace am
