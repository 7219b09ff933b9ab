// Newton-Schulz orthogonalisation of the per-chunk surprise (Atlas-Torch README, Atlas
// Extensions table, Muon / Newton-Schulz; ATLAS summary, section 5), one workgroup per matrix.
//
// X0 = G / (||G||_F + eps) in the orientation with rows <= cols (m x n, m <= 64, n <= 128,
// zero-padded to 64 x 128), then `steps` times
//     A = X X^T,   B = b A + c A^2,   X = a X + B X
// on the matrix cores.  X lives in fp32 registers (each wave owns a 64 x 32 column slab of X in
// the output layout of the X-update product, so the a X term needs no memory traffic); its
// bf16 hi/lo split is kept in LDS twice, row-major (operand of X X^T) and transposed (B operand
// of B X); A and B are kept as hi/lo in LDS (A is symmetric, so its rows serve as columns).
// The result is written back in G's orientation, or consumed by the momentum / forgetting
// epilogue S = eta_c S - theta_c X, W = (1 - alpha_c) W + S.
// The B operand of B X (eight consecutive rows of one column of X per lane) is read from the
// row-major copy with the transposing LDS read, so X is kept once: 71.6 KB of LDS per workgroup,
// two workgroups per CU.
#include "common.h"
#include "internal.h"

namespace am {

constexpr int NSM = 64, NSN = 128;
constexpr int LX = NSN + 8;  // row stride of X (bf16)
constexpr int LT = NSM + 8;  // row stride of X^T, A, B (bf16)

typedef short ns_v4i16 __attribute__((ext_vector_type(4)));
// ds_read_b64_tr_b16: within each 16-lane group, lane 4e + q names the 8-byte chunk of row e,
// columns 4q..4q+3 of a 4 x 16 block of bf16; lane i receives column i of the four rows.
__device__ __forceinline__ uint2 ns_tr16(const uint16_t* p) {
  const ns_v4i16 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) ns_v4i16*)(p));
  return __builtin_bit_cast(uint2, v);
}

struct NsArgs {
  const float* G;
  int64_t ldG;
  int rows, cols, steps;
  float a, b, c, eps;
  float* out;
  NsUpdate u;
  int has_upd;
  // groups of gsize matrices each (block b: group b / gsize, matrix b % gsize of it): shape, offset
  // of the group's matrices in G and in the state (the update epilogue)
  int gsize;
  int grows[3], gcols[3];
  int64_t goff[3], uoff[3];
};

template <bool SPLIT>
__global__ void __launch_bounds__(256) ns_kernel(NsArgs p) {
  __shared__ __attribute__((aligned(16))) uint16_t Xh[NSM * LX];
  __shared__ __attribute__((aligned(16))) uint16_t Xl[SPLIT ? NSM * LX : 8];
  __shared__ __attribute__((aligned(16))) uint16_t Ah[NSM * LT];
  __shared__ __attribute__((aligned(16))) uint16_t Al[SPLIT ? NSM * LT : 8];
  __shared__ __attribute__((aligned(16))) uint16_t Bh[NSM * LT];
  __shared__ __attribute__((aligned(16))) uint16_t Bl[SPLIT ? NSM * LT : 8];
  __shared__ float red[4];

  const int gi = blockIdx.x / p.gsize, mat = blockIdx.x - gi * p.gsize;
  const int rows = p.grows[gi], cols = p.gcols[gi];
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int lr = lane & 15, lq = lane >> 4, lk = lq * 8;
  const bool tr = rows > cols;
  const int m = tr ? cols : rows;
  const int n = tr ? rows : cols;
  const float* g = p.G + p.goff[gi] + (int64_t)mat * p.ldG;

  // x[ri][cj][r]: X(i, j) with i = 16 ri + 4 lq + r, j = 32 w + 16 cj + lr
  float x[4][2][4];
  float ss = 0.0f;
#pragma unroll
  for (int ri = 0; ri < 4; ++ri)
#pragma unroll
    for (int cj = 0; cj < 2; ++cj)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 16 * ri + 4 * lq + r, j = 32 * w + 16 * cj + lr;
        float v = 0.0f;
        if (i < m && j < n) v = tr ? g[(int64_t)j * cols + i] : g[(int64_t)i * cols + j];
        x[ri][cj][r] = v;
        ss = fmaf(v, v, ss);
      }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off, 64);
  if (lane == 0) red[w] = ss;
  __syncthreads();
  const float inv = 1.0f / (sqrtf(red[0] + red[1] + red[2] + red[3]) + p.eps);

  auto store_x = [&]() {
#pragma unroll
    for (int ri = 0; ri < 4; ++ri)
#pragma unroll
      for (int cj = 0; cj < 2; ++cj)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = 16 * ri + 4 * lq + r, j = 32 * w + 16 * cj + lr;
          uint32_t hi, lo;
          split_bf16(x[ri][cj][r], hi, lo);
          Xh[i * LX + j] = (uint16_t)hi;
          if (SPLIT) Xl[i * LX + j] = (uint16_t)lo;
        }
  };
#pragma unroll
  for (int ri = 0; ri < 4; ++ri)
#pragma unroll
    for (int cj = 0; cj < 2; ++cj)
#pragma unroll
      for (int r = 0; r < 4; ++r) x[ri][cj][r] *= inv;
  store_x();
  __syncthreads();

  for (int step = 0; step < p.steps; ++step) {
    // A = X X^T: wave w owns rows 16w..16w+15, all 64 columns
    f32x4 accA[4];
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) accA[cb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < NSN / 32; ++kk) {
      const int ao = (16 * w + lr) * LX + kk * 32 + lk;
      const u32x4 ah = *(const u32x4*)&Xh[ao];
      u32x4 al;
      if (SPLIT) al = *(const u32x4*)&Xl[ao];
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) {
        const int bo = (16 * cb + lr) * LX + kk * 32 + lk;
        const u32x4 bh = *(const u32x4*)&Xh[bo];
        accA[cb] = mfma16(ah, bh, accA[cb]);
        if (SPLIT) {
          const u32x4 bl = *(const u32x4*)&Xl[bo];
          accA[cb] = mfma16(ah, bl, accA[cb]);
          accA[cb] = mfma16(al, bh, accA[cb]);
        }
      }
    }
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 16 * w + 4 * lq + r, j = 16 * cb + lr;
        uint32_t hi, lo;
        split_bf16(accA[cb][r], hi, lo);
        Ah[i * LT + j] = (uint16_t)hi;
        if (SPLIT) Al[i * LT + j] = (uint16_t)lo;
      }
    __syncthreads();
    // B = b A + c A^2 (same layout as A)
    f32x4 accB[4];
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) accB[cb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < NSM / 32; ++kk) {
      const int ao = (16 * w + lr) * LT + kk * 32 + lk;
      const u32x4 ah = *(const u32x4*)&Ah[ao];
      u32x4 al;
      if (SPLIT) al = *(const u32x4*)&Al[ao];
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) {
        const int bo = (16 * cb + lr) * LT + kk * 32 + lk;  // column j of A = row j (symmetric)
        const u32x4 bh = *(const u32x4*)&Ah[bo];
        accB[cb] = mfma16(ah, bh, accB[cb]);
        if (SPLIT) {
          const u32x4 bl = *(const u32x4*)&Al[bo];
          accB[cb] = mfma16(ah, bl, accB[cb]);
          accB[cb] = mfma16(al, bh, accB[cb]);
        }
      }
    }
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 16 * w + 4 * lq + r, j = 16 * cb + lr;
        const float bv = p.b * accA[cb][r] + p.c * accB[cb][r];
        uint32_t hi, lo;
        split_bf16(bv, hi, lo);
        Bh[i * LT + j] = (uint16_t)hi;
        if (SPLIT) Bl[i * LT + j] = (uint16_t)lo;
      }
    __syncthreads();
    // X = a X + B X: wave w owns columns 32w..32w+31, all 64 rows
    f32x4 acc[4][2];
#pragma unroll
    for (int ri = 0; ri < 4; ++ri)
#pragma unroll
      for (int cj = 0; cj < 2; ++cj) acc[ri][cj] = f32x4{0.f, 0.f, 0.f, 0.f};
    // transposing reads: lane 4e + q of group lq addresses row 32 kk + 8 lq + e (+4), columns
    // 32 w + 16 cj + 4q .. +3, and receives column 32 w + 16 cj + lr of those rows
    const int te = (lane & 15) >> 2, tq = lane & 3;
#pragma unroll
    for (int kk = 0; kk < NSM / 32; ++kk) {
      u32x4 bh[2], bl[2];
#pragma unroll
      for (int cj = 0; cj < 2; ++cj) {
        const int bo = (32 * kk + 8 * lq + te) * LX + 32 * w + 16 * cj + 4 * tq;
        const uint2 h0 = ns_tr16(&Xh[bo]), h1 = ns_tr16(&Xh[bo + 4 * LX]);
        bh[cj] = u32x4{h0.x, h0.y, h1.x, h1.y};
        if (SPLIT) {
          const uint2 l0 = ns_tr16(&Xl[bo]), l1 = ns_tr16(&Xl[bo + 4 * LX]);
          bl[cj] = u32x4{l0.x, l0.y, l1.x, l1.y};
        }
      }
#pragma unroll
      for (int ri = 0; ri < 4; ++ri) {
        const int ao = (16 * ri + lr) * LT + kk * 32 + lk;
        const u32x4 ah = *(const u32x4*)&Bh[ao];
        u32x4 al;
        if (SPLIT) al = *(const u32x4*)&Bl[ao];
#pragma unroll
        for (int cj = 0; cj < 2; ++cj) {
          acc[ri][cj] = mfma16(ah, bh[cj], acc[ri][cj]);
          if (SPLIT) {
            acc[ri][cj] = mfma16(ah, bl[cj], acc[ri][cj]);
            acc[ri][cj] = mfma16(al, bh[cj], acc[ri][cj]);
          }
        }
      }
    }
#pragma unroll
    for (int ri = 0; ri < 4; ++ri)
#pragma unroll
      for (int cj = 0; cj < 2; ++cj)
#pragma unroll
        for (int r = 0; r < 4; ++r) x[ri][cj][r] = p.a * x[ri][cj][r] + acc[ri][cj][r];
    __syncthreads();  // every wave is done reading X and B
    store_x();
    __syncthreads();
  }

  // write back in G's orientation, or apply the momentum / forgetting update
  bool bad = false;
#pragma unroll
  for (int ri = 0; ri < 4; ++ri)
#pragma unroll
    for (int cj = 0; cj < 2; ++cj)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 16 * ri + 4 * lq + r, j = 32 * w + 16 * cj + lr;
        if (i < m && j < n) {
          const int gr = tr ? j : i, gc = tr ? i : j;
          const float v = x[ri][cj][r];
          if (!p.has_upd) {
            p.out[(int64_t)mat * rows * cols + (int64_t)gr * cols + gc] = v;
          } else {
            const NsUpdate& u = p.u;
            const int mem = mat / u.mats_per_mem;
            const int64_t e = (int64_t)mem * u.P + p.uoff[gi] + (int64_t)gr * cols + gc;
            const int64_t gi = (int64_t)mem * u.ld_gate + u.k;
            const float s = u.eta[gi] * u.Sin[e] - u.theta[gi] * v;
            const float wv = (1.0f - u.alpha[gi]) * u.Win[e] + s;
            u.Sout[e] = s;
            u.Wout[e] = wv;
            bad |= !(isfinite(s) && isfinite(wv));
          }
        }
      }
  if (bad) p.u.flag[0] = 1;
}

// The F32 precision: the same iteration with fp32 operands and fp32 fused multiply-adds on the
// vector units, one workgroup per matrix.  X (64 x 128, zero-padded), A and B live in LDS as fp32;
// every product walks its k index in natural order.  For configurations whose rounding the split
// bf16 products amplify beyond the tolerance; speed is not the point here.
constexpr int FXL = NSN + 1;  // fp32 row strides (odd: a column walk touches distinct banks)
constexpr int FAL = NSM + 1;

__global__ void __launch_bounds__(256) ns_f32_kernel(NsArgs p) {
  __shared__ float Xs[NSM * FXL];
  __shared__ float As[NSM * FAL];  // A, then B = b A + c A^2 in its place
  __shared__ float red[4];
  const int gi = blockIdx.x / p.gsize, mat = blockIdx.x - gi * p.gsize;
  const int rows = p.grows[gi], cols = p.gcols[gi];
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const bool tr = rows > cols;
  const int m = tr ? cols : rows;
  const int n = tr ? rows : cols;
  const float* g = p.G + p.goff[gi] + (int64_t)mat * p.ldG;
  float ss = 0.0f;
  for (int e = t; e < NSM * NSN; e += 256) {
    const int i = e / NSN, j = e % NSN;
    float v = 0.0f;
    if (i < m && j < n) v = tr ? g[(int64_t)j * cols + i] : g[(int64_t)i * cols + j];
    Xs[i * FXL + j] = v;
    ss = fmaf(v, v, ss);
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off, 64);
  if (lane == 0) red[w] = ss;
  __syncthreads();
  const float inv = 1.0f / (sqrtf(red[0] + red[1] + red[2] + red[3]) + p.eps);
  for (int e = t; e < NSM * NSN; e += 256) Xs[(e / NSN) * FXL + e % NSN] *= inv;
  __syncthreads();
  // thread t owns row i = t / 4 and columns j = t % 4 + 4 q of A and B (q < 16) and of X (q < 32)
  const int i = t >> 2, j0 = t & 3;
  for (int step = 0; step < p.steps; ++step) {
    float acc[32];
#pragma unroll
    for (int q = 0; q < 16; ++q) acc[q] = 0.0f;
    for (int k = 0; k < NSN; ++k) {  // A = X X^T
      const float xi = Xs[i * FXL + k];
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[q] = fmaf(xi, Xs[(j0 + 4 * q) * FXL + k], acc[q]);
    }
#pragma unroll
    for (int q = 0; q < 16; ++q) As[i * FAL + j0 + 4 * q] = acc[q];
    __syncthreads();
#pragma unroll
    for (int q = 0; q < 16; ++q) acc[q] = 0.0f;
    for (int k = 0; k < NSM; ++k) {  // A^2
      const float aik = As[i * FAL + k];
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[q] = fmaf(aik, As[k * FAL + j0 + 4 * q], acc[q]);
    }
#pragma unroll
    for (int q = 0; q < 16; ++q) acc[q] = fmaf(p.b, As[i * FAL + j0 + 4 * q], p.c * acc[q]);
    __syncthreads();  // every thread is done reading A
#pragma unroll
    for (int q = 0; q < 16; ++q) As[i * FAL + j0 + 4 * q] = acc[q];
    __syncthreads();
#pragma unroll
    for (int q = 0; q < 32; ++q) acc[q] = 0.0f;
    for (int k = 0; k < NSM; ++k) {  // B X
      const float bik = As[i * FAL + k];
#pragma unroll
      for (int q = 0; q < 32; ++q) acc[q] = fmaf(bik, Xs[k * FXL + j0 + 4 * q], acc[q]);
    }
#pragma unroll
    for (int q = 0; q < 32; ++q) acc[q] = fmaf(p.a, Xs[i * FXL + j0 + 4 * q], acc[q]);
    __syncthreads();  // every thread is done reading X
#pragma unroll
    for (int q = 0; q < 32; ++q) Xs[i * FXL + j0 + 4 * q] = acc[q];
    __syncthreads();
  }
  bool bad = false;
  for (int e = t; e < NSM * NSN; e += 256) {
    const int ii = e / NSN, jj = e % NSN;
    if (ii >= m || jj >= n) continue;
    const int gr = tr ? jj : ii, gc = tr ? ii : jj;
    const float v = Xs[ii * FXL + jj];
    if (!p.has_upd) {
      p.out[(int64_t)mat * rows * cols + (int64_t)gr * cols + gc] = v;
    } else {
      const NsUpdate& u = p.u;
      const int mem = mat / u.mats_per_mem;
      const int64_t el = (int64_t)mem * u.P + p.uoff[gi] + (int64_t)gr * cols + gc;
      const int64_t gk = (int64_t)mem * u.ld_gate + u.k;
      const float sn = u.eta[gk] * u.Sin[el] - u.theta[gk] * v;
      const float wn = (1.0f - u.alpha[gk]) * u.Win[el] + sn;
      u.Sout[el] = sn;
      u.Wout[el] = wn;
      bad |= !(isfinite(sn) && isfinite(wn));
    }
  }
  if (bad) p.u.flag[0] = 1;
}

bool ns_supported(int rows, int cols) {
  const int m = rows < cols ? rows : cols, n = rows < cols ? cols : rows;
  return m >= 1 && m <= NSM && n <= NSN;
}

atlasmem_status launch_ns(const float* G, int64_t ldG_mat, int n_mat, int rows, int cols, int steps, float a, float b,
                          float c, float eps, int prec, float* out, const NsUpdate* upd, hipStream_t st) {
  if (!ns_supported(rows, cols)) return ATLASMEM_E_UNSUPPORTED;
  if (n_mat == 0) return ATLASMEM_OK;
  NsArgs p;
  p.G = G;
  p.ldG = ldG_mat;
  p.rows = rows;
  p.cols = cols;
  p.steps = steps;
  p.a = a;
  p.b = b;
  p.c = c;
  p.eps = eps;
  p.out = out;
  p.has_upd = upd != nullptr;
  if (upd) p.u = *upd;
  else p.u = NsUpdate{};
  p.gsize = n_mat;
  p.grows[0] = rows;
  p.gcols[0] = cols;
  p.goff[0] = 0;
  p.uoff[0] = upd ? upd->off : 0;
  if (prec == 2) hipLaunchKernelGGL(ns_f32_kernel, dim3(n_mat), dim3(256), 0, st, p);
  else if (prec == 1) hipLaunchKernelGGL(ns_kernel<true>, dim3(n_mat), dim3(256), 0, st, p);
  else hipLaunchKernelGGL(ns_kernel<false>, dim3(n_mat), dim3(256), 0, st, p);
  AM_LAUNCH_CHECK();
  return ATLASMEM_OK;
}

atlasmem_status launch_ns_groups(const float* G, int64_t ldG_mat, int n_mat, int ngroups, const NsGroup* grp, int steps,
                                 float a, float b, float c, float eps, int prec, const NsUpdate& upd,
                                 hipStream_t st) {
  if (ngroups < 1 || ngroups > 3) return ATLASMEM_E_INVALID;
  for (int i = 0; i < ngroups; ++i)
    if (!ns_supported(grp[i].rows, grp[i].cols)) return ATLASMEM_E_UNSUPPORTED;
  if (n_mat == 0) return ATLASMEM_OK;
  NsArgs p;
  p.G = G;
  p.ldG = ldG_mat;
  p.rows = grp[0].rows;
  p.cols = grp[0].cols;
  p.steps = steps;
  p.a = a;
  p.b = b;
  p.c = c;
  p.eps = eps;
  p.out = nullptr;
  p.has_upd = 1;
  p.u = upd;
  p.gsize = n_mat;
  for (int i = 0; i < 3; ++i) {
    const NsGroup& q = grp[i < ngroups ? i : 0];
    p.grows[i] = q.rows;
    p.gcols[i] = q.cols;
    p.goff[i] = q.goff;
    p.uoff[i] = q.uoff;
  }
  const dim3 grid((unsigned)((int64_t)n_mat * ngroups));
  if (prec == 2) hipLaunchKernelGGL(ns_f32_kernel, grid, dim3(256), 0, st, p);
  else if (prec == 1) hipLaunchKernelGGL(ns_kernel<true>, grid, dim3(256), 0, st, p);
  else hipLaunchKernelGGL(ns_kernel<false>, grid, dim3(256), 0, st, p);
  AM_LAUNCH_CHECK();
  return ATLASMEM_OK;
}

}  // namespace am
