// 2-layer SiLU MLP memory, M_W(x) = W2 silu(W1 x): the chunk-wise update as batched
// matrix-core GEMMs over all memories.
//
// Per chunk [s, s + C) of every memory, with x = phi(k) over the Rk = C + c - 1 key rows
// (the chunk's keys and the c - 1 keys before it, for the Omega window) and the C query rows:
//   Z  = X W1^T              (keys and queries together)            GEMM "Z"
//   Yh = silu(Z) W2^T; key rows give D2 = 2 (Yh - V), query rows are the retrieved Y
//   Pm = D2 W2;  D1 = Pm * silu'(Z)                                   GEMM "P"
// then the weighted-gradient GEMMs, with no per-token gradient ever materialised:
//   per-token gates:  [diag(cW) D2; diag(cS) D2]^T silu(Z) and [diag(cW) D1; diag(cS) D1]^T X,
//                     whose epilogue writes W_end = beta W0 + a_S S0 - G^W, S_end = P S0 - G^S
//   per-chunk gates:  G2 = D2^T silu(Z), G1 = D1^T X, then (optionally Newton-Schulz) and
//                     S = eta_c S - theta_c G, W = (1 - alpha_c) W + S.
// Loss and gradient: titans-pytorch-mlx README, Core Equations, Eq. 12-14; matmul form of the
// summed gradient (delta^T @ activations): same page, MLX Optimizations, Gradient Computation.
// The coefficient vectors cW, cS and the chunk scalars come from the gate scan / Omega kernels.
#include "common.h"
#include "gemm.h"
#include "internal.h"

namespace am {

// ---------------------------------------------------------------------------- feature rows

// Rows [0, Rk) are key rows: token tau = s - (c - 1) + row of the call, from the window
// history when tau < 0.  Rows [Rk, nrows) are query rows: token s + row - Rk.
struct FeatRows {
  const void* K;
  const void* Q;
  int in_bf16;
  const float* hk;  // [M][c-1][dk] fp32
  int64_t T, s;  // T: token stride per memory of the row arrays
  int Rk, nrows;
  int c, dk, din, poly;
  int zdiv;

  __device__ __forceinline__ float raw(int mem, int row, int i) const {
    if (row < Rk) {
      const int64_t tau = s - (c - 1) + row;
      if (tau >= 0) return load_in(K, ((int64_t)mem * T + tau) * dk + i, in_bf16);
      return hk[((int64_t)mem * (c - 1) + (c - 1) + tau) * dk + i];
    }
    const int64_t tau = s + (row - Rk);
    return load_in(Q, ((int64_t)mem * T + tau) * dk + i, in_bf16);
  }
  __device__ __forceinline__ float feat(int mem, int row, int f) const {
    if (poly == 1) return raw(mem, row, f);
    if (f == 0) return 1.0f;
    if (f <= dk) return raw(mem, row, f - 1);
    int i, j;
    pair_of(f - 1 - dk, dk, i, j);
    return 0.5f * (raw(mem, row, i) * raw(mem, row, j));
  }
};

// A role: outer = row, k = feature.
struct FeatA {
  FeatRows fr;
  __device__ __forceinline__ void load8(int z, int row, int f0, float* v) const {
    const int mem = z / fr.zdiv;
    if (row >= fr.nrows) {
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = 0.0f;
      return;
    }
    if (fr.poly == 1) {
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = (f0 + u < fr.din) ? fr.raw(mem, row, f0 + u) : 0.0f;
      return;
    }
    // degree 2: walk the monomials from f0 (decode the first pair once, then step)
    int i = 0, j = 0;
    if (f0 > fr.dk) pair_of(f0 - 1 - fr.dk, fr.dk, i, j);
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int f = f0 + u;
      float x = 0.0f;
      if (f < fr.din) {
        if (f == 0) x = 1.0f;
        else if (f <= fr.dk) x = fr.raw(mem, row, f - 1);
        else {
          if (f == fr.dk + 1) { i = 0; j = 0; }
          x = 0.5f * (fr.raw(mem, row, i) * fr.raw(mem, row, j));
          if (++j == fr.dk) { ++i; j = i; }
        }
      }
      v[u] = x;
    }
  }
};

// B role: outer = feature, k = row.
struct FeatB {
  FeatRows fr;
  __device__ __forceinline__ void load8(int z, int f, int r0, float* v) const {
    const int mem = z / fr.zdiv;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int row = r0 + u;
      v[u] = (f < fr.din && row < fr.nrows) ? fr.feat(mem, row, f) : 0.0f;
    }
  }
};

// ---------------------------------------------------------------------------- epilogues

struct EpiStore {
  float* out;
  int64_t sz;
  int ld;
  int zdiv;
  __device__ __forceinline__ void operator()(int z, int row, int col, float v) const {
    out[(int64_t)(z / zdiv) * sz + (int64_t)row * ld + col] = v;
  }
};

// Key rows: D2 = 2 (Yh - v); query rows: retrieved output.
struct EpiY {
  float* D2;
  int64_t d2z;
  const void* V;
  int in_bf16;
  const float* hv;
  int64_t T, s;  // T: token stride per memory of the row arrays
  int Rk, c, dv;
  void* Y;
  int out_bf16;
  int residual;  // the residual memory adds its input: feature `col` of the same row
  FeatRows fr;   // the rows of the product (keys, then queries), for the residual input
  __device__ __forceinline__ void operator()(int z, int row, int col, float v) const {
    if (residual) v += fr.feat(z, row, col);
    if (row < Rk) {
      const int64_t tau = s - (c - 1) + row;
      const float vv = (tau >= 0) ? load_in(V, ((int64_t)z * T + tau) * dv + col, in_bf16)
                                  : hv[((int64_t)z * (c - 1) + (c - 1) + tau) * dv + col];
      D2[(int64_t)z * d2z + (int64_t)row * dv + col] = 2.0f * (v - vv);
    } else if (Y) {
      const int64_t yo = ((int64_t)z * T + s + (row - Rk)) * dv + col;
      if (out_bf16) ((uint16_t*)Y)[yo] = (uint16_t)bf16_bits(v);
      else ((float*)Y)[yo] = v;
    }
  }
};

// Per-token retrieval epilogues (rows = the chunk's queries t; bA = (beta_t, a_t)).
// Zq = beta_t Z0 + a_t ZS - acc, in place in ZS: Z0 = the chunk-start first-layer product of the
// queries (rows zr0.. of Z), ZS = their product with the chunk-start momentum.
struct EpiZq {
  float* ZS;
  const float* Z;
  const float* bA;
  int64_t zs_z, z_z, zr0;
  int dz, C;
  __device__ __forceinline__ void operator()(int z, int row, int col, float v) const {
    float* o = ZS + (int64_t)z * zs_z + (int64_t)row * dz + col;
    const float* b = bA + ((int64_t)z * C + row) * 2;
    *o = b[0] * Z[(int64_t)z * z_z + (zr0 + row) * dz + col] + b[1] * *o - v;
  }
};
// out = which-th coefficient of the row times acc (acc = 0) or added to out (acc = 1)
struct EpiRowMix {
  float* out;
  const float* bA;
  int64_t oz;
  int ld, C, which, add;
  __device__ __forceinline__ void operator()(int z, int row, int col, float v) const {
    float* o = out + (int64_t)z * oz + (int64_t)row * ld + col;
    const float x = bA[((int64_t)z * C + row) * 2 + which] * v;
    *o = add ? *o + x : x;
  }
};
// Y of the chunk's queries: the accumulated beta/a terms minus acc (plus the query's features for
// the residual memory)
struct EpiYptr {
  const float* YB;
  int64_t yb_z;
  int dv;
  int64_t ld, s;  // token stride of Y per memory, first token of the chunk
  void* Y;
  int out_bf16;
  int residual;
  FeatRows fr;    // the queries, for the residual input
  __device__ __forceinline__ void operator()(int z, int row, int col, float v) const {
    float y = YB[(int64_t)z * yb_z + (int64_t)row * dv + col] - v;
    if (residual) y += fr.feat(z, row, col);
    const int64_t yo = ((int64_t)z * ld + s + row) * dv + col;
    if (out_bf16) ((uint16_t*)Y)[yo] = (uint16_t)bf16_bits(y);
    else ((float*)Y)[yo] = y;
  }
};

// D1 = Pm * silu'(Z).  Gated memory (rows of Z and D1 hold [Z1 | Z3] and [D1 | D3]):
// D1 = Pm * Z3 * silu'(Z1), D3 = Pm * silu(Z1).
struct EpiP {
  float* D1;
  const float* Z;
  int64_t d1z, zz;
  int dh, dz, gated;
  __device__ __forceinline__ void operator()(int z, int row, int col, float v) const {
    const float* zr = Z + (int64_t)z * zz + (int64_t)row * dz;
    float* dr = D1 + (int64_t)z * d1z + (int64_t)row * dz;
    const float z1 = zr[col];
    if (gated) {
      const float z3 = zr[dh + col];
      dr[col] = v * z3 * silu_primef_(z1);
      dr[dh + col] = v * siluf_(z1);
    } else {
      dr[col] = v * silu_primef_(z1);
    }
  }
};

// Per-token gates: batch z = 2 mem + which; which 0 -> W_end, 1 -> S_end.
struct EpiUpdPair {
  const float* Win;
  const float* Sin;
  float* Wout;
  float* Sout;
  int64_t P, off;
  int ld;
  const float* scal;  // chunk scalars of this chunk: scal + mem * ld_s -> (P, beta, a_S)
  int64_t ld_s;
  int* flag;
  __device__ __forceinline__ void operator()(int z, int row, int col, float v) const {
    const int mem = z >> 1;
    const int64_t e = (int64_t)mem * P + off + (int64_t)row * ld + col;
    const float* sc = scal + (int64_t)mem * ld_s;
    float o;
    if ((z & 1) == 0) {
      o = sc[1] * Win[e] + sc[2] * Sin[e] - v;
      Wout[e] = o;
    } else {
      o = sc[0] * Sin[e] - v;
      Sout[e] = o;
    }
    if (!isfinite(o)) flag[0] = 1;
  }
};

// Per-chunk gates without orthogonalisation: S = eta S - theta G, W = (1 - alpha) W + S.
struct EpiUpdChunk {
  const float* Win;
  const float* Sin;
  float* Wout;
  float* Sout;
  int64_t P, off;
  int ld;
  const float* theta;
  const float* eta;
  const float* alpha;
  int64_t ld_gate, k;
  int* flag;
  __device__ __forceinline__ void operator()(int z, int row, int col, float v) const {
    const int64_t e = (int64_t)z * P + off + (int64_t)row * ld + col;
    const int64_t g = (int64_t)z * ld_gate + k;
    const float s = eta[g] * Sin[e] - theta[g] * v;
    const float w = (1.0f - alpha[g]) * Win[e] + s;
    Sout[e] = s;
    Wout[e] = w;
    if (!(isfinite(s) && isfinite(w))) flag[0] = 1;
  }
};

// ---------------------------------------------------------------------------- helpers

static StridedLoader strided(const float* base, int64_t sz, int64_t so, int64_t sk, int zdiv, int outer_dim, int K,
                             int xf = XF_NONE) {
  StridedLoader l;
  l.base = base;
  l.sz = sz;
  l.so = so;
  l.sk = sk;
  l.zdiv = zdiv;
  l.outer_dim = outer_dim;
  l.K = K;
  l.xf = xf;
  l.coef0 = l.coef1 = nullptr;
  l.cz = 0;
  l.scale = nullptr;
  l.gofs = 0;
  l.cld = 0;
  return l;
}

// The hidden activation H of the memory from the stored first-layer outputs: silu(Z) or, for the
// gated memory, silu(Z1) * Z3 with Z3 d_hidden elements after Z1.
static StridedLoader hidden(const Dims& d, const float* Z, int64_t sz, int64_t so, int64_t sk, int zdiv, int outer_dim,
                            int K) {
  StridedLoader l = strided(Z, sz, so, sk, zdiv, outer_dim, K, d.gated ? XF_GATED : XF_SILU);
  l.gofs = d.dh;
  return l;
}

template <class LA, class LB, class EP>
static void gemm_any(bool split, bool a_exact, bool b_exact, int M, int N, int K, int batch, const LA& la, const LB& lb,
                     const EP& ep, hipStream_t st) {
  if (a_exact && b_exact) launch_gemm<true, true>(split, M, N, K, batch, la, lb, ep, st);
  else if (a_exact) launch_gemm<true, false>(split, M, N, K, batch, la, lb, ep, st);
  else if (b_exact) launch_gemm<false, true>(split, M, N, K, batch, la, lb, ep, st);
  else launch_gemm<false, false>(split, M, N, K, batch, la, lb, ep, st);
}

static FeatRows feat_rows(const Handle* h, const void* K, const void* Q, int64_t ld, int64_t s, int Rk, int nrows,
                          int zdiv) {
  const Dims& d = h->d;
  FeatRows fr;
  fr.K = K;
  fr.Q = Q;
  fr.in_bf16 = d.in_bf16;
  fr.hk = h->hk[h->hcur];
  fr.T = ld;
  fr.s = s;
  fr.Rk = Rk;
  fr.nrows = nrows;
  fr.c = d.c;
  fr.dk = d.dk;
  fr.din = d.din;
  fr.poly = d.poly;
  fr.zdiv = zdiv;
  return fr;
}

// ---------------------------------------------------------------------------- per-token retrieval

// Queries of the chunk starting at token s answered from W_t, the state right after token t's
// update (Atlas-Torch README, "Known deviations from the paper's MAC": the post-update per-token
// state), without forming any W_t.  With W_t = beta_t W0 + a_t S0 - sum_i Om[t][i] g_i (the
// coefficients of launch_ptr_coeffs) and the MLP gradients g_i = (D1_i x_i^T, D2_i h_i^T) that the
// update has just formed at the chunk-start weights:
//   Zq_t = beta_t (W0_1 q_t) + a_t (S0_1 q_t) - sum_i Om[t][i] (x_i . q_t) D1_i
//   y_t  = beta_t (W0_2 Hq_t) + a_t (S0_2 Hq_t) - sum_i Om[t][i] (h_i . Hq_t) D2_i,  Hq = H(Zq)
// i.e. masked query-key score products, as in attention.  The gated memory's first layer is the
// [W1; W3] block throughout.
static atlasmem_status ptr_retrieve(Handle* h, const Dims& d, const void* K, const void* Q, const float* theta,
                                    const float* eta, const float* alpha, const float* gamma, int64_t ld, int64_t s,
                                    const float* Win, const float* Sin, void* Y, hipStream_t st) {
  const int M = d.M, C = d.C, Rk = d.Rk, dh = d.dh, dv = d.dv, din = d.din, dz = d.dz;
  const bool split = d.split, feat_exact = d.poly == 1 && d.in_bf16;
  const int64_t zsz = (int64_t)d.Rt * dz, qz = (int64_t)C * dz, az = (int64_t)C * Rk, yz = (int64_t)C * dv;
  atlasmem_status stt = launch_ptr_coeffs(theta, eta, alpha, gamma, ld, h->hg[h->hcur], M, s, C, d.c, h->pbA,
                                          h->pOm, st);
  if (stt != ATLASMEM_OK) return stt;
  const FeatRows qrows = feat_rows(h, nullptr, Q, ld, s, 0, C, 1);
  // ZS = Q S0_1^T
  {
    FeatA la{qrows};
    StridedLoader lb = strided(Sin, d.P, din, 1, 1, dz, din);
    EpiStore ep{h->pZS, qz, dz, 1};
    gemm_any(split, feat_exact, false, C, dz, din, M, la, lb, ep, st);
  }
  // scores A1[t][r] = q_t . x_r over the key rows (window history included)
  {
    FeatA la{qrows};
    FeatA lb{feat_rows(h, K, Q, ld, s, Rk, Rk, 1)};
    EpiStore ep{h->pA1, az, Rk, 1};
    gemm_any(split, feat_exact, feat_exact, C, Rk, din, M, la, lb, ep, st);
  }
  // Zq = beta Z0 + a ZS - (Om * A1) D1
  {
    StridedLoader la = strided(h->pA1, az, Rk, 1, 1, C, Rk, XF_MAT);
    la.coef0 = h->pOm;
    la.cz = az;
    la.cld = Rk;
    StridedLoader lb = strided(h->D1, (int64_t)Rk * dz, 1, dz, 1, dz, Rk);  // B(k=r, j) = D1[r][j]
    EpiZq ep{h->pZS, h->Z, h->pbA, qz, zsz, (int64_t)Rk, dz, C};
    gemm_any(split, false, false, C, dz, Rk, M, la, lb, ep, st);
  }
  // scores A2[t][r] = Hq_t . h_r
  {
    StridedLoader la = hidden(d, h->pZS, qz, dz, 1, 1, C, dh);
    StridedLoader lb = hidden(d, h->Z, zsz, dz, 1, 1, Rk, dh);  // B(k=h, j=r) = H[r][h]
    EpiStore ep{h->pA1, az, Rk, 1};
    gemm_any(split, false, false, C, Rk, dh, M, la, lb, ep, st);
  }
  // YB = beta Hq W0_2^T + a Hq S0_2^T
  for (int which = 0; which < 2; ++which) {
    StridedLoader la = hidden(d, h->pZS, qz, dz, 1, 1, C, dh);
    StridedLoader lb = strided((which ? Sin : Win) + d.P1, d.P, dh, 1, 1, dv, dh);  // B(k=h, j=v) = W2[v][h]
    EpiRowMix ep{h->pYB, h->pbA, yz, dv, C, which, which};
    gemm_any(split, false, false, C, dv, dh, M, la, lb, ep, st);
  }
  // Y = YB - (Om * A2) D2 (+ the query's features for the residual memory)
  {
    StridedLoader la = strided(h->pA1, az, Rk, 1, 1, C, Rk, XF_MAT);
    la.coef0 = h->pOm;
    la.cz = az;
    la.cld = Rk;
    StridedLoader lb = strided(h->D2, (int64_t)Rk * dv, 1, dv, 1, dv, Rk);  // B(k=r, j=v) = D2[r][v]
    EpiYptr ep{h->pYB, yz, dv, ld, s, Y, d.out_bf16, d.residual, qrows};
    gemm_any(split, false, false, C, dv, Rk, M, la, lb, ep, st);
  }
  return ATLASMEM_OK;
}

// ---------------------------------------------------------------------------- one call

atlasmem_status mlp_update(Handle* h, const Dims& d, const void* K, const void* Q, const void* V, const float* theta,
                           const float* eta, const float* alpha, const float* gamma, const Span& sp, void* Y,
                           hipStream_t st) {
  const int64_t T = sp.T, ld = sp.ld;
  const int M = d.M, C = d.C, c = d.c, Rk = d.Rk, dh = d.dh, dv = d.dv, din = d.din, dz = d.dz;
  const bool split = d.split;
  const bool feat_exact = d.poly == 1 && d.in_bf16;
  const int64_t nchunks = T / C;
  const int nq = Y ? C : 0;
  const int nrows = Rk + nq;
  const int64_t zsz = (int64_t)d.Rt * dz;
  const bool per_token = d.gate_mode == ATLASMEM_PER_TOKEN;
  atlasmem_status stt;
  if (!d.no_fused && fused_supported(d)) return launch_fused(h, d, K, Q, V, theta, eta, alpha, sp, Y, st);

  for (int64_t kb0 = 0; kb0 < nchunks; kb0 += h->ncb) {
    const int nb = (int)((nchunks - kb0) < h->ncb ? (nchunks - kb0) : h->ncb);
    if (per_token) {
      stt = launch_gate_scan(theta, eta, alpha, M, ld, kb0 * C, nb, C, h->cW, h->cS, (int64_t)h->ncb * C, h->scal,
                             (int64_t)h->ncb * 3, st);
      if (stt != ATLASMEM_OK) return stt;
      if (c > 1) {
        stt = launch_omega(h->cW, h->cS, (int64_t)h->ncb * C, gamma, ld, h->hg[h->hcur], M, kb0 * C, nb, C, c, h->oW,
                           h->oS, (int64_t)h->ncb * Rk, st);
        if (stt != ATLASMEM_OK) return stt;
      }
    }
    for (int kb = 0; kb < nb; ++kb) {
      const int64_t k = kb0 + kb;
      const int64_t s = k * C;
      const float* Win = h->W[h->cur];
      const float* Sin = h->S[h->cur];
      float* Wout = h->W[1 - h->cur];
      float* Sout = h->S[1 - h->cur];
      const float* W1 = Win;
      const float* W2 = Win + d.P1;

      // Z = X W1^T over key rows (+ query rows); gated: [Z1 | Z3] = X [W1; W3]^T
      {
        FeatA la{feat_rows(h, K, Q, ld, s, Rk, nrows, 1)};
        StridedLoader lb = strided(W1, d.P, din, 1, 1, dz, din);  // B(k=f, j=h) = W1[h][f]
        EpiStore ep{h->Z, zsz, dz, 1};
        gemm_any(split, feat_exact, false, nrows, dz, din, M, la, lb, ep, st);
      }
      // Yh = H W2^T -> D2 (key rows), Y (query rows; with per-token retrieval they are answered
      // below from the per-token states instead)
      const int yrows = d.ptr ? Rk : nrows;
      {
        StridedLoader la = hidden(d, h->Z, zsz, dz, 1, 1, yrows, dh);
        StridedLoader lb = strided(W2, d.P, dh, 1, 1, dv, dh);  // B(k=h, j=v) = W2[v][h]
        EpiY ep{h->D2, (int64_t)Rk * dv, V, d.in_bf16, h->hv[h->hcur], ld, s, Rk, c, dv, Y, d.out_bf16,
                d.residual, feat_rows(h, K, Q, ld, s, Rk, nrows, 1)};
        gemm_any(split, false, false, yrows, dv, dh, M, la, lb, ep, st);
      }
      // Pm = D2 W2 -> D1 = Pm * silu'(Z)
      {
        StridedLoader la = strided(h->D2, (int64_t)Rk * dv, dv, 1, 1, Rk, dv);
        StridedLoader lb = strided(W2, d.P, 1, dh, 1, dh, dv);  // B(k=v, j=h) = W2[v][h]
        EpiP ep{h->D1, h->Z, (int64_t)Rk * dz, zsz, dh, dz, d.gated};
        gemm_any(split, false, false, Rk, dh, dv, M, la, lb, ep, st);
      }
      if (per_token) {
        const float* c0 = (c > 1) ? h->oW + (int64_t)kb * Rk : h->cW + (int64_t)kb * C;
        const float* c1 = (c > 1) ? h->oS + (int64_t)kb * Rk : h->cS + (int64_t)kb * C;
        const int64_t cz = (c > 1) ? (int64_t)h->ncb * Rk : (int64_t)h->ncb * C;
        const float* sc = h->scal + (int64_t)kb * 3;
        // W2 pair: A(i=v, k=row) = D2[row][v] * coef[row], B(k=row, j=h) = H[row][h]
        {
          StridedLoader la = strided(h->D2, (int64_t)Rk * dv, 1, dv, 2, dv, Rk, XF_COEF);
          la.coef0 = c0;
          la.coef1 = c1;
          la.cz = cz;
          StridedLoader lb = hidden(d, h->Z, zsz, 1, dz, 2, dh, Rk);
          EpiUpdPair ep{Win, Sin, Wout, Sout, d.P, d.P1, dh, sc, (int64_t)h->ncb * 3, h->flag};
          gemm_any(split, false, false, dv, dh, Rk, 2 * M, la, lb, ep, st);
        }
        // W1 pair (gated: W1 and W3 as one block of 2 d_hidden rows): A(i=h, k=row) =
        // D1[row][h] * coef[row], B(k=row, j=f) = X[row][f]
        {
          StridedLoader la = strided(h->D1, (int64_t)Rk * dz, 1, dz, 2, dz, Rk, XF_COEF);
          la.coef0 = c0;
          la.coef1 = c1;
          la.cz = cz;
          FeatB lb{feat_rows(h, K, Q, ld, s, Rk, Rk, 2)};
          EpiUpdPair ep{Win, Sin, Wout, Sout, d.P, 0, din, sc, (int64_t)h->ncb * 3, h->flag};
          gemm_any(split, false, feat_exact, dz, din, Rk, 2 * M, la, lb, ep, st);
        }
      } else if (d.ns_steps == 0) {
        {
          StridedLoader la = strided(h->D2, (int64_t)Rk * dv, 1, dv, 1, dv, Rk);
          StridedLoader lb = hidden(d, h->Z, zsz, 1, dz, 1, dh, Rk);
          EpiUpdChunk ep{Win, Sin, Wout, Sout, d.P, d.P1, dh, theta, eta, alpha, sp.ldg, k, h->flag};
          gemm_any(split, false, false, dv, dh, Rk, M, la, lb, ep, st);
        }
        {
          StridedLoader la = strided(h->D1, (int64_t)Rk * dz, 1, dz, 1, dz, Rk);
          FeatB lb{feat_rows(h, K, Q, ld, s, Rk, Rk, 1)};
          EpiUpdChunk ep{Win, Sin, Wout, Sout, d.P, 0, din, theta, eta, alpha, sp.ldg, k, h->flag};
          gemm_any(split, false, feat_exact, dz, din, Rk, M, la, lb, ep, st);
        }
      } else {
        {
          StridedLoader la = strided(h->D2, (int64_t)Rk * dv, 1, dv, 1, dv, Rk);
          StridedLoader lb = hidden(d, h->Z, zsz, 1, dz, 1, dh, Rk);
          EpiStore ep{h->G + d.P1, d.P, dh, 1};
          gemm_any(split, false, false, dv, dh, Rk, M, la, lb, ep, st);
        }
        {
          StridedLoader la = strided(h->D1, (int64_t)Rk * dz, 1, dz, 1, dz, Rk);
          FeatB lb{feat_rows(h, K, Q, ld, s, Rk, Rk, 1)};
          EpiStore ep{h->G, d.P, din, 1};
          gemm_any(split, false, feat_exact, dz, din, Rk, M, la, lb, ep, st);
        }
        // each weight matrix separately: W1, (W3,) W2
        NsUpdate u1{Win, Sin, Wout, Sout, d.P, 0, 1, theta, eta, alpha, sp.ldg, k, h->flag};
        stt = launch_ns(h->G, d.P, M, dh, din, d.ns_steps, d.ns_a, d.ns_b, d.ns_c, d.ns_eps, split, nullptr, &u1, st);
        if (stt != ATLASMEM_OK) return stt;
        if (d.gated) {
          const int64_t o3 = (int64_t)dh * din;
          NsUpdate u3{Win, Sin, Wout, Sout, d.P, o3, 1, theta, eta, alpha, sp.ldg, k, h->flag};
          stt = launch_ns(h->G + o3, d.P, M, dh, din, d.ns_steps, d.ns_a, d.ns_b, d.ns_c, d.ns_eps, split, nullptr,
                          &u3, st);
          if (stt != ATLASMEM_OK) return stt;
        }
        NsUpdate u2{Win, Sin, Wout, Sout, d.P, d.P1, 1, theta, eta, alpha, sp.ldg, k, h->flag};
        stt = launch_ns(h->G + d.P1, d.P, M, dv, dh, d.ns_steps, d.ns_a, d.ns_b, d.ns_c, d.ns_eps, split, nullptr,
                        &u2, st);
        if (stt != ATLASMEM_OK) return stt;
      }
      if (d.ptr && Y) {
        stt = ptr_retrieve(h, d, K, Q, theta, eta, alpha, gamma, ld, s, Win, Sin, Y, st);
        if (stt != ATLASMEM_OK) return stt;
      }
      AM_LAUNCH_CHECK();
      h->cur = 1 - h->cur;
    }
  }
  stt = launch_history_update(h, K, V, gamma, T, ld, st);
  if (stt != ATLASMEM_OK) return stt;
  if (c > 1 && T > 0) h->hcur = 1 - h->hcur;
  return ATLASMEM_OK;
}

atlasmem_status mlp_retrieve(Handle* h, const void* Q, int64_t T, int64_t ld, void* Y, hipStream_t st) {
  const Dims& d = h->d;
  const int M = d.M, dh = d.dh, dv = d.dv, din = d.din, dz = d.dz;
  const bool feat_exact = d.poly == 1 && d.in_bf16;
  const float* W1 = h->W[h->cur];
  const float* W2 = W1 + d.P1;
  const int64_t zsz = (int64_t)h->rb * dz;
  for (int64_t s = 0; s < T; s += h->rb) {
    const int rows = (int)((T - s) < h->rb ? (T - s) : h->rb);
    {
      FeatA la{feat_rows(h, nullptr, Q, ld, s, 0, rows, 1)};
      StridedLoader lb = strided(W1, d.P, din, 1, 1, dz, din);
      EpiStore ep{h->Zr, zsz, dz, 1};
      gemm_any(d.split, feat_exact, false, rows, dz, din, M, la, lb, ep, st);
    }
    {
      StridedLoader la = hidden(d, h->Zr, zsz, dz, 1, 1, rows, dh);
      StridedLoader lb = strided(W2, d.P, dh, 1, 1, dv, dh);
      EpiY ep{nullptr, 0, nullptr, d.in_bf16, nullptr, ld, s, 0, d.c, dv, Y, d.out_bf16, d.residual,
              feat_rows(h, nullptr, Q, ld, s, 0, rows, 1)};
      gemm_any(d.split, false, false, rows, dv, dh, M, la, lb, ep, st);
    }
    AM_LAUNCH_CHECK();
  }
  return ATLASMEM_OK;
}

}  // namespace am
