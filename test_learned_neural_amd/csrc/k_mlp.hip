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
#include "conv_rows.h"
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

  // Batched loads (FeatA, FeatB): the source of a row is located first, then every load of a
  // call is issued as raw bits before any is converted, so that the loads overlap.
  // Row `row` (< nrows): element i at src[off + i] (K or Q), or, for a key row before the call's
  // first token, at hk[hoff + i] (hist).
  __device__ __forceinline__ void locate(int mem, int row, const void*& src, int64_t& off, int64_t& hoff,
                                         bool& hist) const {
    if (row < Rk) {
      const int64_t tau = s - (c - 1) + row;
      hist = tau < 0;
      src = K;
      off = ((int64_t)mem * T + (hist ? 0 : tau)) * dk;
      hoff = hist ? ((int64_t)mem * (c - 1) + (c - 1) + tau) * dk : 0;
    } else {
      hist = false;
      src = Q;
      off = ((int64_t)mem * T + s + (row - Rk)) * dk;
      hoff = 0;
    }
  }
  // whether any row of this chunk comes from the window history (uniform)
  __device__ __forceinline__ bool any_hist() const { return c > 1 && s < c - 1; }
  __device__ __forceinline__ uint32_t ld_bits(const void* src, int64_t idx) const {
    return in_bf16 ? (uint32_t)((const uint16_t*)src)[idx] : __float_as_uint(((const float*)src)[idx]);
  }
  __device__ __forceinline__ float bits_val(uint32_t b) const {
    return in_bf16 ? __uint_as_float(b << 16) : __uint_as_float(b);
  }
};

// Feature f of the map: 0 the constant, 1 a raw element (index i), 2 half the product of
// elements i and j, 3 padding beyond din.
__device__ __forceinline__ int feat_kind(const FeatRows& fr, int f, int& i, int& j) {
  if (f >= fr.din) {
    i = j = 0;
    return 3;
  }
  if (fr.poly == 1) {
    i = j = f;
    return 1;
  }
  if (f == 0) {
    i = j = 0;
    return 0;
  }
  if (f <= fr.dk) {
    i = j = f - 1;
    return 1;
  }
  pair_of(f - 1 - fr.dk, fr.dk, i, j);
  return 2;
}

__device__ __forceinline__ float feat_value(int kind, float xi, float xj) {
  return kind == 0 ? 1.0f : kind == 1 ? xi : kind == 2 ? 0.5f * (xi * xj) : 0.0f;
}

// A role: outer = row, k = feature.
struct FeatA {
  FeatRows fr;
  __device__ __forceinline__ void load8(int z, int row, int f0, float* v) const {
    const int mem = z / fr.zdiv;
    const bool rok = row < fr.nrows;
    const void* src;
    int64_t off, hoff;
    bool hist;
    fr.locate(mem, rok ? row : 0, src, off, hoff, hist);
    const bool hh = fr.any_hist();
    if (fr.poly == 1 && fr.in_bf16 && !hh && f0 + 8 <= fr.din &&
        (((uintptr_t)((const uint16_t*)src + off + f0)) & 15) == 0) {
      // eight consecutive bf16 of one row: a single 16-byte load
      const u32x4 w4 = *(const u32x4*)((const uint16_t*)src + off + f0);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        v[2 * q] = rok ? __uint_as_float(w4[q] << 16) : 0.0f;
        v[2 * q + 1] = rok ? __uint_as_float(w4[q] & 0xFFFF0000u) : 0.0f;
      }
      return;
    }
    int kind[8], ia[8], ja[8];
    if (fr.poly == 1 || f0 + 8 <= fr.dk + 1) {
#pragma unroll
      for (int u = 0; u < 8; ++u) kind[u] = feat_kind(fr, f0 + u, ia[u], ja[u]);
    } else {
      // degree 2: decode the first pair once, then step through the monomials
      int i = 0, j = 0;
      if (f0 > fr.dk) pair_of(f0 - 1 - fr.dk, fr.dk, i, j);
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int f = f0 + u;
        if (f >= fr.din) {
          kind[u] = 3;
          ia[u] = ja[u] = 0;
        } else if (f == 0) {
          kind[u] = 0;
          ia[u] = ja[u] = 0;
        } else if (f <= fr.dk) {
          kind[u] = 1;
          ia[u] = ja[u] = f - 1;
        } else {
          if (f == fr.dk + 1) i = j = 0;
          kind[u] = 2;
          ia[u] = i;
          ja[u] = j;
          if (++j == fr.dk) {
            ++i;
            j = i;
          }
        }
      }
    }
    uint32_t bi[8], bj[8];
    float hi[8], hj[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      bi[u] = fr.ld_bits(src, off + ia[u]);
      bj[u] = fr.poly == 2 ? fr.ld_bits(src, off + ja[u]) : 0u;
      if (hh) {
        hi[u] = fr.hk[hoff + ia[u]];
        hj[u] = fr.hk[hoff + ja[u]];
      }
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      float xi = fr.bits_val(bi[u]), xj = fr.bits_val(bj[u]);
      if (hh && hist) {
        xi = hi[u];
        xj = hj[u];
      }
      v[u] = rok ? feat_value(kind[u], xi, xj) : 0.0f;
    }
  }
};

// B role: outer = feature, k = row.
struct FeatB {
  FeatRows fr;
  __device__ __forceinline__ void load8(int z, int f, int r0, float* v) const {
    const int mem = z / fr.zdiv;
    int i, j;
    const int kind = feat_kind(fr, f, i, j);
    const bool hh = fr.any_hist();
    if (!hh && r0 + 8 <= fr.nrows && (r0 + 8 <= fr.Rk || r0 >= fr.Rk)) {
      // eight consecutive rows of one array (K or Q): one base, a 32-bit row stride; the
      // feature's monomial (i, j) is the same for all eight
      const void* src;
      int64_t off, hoff;
      bool hist;
      fr.locate(mem, r0, src, off, hoff, hist);
      const int st = fr.dk;
      uint32_t bi[8], bj[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        bi[u] = fr.ld_bits(src, off + i + (int64_t)(u * st));
        bj[u] = kind == 2 ? fr.ld_bits(src, off + j + (int64_t)(u * st)) : 0u;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = feat_value(kind, fr.bits_val(bi[u]), fr.bits_val(bj[u]));
      return;
    }
    uint32_t bi[8], bj[8];
    float hi[8], hj[8];
    bool hist[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int row = r0 + u;
      const void* src;
      int64_t off, hoff;
      fr.locate(mem, row < fr.nrows ? row : 0, src, off, hoff, hist[u]);
      bi[u] = fr.ld_bits(src, off + i);
      bj[u] = fr.poly == 2 ? fr.ld_bits(src, off + j) : 0u;
      if (hh) {
        hi[u] = fr.hk[hoff + i];
        hj[u] = fr.hk[hoff + j];
      }
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      float xi = fr.bits_val(bi[u]), xj = fr.bits_val(bj[u]);
      if (hh && hist[u]) {
        xi = hi[u];
        xj = hj[u];
      }
      v[u] = (r0 + u < fr.nrows) ? feat_value(kind, xi, xj) : 0.0f;
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
  struct Pre {
    float vv, res;  // the key row's value, the residual input
  };
  __device__ __forceinline__ Pre load(int z, int row, int col) const {
    Pre p{0.0f, 0.0f};
    if (residual) p.res = fr.feat(z, row, col);
    if (row < Rk) {
      const int64_t tau = s - (c - 1) + row;
      p.vv = (tau >= 0) ? load_in(V, ((int64_t)z * T + tau) * dv + col, in_bf16)
                        : hv[((int64_t)z * (c - 1) + (c - 1) + tau) * dv + col];
    }
    return p;
  }
  __device__ __forceinline__ void store(int z, int row, int col, float v, const Pre& p) const {
    if (residual) v += p.res;
    if (row < Rk) {
      D2[(int64_t)z * d2z + (int64_t)row * dv + col] = 2.0f * (v - p.vv);
    } else if (Y) {
      const int64_t yo = ((int64_t)z * T + s + (row - Rk)) * dv + col;
      if (out_bf16) ((uint16_t*)Y)[yo] = (uint16_t)bf16_bits(v);
      else ((float*)Y)[yo] = v;
    }
  }
};

// ---------------------------------------------------------------------------- convolved rows
//
// The rows of a call to atlasmem_update_chunked_conv: K, Q, V hold raw rows that are convolved as
// they are read (conv_rows.h); the window history rows are already convolved.  Separate types, so
// that the plain loaders above keep their code.
struct ConvRows {
  FeatRows fr;
  ConvTensor ck, cq, cv;
  __device__ __forceinline__ float raw(int mem, int row, int i) const {
    if (row < fr.Rk) {
      const int64_t tau = fr.s - (fr.c - 1) + row;
      if (tau >= 0) return ck.at(mem, fr.T, tau, i);
      return fr.hk[((int64_t)mem * (fr.c - 1) + (fr.c - 1) + tau) * fr.dk + i];
    }
    return cq.at(mem, fr.T, fr.s + (row - fr.Rk), i);
  }
  __device__ __forceinline__ float feat(int mem, int row, int f) const {
    if (f >= fr.din) return 0.0f;
    if (fr.poly == 1) return raw(mem, row, f);
    if (f == 0) return 1.0f;
    if (f <= fr.dk) return raw(mem, row, f - 1);
    int i, j;
    pair_of(f - 1 - fr.dk, fr.dk, i, j);
    return 0.5f * (raw(mem, row, i) * raw(mem, row, j));
  }
};
// Eight convolved elements at once: channels i0..i0+7 of token tau (eight consecutive bf16 per row,
// one 16-byte load per tap row), or channel i of tokens tau0..tau0+7 (a sliding window over eleven
// rows).  Same multiply-adds in the same order as ConvTensor::at.
__device__ __forceinline__ void conv_row8(const ConvTensor& ct, int m, int64_t ld, int64_t tau, int i0, float* v) {
  const int h = m % ct.heads;
  uint32_t w[4][4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int64_t t2 = tau - 3 + j;
    const uint16_t* src = t2 >= 0 ? (const uint16_t*)ct.X + ((int64_t)m * ld + t2) * ct.d + i0
                                  : (const uint16_t*)ct.hist + ((int64_t)m * 3 + 3 + t2) * ct.d + i0;
    const u32x4 q = *(const u32x4*)src;
#pragma unroll
    for (int p = 0; p < 4; ++p) w[j][p] = q[p];
  }
  const float4* tp = (const float4*)(ct.taps + ((int64_t)h * ct.d + i0) * 4);
  const float sc = ct.inv ? ct.inv[(int64_t)m * ct.ninv + (tau - ct.t0)] : 1.0f;
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const float4 t4 = tp[u];
    float x[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) x[j] = __uint_as_float((u & 1) ? (w[j][u >> 1] & 0xFFFF0000u) : (w[j][u >> 1] << 16));
    float acc = ct.bias ? ct.bias[(int64_t)h * ct.d + i0 + u] : 0.0f;
    acc = fmaf(t4.x, x[0], acc);
    acc = fmaf(t4.y, x[1], acc);
    acc = fmaf(t4.z, x[2], acc);
    acc = fmaf(t4.w, x[3], acc);
    if (ct.inv) acc *= sc;
    v[u] = bf16_value(bf16_bits(acc));
  }
}
__device__ __forceinline__ void conv_col8(const ConvTensor& ct, int m, int64_t ld, int64_t tau0, int i, float* v) {
  const int h = m % ct.heads;
  float x[11];
#pragma unroll
  for (int r = 0; r < 11; ++r) {
    const int64_t t2 = tau0 - 3 + r;
    x[r] = t2 >= 0 ? load_in(ct.X, ((int64_t)m * ld + t2) * ct.d + i, ct.in_bf16)
                   : load_in(ct.hist, ((int64_t)m * 3 + 3 + t2) * ct.d + i, ct.in_bf16);
  }
  const float4 t4 = *(const float4*)(ct.taps + ((int64_t)h * ct.d + i) * 4);
  const float b = ct.bias ? ct.bias[(int64_t)h * ct.d + i] : 0.0f;
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    float acc = b;
    acc = fmaf(t4.x, x[u], acc);
    acc = fmaf(t4.y, x[u + 1], acc);
    acc = fmaf(t4.z, x[u + 2], acc);
    acc = fmaf(t4.w, x[u + 3], acc);
    if (ct.inv) acc *= ct.inv[(int64_t)m * ct.ninv + (tau0 + u - ct.t0)];
    v[u] = ct.in_bf16 ? bf16_value(bf16_bits(acc)) : acc;
  }
}

struct FeatAConv {
  ConvRows cr;
  __device__ __forceinline__ void load8(int z, int row, int f0, float* v) const {
    const FeatRows& fr = cr.fr;
    const int mem = z / fr.zdiv;
    const bool rok = row < fr.nrows;
    if (rok && fr.poly == 1 && fr.in_bf16 && (fr.dk & 7) == 0 && f0 + 8 <= fr.din) {
      const bool key = row < fr.Rk;
      const int64_t tau = key ? fr.s - (fr.c - 1) + row : fr.s + (row - fr.Rk);
      const ConvTensor& ct = key ? cr.ck : cr.cq;
      if (tau >= 0 && (((uintptr_t)ct.X) & 15) == 0) {  // rows of dk bf16 (dk % 8 == 0): 16-byte aligned
        conv_row8(ct, mem, fr.T, tau, f0, v);
        return;
      }
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = rok ? cr.feat(mem, row, f0 + u) : 0.0f;
  }
};
struct FeatBConv {
  ConvRows cr;
  __device__ __forceinline__ void load8(int z, int f, int r0, float* v) const {
    const FeatRows& fr = cr.fr;
    const int mem = z / fr.zdiv;
    if (fr.poly == 1 && f < fr.din && r0 + 8 <= fr.Rk && fr.s - (fr.c - 1) + r0 >= 0) {
      conv_col8(cr.ck, mem, fr.T, fr.s - (fr.c - 1) + r0, f, v);  // eight key rows of this call
      return;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = (r0 + u < fr.nrows) ? cr.feat(mem, r0 + u, f) : 0.0f;
  }
};
// EpiY on convolved rows: the key row's value and the residual input come from the convolution.
// One element at a time (no two-phase gather): each value is a short chain of loads and
// multiply-adds, and gathering sixteen of them at once spills.
struct EpiYConv {
  float* D2;
  int64_t d2z;
  const float* hv;
  int64_t s;
  int Rk, c, dv;
  void* Y;
  int out_bf16;
  int residual;
  ConvRows cr;
  __device__ __forceinline__ void operator()(int z, int row, int col, float v) const {
    if (residual) v += cr.feat(z, row, col);
    if (row < Rk) {
      const int64_t tau = s - (c - 1) + row;
      const float vv = (tau >= 0) ? cr.cv.at(z, cr.fr.T, tau, col) : hv[((int64_t)z * (c - 1) + (c - 1) + tau) * dv + col];
      D2[(int64_t)z * d2z + (int64_t)row * dv + col] = 2.0f * (v - vv);
    } else if (Y) {
      const int64_t yo = ((int64_t)z * cr.fr.T + s + (row - Rk)) * dv + col;
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
  struct Pre {
    float b0, b1, z0, zs;
  };
  __device__ __forceinline__ Pre load(int z, int row, int col) const {
    const float* b = bA + ((int64_t)z * C + row) * 2;
    return Pre{b[0], b[1], Z[(int64_t)z * z_z + (zr0 + row) * dz + col], ZS[(int64_t)z * zs_z + (int64_t)row * dz + col]};
  }
  __device__ __forceinline__ void store(int z, int row, int col, float v, const Pre& p) const {
    ZS[(int64_t)z * zs_z + (int64_t)row * dz + col] = p.b0 * p.z0 + p.b1 * p.zs - v;
  }
};
// out = which-th coefficient of the row times acc (acc = 0) or added to out (acc = 1)
struct EpiRowMix {
  float* out;
  const float* bA;
  int64_t oz;
  int ld, C, which, add;
  struct Pre {
    float coef, old;
  };
  __device__ __forceinline__ Pre load(int z, int row, int col) const {
    return Pre{bA[((int64_t)z * C + row) * 2 + which], add ? out[(int64_t)z * oz + (int64_t)row * ld + col] : 0.0f};
  }
  __device__ __forceinline__ void store(int z, int row, int col, float v, const Pre& p) const {
    const float x = p.coef * v;
    out[(int64_t)z * oz + (int64_t)row * ld + col] = add ? p.old + x : x;
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
  struct Pre {
    float yb, res;
  };
  __device__ __forceinline__ Pre load(int z, int row, int col) const {
    return Pre{YB[(int64_t)z * yb_z + (int64_t)row * dv + col], residual ? fr.feat(z, row, col) : 0.0f};
  }
  __device__ __forceinline__ void store(int z, int row, int col, float v, const Pre& p) const {
    float y = p.yb - v;
    if (residual) y += p.res;
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
  struct Pre {
    float z1, z3;
  };
  __device__ __forceinline__ Pre load(int z, int row, int col) const {
    const float* zr = Z + (int64_t)z * zz + (int64_t)row * dz;
    return Pre{zr[col], gated ? zr[dh + col] : 0.0f};
  }
  __device__ __forceinline__ void store(int z, int row, int col, float v, const Pre& p) const {
    float* dr = D1 + (int64_t)z * d1z + (int64_t)row * dz;
    const float z1 = p.z1;
    if (gated) {
      const float z3 = p.z3;
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
  struct Pre {
    float s0, s1, s2, w, s;  // chunk scalars, W and S at the element
  };
  __device__ __forceinline__ Pre load(int z, int row, int col) const {
    const int mem = z >> 1;
    const int64_t e = (int64_t)mem * P + off + (int64_t)row * ld + col;
    const float* sc = scal + (int64_t)mem * ld_s;
    return Pre{sc[0], sc[1], sc[2], (z & 1) == 0 ? Win[e] : 0.0f, Sin[e]};
  }
  __device__ __forceinline__ void store(int z, int row, int col, float v, const Pre& p) const {
    const int mem = z >> 1;
    const int64_t e = (int64_t)mem * P + off + (int64_t)row * ld + col;
    float o;
    // explicit fused multiply-adds: every kernel that inlines this epilogue (the per-product
    // launches and the chunk loop) rounds alike, whatever the compiler would contract
    if ((z & 1) == 0) {
      o = fmaf(p.s1, p.w, fmaf(p.s2, p.s, -v));
      Wout[e] = o;
    } else {
      o = fmaf(p.s0, p.s, -v);
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
  struct Pre {
    float et, th, al, w, s;  // the chunk's gates, W and S at the element
  };
  __device__ __forceinline__ Pre load(int z, int row, int col) const {
    const int64_t e = (int64_t)z * P + off + (int64_t)row * ld + col;
    const int64_t g = (int64_t)z * ld_gate + k;
    return Pre{eta[g], theta[g], alpha[g], Win[e], Sin[e]};
  }
  __device__ __forceinline__ void store(int z, int row, int col, float v, const Pre& p) const {
    const int64_t e = (int64_t)z * P + off + (int64_t)row * ld + col;
    const float s = p.et * p.s - p.th * v;
    const float w = (1.0f - p.al) * p.w + s;
    Sout[e] = s;
    Wout[e] = w;
    if (!(isfinite(s) && isfinite(w))) flag[0] = 1;
  }
};

// ---------------------------------------------------------------------------- helpers

static __host__ __device__ StridedLoader strided(const float* base, int64_t sz, int64_t so, int64_t sk, int zdiv, int outer_dim, int K,
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
static __host__ __device__ StridedLoader hidden(const Dims& d, const float* Z, int64_t sz, int64_t so, int64_t sk, int zdiv, int outer_dim,
                            int K) {
  StridedLoader l = strided(Z, sz, so, sk, zdiv, outer_dim, K, d.gated ? XF_GATED : XF_SILU);
  l.gofs = d.dh;
  return l;
}

// `h` supplies the split-K scratch (null: no split).
// `prec`: 0 plain bf16 operands, 1 split bf16 (hi/lo), 2 fp32 operands (Dims::prec).
template <class LA, class LB, class EP>
static void gemm_any(int prec, bool a_exact, bool b_exact, int M, int N, int K, int batch, const LA& la, const LB& lb,
                     const EP& ep, hipStream_t st, const Handle* h = nullptr) {
  if (prec == 2) {
    launch_gemm_f32(M, N, K, batch, la, lb, ep, st);
    return;
  }
  const bool split = prec == 1;
  float* sk = (h && !h->d.no_splitk) ? h->sk : nullptr;
  const int64_t skf = h ? h->sk_floats : 0;
  if (a_exact && b_exact) launch_gemm<true, true>(split, M, N, K, batch, la, lb, ep, st, sk, skf);
  else if (a_exact) launch_gemm<true, false>(split, M, N, K, batch, la, lb, ep, st, sk, skf);
  else if (b_exact) launch_gemm<false, true>(split, M, N, K, batch, la, lb, ep, st, sk, skf);
  else launch_gemm<false, false>(split, M, N, K, batch, la, lb, ep, st, sk, skf);
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

// The rows of a convolved call (h->conv set): FeatRows plus the three tensors' convolutions.
static ConvRows conv_rows(const Handle* h, const void* K, const void* Q, int64_t ld, int64_t s, int Rk, int nrows,
                          int zdiv) {
  const Dims& d = h->d;
  ConvRows cr;
  cr.fr = feat_rows(h, K, Q, ld, s, Rk, nrows, zdiv);
  const atlasmem_short_conv_params* p = h->conv;
  const int heads = h->cfg.heads;
  const int nk = h->ncb * d.C + d.c - 1, nq = h->ncb * d.C;
  cr.ck = ConvTensor{K, h->chk[h->chcur], p->taps_k, p->bias_k, p->l2norm_k ? h->cinvk : nullptr, h->cinv_t0k, nk,
                     heads, d.dk, d.in_bf16};
  cr.cq = ConvTensor{Q, h->chq[h->chcur], p->taps_q, p->bias_q, p->l2norm_q ? h->cinvq : nullptr, h->cinv_t0q, nq,
                     heads, d.dk, d.in_bf16};
  cr.cv = ConvTensor{h->conv_v, h->chv[h->chcur], p->taps_v, p->bias_v, nullptr, 0, 0, heads, d.dv, d.in_bf16};
  return cr;
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
  const int split = d.prec;
  const bool feat_exact = d.poly == 1 && d.in_bf16;
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
    gemm_any(split, feat_exact, false, C, dz, din, M, la, lb, ep, st, h);
  }
  // scores A1[t][r] = q_t . x_r over the key rows (window history included)
  {
    FeatA la{qrows};
    FeatA lb{feat_rows(h, K, Q, ld, s, Rk, Rk, 1)};
    EpiStore ep{h->pA1, az, Rk, 1};
    gemm_any(split, feat_exact, feat_exact, C, Rk, din, M, la, lb, ep, st, h);
  }
  // Zq = beta Z0 + a ZS - (Om * A1) D1
  {
    StridedLoader la = strided(h->pA1, az, Rk, 1, 1, C, Rk, XF_MAT);
    la.coef0 = h->pOm;
    la.cz = az;
    la.cld = Rk;
    StridedLoader lb = strided(h->D1, (int64_t)Rk * dz, 1, dz, 1, dz, Rk);  // B(k=r, j) = D1[r][j]
    EpiZq ep{h->pZS, h->Z, h->pbA, qz, zsz, (int64_t)Rk, dz, C};
    gemm_any(split, false, false, C, dz, Rk, M, la, lb, ep, st, h);
  }
  // scores A2[t][r] = Hq_t . h_r
  {
    StridedLoader la = hidden(d, h->pZS, qz, dz, 1, 1, C, dh);
    StridedLoader lb = hidden(d, h->Z, zsz, dz, 1, 1, Rk, dh);  // B(k=h, j=r) = H[r][h]
    EpiStore ep{h->pA1, az, Rk, 1};
    gemm_any(split, false, false, C, Rk, dh, M, la, lb, ep, st, h);
  }
  // YB = beta Hq W0_2^T + a Hq S0_2^T
  for (int which = 0; which < 2; ++which) {
    StridedLoader la = hidden(d, h->pZS, qz, dz, 1, 1, C, dh);
    StridedLoader lb = strided((which ? Sin : Win) + d.P1, d.P, dh, 1, 1, dv, dh);  // B(k=h, j=v) = W2[v][h]
    EpiRowMix ep{h->pYB, h->pbA, yz, dv, C, which, which};
    gemm_any(split, false, false, C, dv, dh, M, la, lb, ep, st, h);
  }
  // Y = YB - (Om * A2) D2 (+ the query's features for the residual memory)
  {
    StridedLoader la = strided(h->pA1, az, Rk, 1, 1, C, Rk, XF_MAT);
    la.coef0 = h->pOm;
    la.cz = az;
    la.cld = Rk;
    StridedLoader lb = strided(h->D2, (int64_t)Rk * dv, 1, dv, 1, dv, Rk);  // B(k=r, j=v) = D2[r][v]
    EpiYptr ep{h->pYB, yz, dv, ld, s, Y, d.out_bf16, d.residual, qrows};
    gemm_any(split, false, false, C, dv, Rk, M, la, lb, ep, st, h);
  }
  return ATLASMEM_OK;
}

// ---------------------------------------------------------------------------- one call

// ---------------------------------------------------------------------------- chunk loop

// The same chunk sequence as the per-product launches of mlp_update (Z, Yh, Pm, then the two
// weighted-gradient products with the state update in their epilogues), run for a block of
// chunks inside one launch: workgroup m walks the chunks of memory m, and its four groups of 256
// threads share out each product's 64 x 64 output tiles.  The intermediates Z, D2, D1 go through
// the memory's own slice of the workspace (written and read by the same workgroup, so a
// workgroup barrier orders them).  Chunk kb of the block reads state buffer cur ^ (kb & 1).
struct LoopArgs {
  Dims d;
  const void* K;
  const void* Q;
  const void* V;
  const float* theta;  // per-chunk gates (per-chunk gates without Newton-Schulz)
  const float* eta;
  const float* alpha;
  int64_t ld, ldg;  // token stride of K, Q, V, Y; gate stride
  void* Y;
  const float* hk;  // window history at the start of the call
  const float* hv;
  float* W[2];
  float* S[2];
  int cur;
  float* Z;
  float* D2;
  float* D1;
  const float* cW;  // coefficients of the block (per-token gates)
  const float* cS;
  const float* oW;
  const float* oS;
  const float* scal;
  int ncb;
  int64_t kb0;  // first chunk of the block within the call
  int nb;       // chunks in the block
  int* flag;
};

constexpr int LOOP_GROUPS = 4;
constexpr int LOOP_THREADS = 256 * LOOP_GROUPS;
constexpr int LOOP_LDS = LOOP_GROUPS * (int)sizeof(TileSmem<true, false, false>);

// All tiles of one product (batches z0 .. z0 + nz - 1), LOOP_GROUPS at a time, then a barrier so
// that the next product reads this one's epilogue stores.
template <bool SPLIT, bool AE, bool BE, class LA, class LB, class EP>
__device__ __forceinline__ void loop_stage(int M, int N, int K, int z0, int nz, const LA& la, const LB& lb,
                                           const EP& ep, uint16_t* lsm) {
  if (M <= 0 || N <= 0) return;
  // the thread index made opaque here, so that the compiler derives each product's addresses
  // where they are used instead of keeping every product's live across the whole chunk loop
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  const int grp = __builtin_amdgcn_readfirstlane(tid >> 8), t = tid & 255;
  auto& sm = ((TileSmem<SPLIT, AE, BE>*)lsm)[grp];
  const int tm = (M + GT - 1) / GT, tn = (N + GT - 1) / GT, per = tm * tn, nt = per * nz;
  for (int r0 = 0; r0 < nt; r0 += LOOP_GROUPS) {
    const int tile = r0 + grp;
    const bool active = tile < nt;
    const int tz = active ? tile / per : 0, rem = active ? tile % per : 0;
    gemm_tile<SPLIT, AE, BE>(M, N, K, la, lb, ep, z0 + tz, (rem / tn) * GT, (rem % tn) * GT, t, sm, active);
  }
  __syncthreads();
}

template <bool SPLIT, bool FEAT_EXACT>
__global__ void __launch_bounds__(LOOP_THREADS) mlp_loop_kernel(LoopArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint16_t lsm[];
  const Dims& d = a.d;
  const int mem = blockIdx.x;
  const int C = d.C, c = d.c, Rk = d.Rk, dh = d.dh, dv = d.dv, din = d.din, dz = d.dz;
  const int nrows = Rk + (a.Y ? C : 0);
  const int64_t zsz = (int64_t)d.Rt * dz;
  const bool per_token = d.gate_mode == ATLASMEM_PER_TOKEN;
  for (int kb = 0; kb < a.nb; ++kb) {
    const int64_t k = a.kb0 + kb;
    const int64_t s = k * C;
    const int pp = a.cur ^ (kb & 1);
    const float* Win = a.W[pp];
    const float* Sin = a.S[pp];
    float* Wout = a.W[1 - pp];
    float* Sout = a.S[1 - pp];
    FeatRows fr;
    fr.K = a.K;
    fr.Q = a.Q;
    fr.in_bf16 = d.in_bf16;
    fr.hk = a.hk;
    fr.T = a.ld;
    fr.s = s;
    fr.Rk = Rk;
    fr.nrows = nrows;
    fr.c = c;
    fr.dk = d.dk;
    fr.din = din;
    fr.poly = d.poly;
    fr.zdiv = 1;
    FeatRows frk = fr;  // key rows only
    frk.nrows = Rk;
    {  // Z = X W1^T over key and query rows
      FeatA la{fr};
      StridedLoaderC lb = clamped(strided(Win, d.P, din, 1, 1, dz, din));
      EpiStore ep{a.Z, zsz, dz, 1};
      loop_stage<SPLIT, FEAT_EXACT, false>(nrows, dz, din, mem, 1, la, lb, ep, lsm);
    }
    {  // Yh = H W2^T -> D2 (key rows), Y (query rows)
      StridedLoaderC la = clamped(hidden(d, a.Z, zsz, dz, 1, 1, nrows, dh));
      StridedLoaderC lb = clamped(strided(Win + d.P1, d.P, dh, 1, 1, dv, dh));
      EpiY ep{a.D2, (int64_t)Rk * dv, a.V, d.in_bf16, a.hv, a.ld, s, Rk, c, dv, a.Y, d.out_bf16, d.residual, fr};
      loop_stage<SPLIT, false, false>(nrows, dv, dh, mem, 1, la, lb, ep, lsm);
    }
    {  // Pm = D2 W2 -> D1
      StridedLoaderC la = clamped(strided(a.D2, (int64_t)Rk * dv, dv, 1, 1, Rk, dv));
      StridedLoaderC lb = clamped(strided(Win + d.P1, d.P, 1, dh, 1, dh, dv));
      EpiP ep{a.D1, a.Z, (int64_t)Rk * dz, zsz, dh, dz, d.gated};
      loop_stage<SPLIT, false, false>(Rk, dh, dv, mem, 1, la, lb, ep, lsm);
    }
    if (per_token) {
      const float* c0 = (c > 1) ? a.oW + (int64_t)kb * Rk : a.cW + (int64_t)kb * C;
      const float* c1 = (c > 1) ? a.oS + (int64_t)kb * Rk : a.cS + (int64_t)kb * C;
      const int64_t cz = (c > 1) ? (int64_t)a.ncb * Rk : (int64_t)a.ncb * C;
      const float* sc = a.scal + (int64_t)kb * 3;
      {
        StridedLoaderC la = clamped(strided(a.D2, (int64_t)Rk * dv, 1, dv, 2, dv, Rk, XF_COEF));
        la.coef0 = c0;
        la.coef1 = c1;
        la.cz = cz;
        StridedLoaderC lb = clamped(hidden(d, a.Z, zsz, 1, dz, 2, dh, Rk));
        EpiUpdPair ep{Win, Sin, Wout, Sout, d.P, d.P1, dh, sc, (int64_t)a.ncb * 3, a.flag};
        loop_stage<SPLIT, false, false>(dv, dh, Rk, 2 * mem, 2, la, lb, ep, lsm);
      }
      {
        StridedLoaderC la = clamped(strided(a.D1, (int64_t)Rk * dz, 1, dz, 2, dz, Rk, XF_COEF));
        la.coef0 = c0;
        la.coef1 = c1;
        la.cz = cz;
        FeatB lb{frk};
        lb.fr.zdiv = 2;
        EpiUpdPair ep{Win, Sin, Wout, Sout, d.P, 0, din, sc, (int64_t)a.ncb * 3, a.flag};
        loop_stage<SPLIT, false, FEAT_EXACT>(dz, din, Rk, 2 * mem, 2, la, lb, ep, lsm);
      }
    } else {
      {
        StridedLoaderC la = clamped(strided(a.D2, (int64_t)Rk * dv, 1, dv, 1, dv, Rk));
        StridedLoaderC lb = clamped(hidden(d, a.Z, zsz, 1, dz, 1, dh, Rk));
        EpiUpdChunk ep{Win, Sin, Wout, Sout, d.P, d.P1, dh, a.theta, a.eta, a.alpha, a.ldg, k, a.flag};
        loop_stage<SPLIT, false, false>(dv, dh, Rk, mem, 1, la, lb, ep, lsm);
      }
      {
        StridedLoaderC la = clamped(strided(a.D1, (int64_t)Rk * dz, 1, dz, 1, dz, Rk));
        FeatB lb{frk};
        EpiUpdChunk ep{Win, Sin, Wout, Sout, d.P, 0, din, a.theta, a.eta, a.alpha, a.ldg, k, a.flag};
        loop_stage<SPLIT, false, FEAT_EXACT>(dz, din, Rk, mem, 1, la, lb, ep, lsm);
      }
    }
  }
}

// Length of the chunk's dependent chain in tile steps when one workgroup with LOOP_GROUPS tile
// groups runs a memory's products: sum over the products of ceil(tiles / groups) x k-steps.
static int64_t loop_chain(const Dims& d, bool with_y) {
  auto cd = [](int64_t a, int64_t b) { return (a + b - 1) / b; };
  const int64_t nrows = d.Rk + (with_y ? d.C : 0);
  const int64_t pair = d.gate_mode == ATLASMEM_PER_TOKEN ? 2 : 1;
  auto st = [&](int64_t m, int64_t n, int64_t k, int64_t nz) { return cd(cd(m, GT) * cd(n, GT) * nz, LOOP_GROUPS) * cd(k, GK); };
  return st(nrows, d.dz, d.din, 1) + st(nrows, d.dv, d.dh, 1) + st(d.Rk, d.dh, d.dv, 1) +
         st(d.dv, d.dh, d.Rk, pair) + st(d.dz, d.din, d.Rk, pair);
}

// The chunk loop replaces the per-product launches where a memory's chunk is a short chain of
// tile steps: the 64 -> 128 -> 64 memory takes 12 (4.9 -> 3.8 ms for 8 memories x 4096 tokens on
// MI355X).  Longer chains keep one launch per product, whose tiles then spread over many
// workgroups: degree-2 features of 32-wide keys (72 steps) ran 2x slower in the loop, and the
// 384 -> 768 -> 384 memory takes 324.
static bool loop_supported(const Dims& d, bool with_y) {
  return !d.no_loop && !d.ptr && !d.conv && d.prec != 2 && (d.gate_mode == ATLASMEM_PER_TOKEN || d.ns_steps == 0) && loop_chain(d, with_y) <= 24;
}

// The window history of a call whose rows are convolved while read: the last c - 1 convolved keys
// and values (and gammas) of (old history ++ this call), as the plain history kernel keeps them.
__global__ void history_conv_kernel(ConvTensor ck, ConvTensor cv, const float* __restrict__ gamma, int M, int64_t T,
                                    int64_t ld, int c, int dk, int dv, const float* __restrict__ hk,
                                    const float* __restrict__ hv, const float* __restrict__ hg, float* __restrict__ nk,
                                    float* __restrict__ nv, float* __restrict__ ng) {
  const int H = c - 1;
  const int width = dk + dv + 1;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)M * H * width) return;
  const int e = (int)(idx % width);
  const int hrow = (int)((idx / width) % H);
  const int m = (int)(idx / ((int64_t)width * H));
  const int64_t tau = T - H + hrow;
  if (e < dk) {
    nk[((int64_t)m * H + hrow) * dk + e] = tau >= 0 ? ck.at(m, ld, tau, e) : hk[((int64_t)m * H + hrow + T) * dk + e];
  } else if (e < dk + dv) {
    const int ev = e - dk;
    nv[((int64_t)m * H + hrow) * dv + ev] = tau >= 0 ? cv.at(m, ld, tau, ev) : hv[((int64_t)m * H + hrow + T) * dv + ev];
  } else {
    ng[(int64_t)m * H + hrow] = tau >= 0 ? gamma[(int64_t)m * ld + tau] : hg[(int64_t)m * H + hrow + T];
  }
}

atlasmem_status mlp_update(Handle* h, const Dims& d, const void* K, const void* Q, const void* V, const float* theta,
                           const float* eta, const float* alpha, const float* gamma, const Span& sp, void* Y,
                           hipStream_t st) {
  const int64_t T = sp.T, ld = sp.ld;
  const int M = d.M, C = d.C, c = d.c, Rk = d.Rk, dh = d.dh, dv = d.dv, din = d.din, dz = d.dz;
  const int split = d.prec;
  const bool feat_exact = d.poly == 1 && d.in_bf16;
  const int64_t nchunks = T / C;
  const int nq = Y ? C : 0;
  const int nrows = Rk + nq;
  const int64_t zsz = (int64_t)d.Rt * dz;
  const bool per_token = d.gate_mode == ATLASMEM_PER_TOKEN;
  atlasmem_status stt;
  if (!d.no_fused && !d.conv && fused_supported(d)) {
    // E_UNSUPPORTED: the gated memory's workgroup pairs cannot all be resident (or the cooperative
    // launch was refused); nothing ran
    const atlasmem_status fs = launch_fused(h, d, K, Q, V, theta, eta, alpha, sp, Y, st);
    if (fs != ATLASMEM_E_UNSUPPORTED) return fs;
  }

  for (int64_t kb0 = 0; kb0 < nchunks; kb0 += h->ncb) {
    const int nb = (int)((nchunks - kb0) < h->ncb ? (nchunks - kb0) : h->ncb);
    if (d.conv) {  // inverse norms of the block's convolved key rows (window rows included) and queries
      const atlasmem_short_conv_params* p = h->conv;
      const int64_t tk0 = kb0 * C - (c - 1) > 0 ? kb0 * C - (c - 1) : 0, tk1 = (kb0 + nb) * C;
      h->cinv_t0k = tk0;
      h->cinv_t0q = kb0 * C;
      if (p->l2norm_k) {
        stt = launch_conv_inv_norm(K, h->chk[h->chcur], d.in_bf16, M, ld, tk0, tk1 - tk0, d.dk, h->cfg.heads, p->taps_k,
                                   p->bias_k, h->cinvk, (int64_t)h->ncb * C + c - 1, st);
        if (stt != ATLASMEM_OK) return stt;
      }
      if (p->l2norm_q && (Y || d.residual)) {
        stt = launch_conv_inv_norm(Q, h->chq[h->chcur], d.in_bf16, M, ld, kb0 * C, (int64_t)nb * C, d.dk, h->cfg.heads,
                                   p->taps_q, p->bias_q, h->cinvq, (int64_t)h->ncb * C, st);
        if (stt != ATLASMEM_OK) return stt;
      }
    }
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
    if (fused_pt_supported(d)) {
      stt = launch_fused_pt(h, d, K, Q, V, kb0, nb, ld, Y, st);
      if (stt != ATLASMEM_OK) return stt;
      continue;
    }
    // (its vector loads and stores need 16-byte aligned rows, its buffer offsets a memory's rows
    // within 2 GB)
    if (!d.no_fused && h->hsw && hsplit_supported(d) && ld * (d.dk > d.dv ? d.dk : d.dv) * 4 < ((int64_t)1 << 31) &&
        (((uintptr_t)K | (uintptr_t)Q | (uintptr_t)V | (uintptr_t)Y) & 15) == 0) {
      stt = launch_hsplit(h, d, K, Q, V, kb0, nb, ld, Y, st);
      if (stt != ATLASMEM_OK) return stt;
      continue;
    }
    if (loop_supported(d, Y != nullptr)) {
      LoopArgs la;
      la.d = d;
      la.K = K;
      la.Q = Q;
      la.V = V;
      la.theta = theta;
      la.eta = eta;
      la.alpha = alpha;
      la.ld = ld;
      la.ldg = sp.ldg;
      la.Y = Y;
      la.hk = h->hk[h->hcur];
      la.hv = h->hv[h->hcur];
      la.W[0] = h->W[0];
      la.W[1] = h->W[1];
      la.S[0] = h->S[0];
      la.S[1] = h->S[1];
      la.cur = h->cur;
      la.Z = h->Z;
      la.D2 = h->D2;
      la.D1 = h->D1;
      la.cW = h->cW;
      la.cS = h->cS;
      la.oW = h->oW;
      la.oS = h->oS;
      la.scal = h->scal;
      la.ncb = h->ncb;
      la.kb0 = kb0;
      la.nb = nb;
      la.flag = h->flag;
      const void* kern = split == 1 ? (feat_exact ? (const void*)mlp_loop_kernel<true, true> : (const void*)mlp_loop_kernel<true, false>)
                               : (feat_exact ? (const void*)mlp_loop_kernel<false, true> : (const void*)mlp_loop_kernel<false, false>);
      if (hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, LOOP_LDS) != hipSuccess)
        return ATLASMEM_E_DEVICE;
      if (split == 1) {
        if (feat_exact) hipLaunchKernelGGL((mlp_loop_kernel<true, true>), dim3(M), dim3(LOOP_THREADS), LOOP_LDS, st, la);
        else hipLaunchKernelGGL((mlp_loop_kernel<true, false>), dim3(M), dim3(LOOP_THREADS), LOOP_LDS, st, la);
      } else {
        if (feat_exact) hipLaunchKernelGGL((mlp_loop_kernel<false, true>), dim3(M), dim3(LOOP_THREADS), LOOP_LDS, st, la);
        else hipLaunchKernelGGL((mlp_loop_kernel<false, false>), dim3(M), dim3(LOOP_THREADS), LOOP_LDS, st, la);
      }
      AM_LAUNCH_CHECK();
      if (nb & 1) h->cur = 1 - h->cur;
      continue;
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
        StridedLoader lb = strided(W1, d.P, din, 1, 1, dz, din);  // B(k=f, j=h) = W1[h][f]
        EpiStore ep{h->Z, zsz, dz, 1};
        if (d.conv)
          gemm_any(split, feat_exact, false, nrows, dz, din, M, FeatAConv{conv_rows(h, K, Q, ld, s, Rk, nrows, 1)}, lb,
                   ep, st, h);
        else
          gemm_any(split, feat_exact, false, nrows, dz, din, M, FeatA{feat_rows(h, K, Q, ld, s, Rk, nrows, 1)}, lb, ep,
                   st, h);
      }
      // Yh = H W2^T -> D2 (key rows), Y (query rows; with per-token retrieval they are answered
      // below from the per-token states instead)
      const int yrows = d.ptr ? Rk : nrows;
      {
        StridedLoader la = hidden(d, h->Z, zsz, dz, 1, 1, yrows, dh);
        StridedLoader lb = strided(W2, d.P, dh, 1, 1, dv, dh);  // B(k=h, j=v) = W2[v][h]
        if (d.conv) {
          EpiYConv ep{h->D2, (int64_t)Rk * dv, h->hv[h->hcur], s, Rk, c, dv, Y, d.out_bf16, d.residual,
                      conv_rows(h, K, Q, ld, s, Rk, nrows, 1)};
          gemm_any(split, false, false, yrows, dv, dh, M, la, lb, ep, st, h);
        } else {
          EpiY ep{h->D2, (int64_t)Rk * dv, V, d.in_bf16, h->hv[h->hcur], ld, s, Rk, c, dv, Y, d.out_bf16,
                  d.residual, feat_rows(h, K, Q, ld, s, Rk, nrows, 1)};
          gemm_any(split, false, false, yrows, dv, dh, M, la, lb, ep, st, h);
        }
      }
      // Pm = D2 W2 -> D1 = Pm * silu'(Z)
      {
        StridedLoader la = strided(h->D2, (int64_t)Rk * dv, dv, 1, 1, Rk, dv);
        StridedLoader lb = strided(W2, d.P, 1, dh, 1, dh, dv);  // B(k=v, j=h) = W2[v][h]
        EpiP ep{h->D1, h->Z, (int64_t)Rk * dz, zsz, dh, dz, d.gated};
        gemm_any(split, false, false, Rk, dh, dv, M, la, lb, ep, st, h);
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
          gemm_any(split, false, false, dv, dh, Rk, 2 * M, la, lb, ep, st, h);
        }
        // W1 pair (gated: W1 and W3 as one block of 2 d_hidden rows): A(i=h, k=row) =
        // D1[row][h] * coef[row], B(k=row, j=f) = X[row][f]
        {
          StridedLoader la = strided(h->D1, (int64_t)Rk * dz, 1, dz, 2, dz, Rk, XF_COEF);
          la.coef0 = c0;
          la.coef1 = c1;
          la.cz = cz;
          EpiUpdPair ep{Win, Sin, Wout, Sout, d.P, 0, din, sc, (int64_t)h->ncb * 3, h->flag};
          if (d.conv)
            gemm_any(split, false, feat_exact, dz, din, Rk, 2 * M, la, FeatBConv{conv_rows(h, K, Q, ld, s, Rk, Rk, 2)},
                     ep, st, h);
          else
            gemm_any(split, false, feat_exact, dz, din, Rk, 2 * M, la, FeatB{feat_rows(h, K, Q, ld, s, Rk, Rk, 2)}, ep,
                     st, h);
        }
      } else if (d.ns_steps == 0) {
        {
          StridedLoader la = strided(h->D2, (int64_t)Rk * dv, 1, dv, 1, dv, Rk);
          StridedLoader lb = hidden(d, h->Z, zsz, 1, dz, 1, dh, Rk);
          EpiUpdChunk ep{Win, Sin, Wout, Sout, d.P, d.P1, dh, theta, eta, alpha, sp.ldg, k, h->flag};
          gemm_any(split, false, false, dv, dh, Rk, M, la, lb, ep, st, h);
        }
        {
          StridedLoader la = strided(h->D1, (int64_t)Rk * dz, 1, dz, 1, dz, Rk);
          EpiUpdChunk ep{Win, Sin, Wout, Sout, d.P, 0, din, theta, eta, alpha, sp.ldg, k, h->flag};
          if (d.conv)
            gemm_any(split, false, feat_exact, dz, din, Rk, M, la, FeatBConv{conv_rows(h, K, Q, ld, s, Rk, Rk, 1)}, ep,
                     st, h);
          else
            gemm_any(split, false, feat_exact, dz, din, Rk, M, la, FeatB{feat_rows(h, K, Q, ld, s, Rk, Rk, 1)}, ep, st,
                     h);
        }
      } else {
        {
          StridedLoader la = strided(h->D2, (int64_t)Rk * dv, 1, dv, 1, dv, Rk);
          StridedLoader lb = hidden(d, h->Z, zsz, 1, dz, 1, dh, Rk);
          EpiStore ep{h->G + d.P1, d.P, dh, 1};
          gemm_any(split, false, false, dv, dh, Rk, M, la, lb, ep, st, h);
        }
        {
          StridedLoader la = strided(h->D1, (int64_t)Rk * dz, 1, dz, 1, dz, Rk);
          EpiStore ep{h->G, d.P, din, 1};
          if (d.conv)
            gemm_any(split, false, feat_exact, dz, din, Rk, M, la, FeatBConv{conv_rows(h, K, Q, ld, s, Rk, Rk, 1)}, ep,
                     st, h);
          else
            gemm_any(split, false, feat_exact, dz, din, Rk, M, la, FeatB{feat_rows(h, K, Q, ld, s, Rk, Rk, 1)}, ep, st,
                     h);
        }
        // each weight matrix separately, W1, (W3,) W2, as groups of one launch
        const int64_t o3 = (int64_t)dh * din;
        NsGroup grp[3];
        int ng = 0;
        grp[ng++] = NsGroup{dh, din, 0, 0};
        if (d.gated) grp[ng++] = NsGroup{dh, din, o3, o3};
        grp[ng++] = NsGroup{dv, dh, d.P1, d.P1};
        const NsUpdate u{Win, Sin, Wout, Sout, d.P, 0, 1, theta, eta, alpha, sp.ldg, k, h->flag};
        stt = launch_ns_groups(h->G, d.P, M, ng, grp, d.ns_steps, d.ns_a, d.ns_b, d.ns_c, d.ns_eps, split, u, st);
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
  if (d.conv) {
    if (c > 1 && T > 0) {
      // the window history keeps convolved keys and values: the last c - 1 rows' norms, then the rows
      const atlasmem_short_conv_params* p = h->conv;
      const int64_t th0 = T - (c - 1) > 0 ? T - (c - 1) : 0;
      h->cinv_t0k = th0;
      if (p->l2norm_k) {
        stt = launch_conv_inv_norm(K, h->chk[h->chcur], d.in_bf16, M, ld, th0, T - th0, d.dk, h->cfg.heads, p->taps_k,
                                   p->bias_k, h->cinvk, (int64_t)h->ncb * C + c - 1, st);
        if (stt != ATLASMEM_OK) return stt;
      }
      const ConvRows cr = conv_rows(h, K, Q, ld, 0, 0, 0, 1);
      const int64_t total = (int64_t)M * (c - 1) * (d.dk + d.dv + 1);
      const int src = h->hcur, dst = 1 - h->hcur;
      hipLaunchKernelGGL(history_conv_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st, cr.ck, cr.cv,
                         gamma, M, T, ld, c, d.dk, d.dv, h->hk[src], h->hv[src], h->hg[src], h->hk[dst], h->hv[dst],
                         h->hg[dst]);
      AM_LAUNCH_CHECK();
      h->hcur = 1 - h->hcur;
    }
    return ATLASMEM_OK;
  }
  stt = launch_history_update(h, K, V, gamma, T, ld, st);
  if (stt != ATLASMEM_OK) return stt;
  if (c > 1 && T > 0) h->hcur = 1 - h->hcur;
  return ATLASMEM_OK;
}

atlasmem_status ptr_partial_retrieve(Handle* h, int64_t r, hipStream_t st) {
  // the buffered rows as a chunk of r tokens (token stride C of the pending buffers)
  Dims d = h->d;
  d.C = (int)r;
  d.Rk = d.C + d.c - 1;
  d.Rt = d.Rk + d.C;
  const int M = d.M, Rk = d.Rk, dh = d.dh, dv = d.dv, din = d.din, dz = d.dz;
  const int split = d.prec;
  const bool feat_exact = d.poly == 1 && d.in_bf16;
  const int64_t ld = h->d.C;
  const int64_t zsz = (int64_t)d.Rt * dz;
  const void* K = h->pK;
  const void* Q = h->pQ;
  const float* Win = h->W[h->cur];
  const float* Sin = h->S[h->cur];
  // Z of the key rows (window history included) and of the query rows (their chunk-start part of
  // the per-token first layer), D2 of the keys, then D1, all at the chunk-start weights
  {
    StridedLoader lb = strided(Win, d.P, din, 1, 1, dz, din);
    EpiStore ep{h->Z, zsz, dz, 1};
    gemm_any(split, feat_exact, false, Rk + d.C, dz, din, M, FeatA{feat_rows(h, K, Q, ld, 0, Rk, Rk + d.C, 1)}, lb,
             ep, st, h);
  }
  {
    StridedLoader la = hidden(d, h->Z, zsz, dz, 1, 1, Rk, dh);
    StridedLoader lb = strided(Win + d.P1, d.P, dh, 1, 1, dv, dh);
    EpiY ep{h->D2, (int64_t)Rk * dv, h->pV, d.in_bf16, h->hv[h->hcur], ld, 0, Rk, d.c, dv, nullptr, d.out_bf16,
            d.residual, feat_rows(h, K, Q, ld, 0, Rk, Rk, 1)};
    gemm_any(split, false, false, Rk, dv, dh, M, la, lb, ep, st, h);
  }
  {
    StridedLoader la = strided(h->D2, (int64_t)Rk * dv, dv, 1, 1, Rk, dv);
    StridedLoader lb = strided(Win + d.P1, d.P, 1, dh, 1, dh, dv);
    EpiP ep{h->D1, h->Z, (int64_t)Rk * dz, zsz, dh, dz, d.gated};
    gemm_any(split, false, false, Rk, dh, dv, M, la, lb, ep, st, h);
  }
  const atlasmem_status s = ptr_retrieve(h, d, K, Q, h->pth, h->pet, h->pal, d.c > 1 ? h->pg : nullptr, ld, 0, Win,
                                         Sin, h->pYs, st);
  if (s != ATLASMEM_OK) return s;
  AM_LAUNCH_CHECK();
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
      gemm_any(d.prec, feat_exact, false, rows, dz, din, M, la, lb, ep, st, h);
    }
    {
      StridedLoader la = hidden(d, h->Zr, zsz, dz, 1, 1, rows, dh);
      StridedLoader lb = strided(W2, d.P, dh, 1, 1, dv, dh);
      EpiY ep{nullptr, 0, nullptr, d.in_bf16, nullptr, ld, s, 0, d.c, dv, Y, d.out_bf16, d.residual,
              feat_rows(h, nullptr, Q, ld, s, 0, rows, 1)};
      gemm_any(d.prec, false, false, rows, dv, dh, M, la, lb, ep, st, h);
    }
    AM_LAUNCH_CHECK();
  }
  return ATLASMEM_OK;
}

}  // namespace am
