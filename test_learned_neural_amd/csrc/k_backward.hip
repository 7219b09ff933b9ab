// Outer-loop backward of the chunked update: the gradients of an outer loss with respect to the
// keys, queries, values, gates and initial state of the test-time update (Atlas-Torch README,
// "How the memory works": the outer loop trains through the inner updates).  Scope: the 2-layer
// SiLU memory (plain or residual, x + W2 silu(W1 x)) with window 1 and identity features;
// per-token gates, or per-chunk gates with the
// optional Newton-Schulz orthogonalisation of the chunk gradient (differentiated through its
// iterates, which the reverse step recomputes from the chunk-start checkpoint).
//
// Forward of chunk k from (W, S) = (W1, W2, S1, S2), rows r of the chunk (titans-pytorch-mlx
// README, Eq. 12-14; gradients at the chunk-start weights, ATLAS summary, section 3.3):
//   Z = X W1^T, H = silu(Z), E = 2 (H W2^T - V), P = E W2, D1 = P * silu'(Z)
//   W' = beta W + aS S - sum_r cW_r g_r,  S' = PC S - sum_r cS_r g_r,  g_r = (D1_r x_r^T, E_r h_r^T)
//   Y = silu(Q W1^T) W2^T
// with (cW, cS, PC, beta, aS) from the gate scan.  Given the adjoints (WA, SA) of (W', S') and dY,
// the backward of the chunk is (every product batched over memories on the GEMM engine):
//   U1 = X WA1^T, U1s = X SA1^T, U2 = H WA2^T, U2s = H SA2^T
//   cW'_r = -(<D1_r, U1_r> + <E_r, U2_r>),  cS'_r = -(<D1_r, U1s_r> + <E_r, U2s_r>)
//   D1' = -(cW U1 + cS U1s),  E'_g = -(cW U2 + cS U2s),  P' = D1' silu'(Z),  Z'_1 = D1' P silu''(Z)
//   E' = E'_g + P' W2^T,  V' = -2 E'
//   W2' = E^T P' + (2E')^T H + dY^T Hq
//   H' = -(cW E) WA2 - (cS E) SA2 + (2E') W2,  Z' = Z'_1 + H' silu'(Z)
//   X' = -(cW D1) WA1 - (cS D1) SA1 + Z' W1
//   Zq' = (dY W2) silu'(Zq),  Q' = Zq' W1,  W1' = Z'^T X + Zq'^T Q
//   beta' = <WA, W>, aS' = <WA, S>, PC' = <SA, S>;  gates' from (cW', cS', PC', beta', aS') by the
//   reverse of the gate scan
//   WA <- beta WA + (W1', W2'),  SA <- aS WA + PC SA        (the adjoints at the chunk start)
//
// Per-chunk gates (one triple per chunk): G = sum_r g_r = (D1^T X, E^T H), N = NS(G) (or G),
// S' = eta S - theta N, W' = (1 - alpha) W + S'.  With SAt = SA + WA (S' also feeds W'):
//   theta' = -<SAt, N>, eta' = <SAt, S>, alpha' = -<WA, W>,  N' = -theta SAt,  G' = NS'(N')
// and every row's gradient has the adjoint G', which the row products above take as WA with
// cW = -1 and no momentum term.  NS' runs the iteration X <- a X + (b A + c A^2) X, A = X X^T,
// backwards from its stored iterates:
//   Ba = Xa X^T,  Aa = b Ba + c (Ba A + A Ba),  Xa <- a Xa + B Xa + (Aa + Aa^T) X
// and through the normalisation X_0 = G / (|G| + eps):  G' = Xa_0 / n - (<Xa_0, G> / n^2) G / |G|.
// The carry is WA <- (1 - alpha) WA + (W1', W2'), SA <- eta SAt.
#include "common.h"
#include "gemm.h"
#include "internal.h"

namespace am {
namespace bk {

// One operand source: element (z, outer, k) of base[z * sz + outer * so + k * sk] (fp32, or bf16
// input bits), optionally through silu or scaled by a per-outer coefficient, times `scale`.
struct Src {
  const void* base;
  int bf16;
  int64_t sz, so, sk;
  int outer_dim, K;
  int xf;  // 0 none, 1 silu, 2 times coef[z * cz + outer], 3 silu(x) times the element gofs further on
  const float* coef;
  int64_t cz;
  float scale;
  int64_t gofs;  // xf 3: the gated memory's silu(Z1) * Z3 with Z3 beside Z1 (fp32 sources)
  __device__ __forceinline__ float get(int z, int outer, int k) const {
    if (outer >= outer_dim || k >= K) return 0.0f;
    const int64_t i = (int64_t)z * sz + (int64_t)outer * so + (int64_t)k * sk;
    float x = bf16 ? bf16_value(((const uint16_t*)base)[i]) : ((const float*)base)[i];
    if (xf == 1) x = siluf_(x);
    else if (xf == 2) x *= coef[(int64_t)z * cz + outer];
    else if (xf == 3) x = siluf_(x) * ((const float*)base)[i + gofs];
    return x * scale;
  }
};

__host__ __device__ inline Src src(const void* base, int bf16, int64_t sz, int64_t so, int64_t sk, int outer_dim,
                                   int K, int xf = 0, const float* coef = nullptr, int64_t cz = 0,
                                   float scale = 1.0f) {
  Src s;
  s.base = base;
  s.bf16 = bf16;
  s.sz = sz;
  s.so = so;
  s.sk = sk;
  s.outer_dim = outer_dim;
  s.K = K;
  s.xf = xf;
  s.coef = coef;
  s.cz = cz;
  s.scale = scale;
  s.gofs = 0;
  return s;
}
// the gated hidden activation silu(Z1) * Z3 of rows laid out as [Z1 | Z3] (Z3 at offset gofs)
__host__ __device__ inline Src gated(const float* base, int64_t sz, int64_t so, int64_t sk, int outer_dim, int K,
                                     int64_t gofs) {
  Src s = src(base, 0, sz, so, sk, outer_dim, K, 3);
  s.gofs = gofs;
  return s;
}

// Up to three sources concatenated along k: [0, k1) from a, [k1, k2) from b, [k2, K) from c.
struct Cat {
  Src a, b, c;
  int k1, k2, K;
  __device__ __forceinline__ void load8(int z, int outer, int k0, float* v) const {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int k = k0 + u;
      float x = 0.0f;
      if (k < k1) x = a.get(z, outer, k);
      else if (k < k2) x = b.get(z, outer, k - k1);
      else if (k < K) x = c.get(z, outer, k - k2);
      v[u] = x;
    }
  }
};
inline Cat cat1(const Src& a) { return Cat{a, a, a, a.K, a.K, a.K}; }
inline Cat cat2(const Src& a, const Src& b, int k1) { return Cat{a, b, b, k1, k1 + b.K, k1 + b.K}; }
inline Cat cat3(const Src& a, const Src& b, const Src& c, int k1, int k2) {
  return Cat{a, b, c, k1, k2, k2 + c.K};
}

// ---------------------------------------------------------------------------- epilogues

struct EpiSt {  // out[z * sz + row * ld + col]
  float* out;
  int64_t sz;
  int ld;
  __device__ __forceinline__ void operator()(int z, int row, int col, float v) const {
    out[(int64_t)z * sz + (int64_t)row * ld + col] = v;
  }
};
struct EpiE {  // E = 2 (acc - V), or 2 (acc + X - V) for the residual memory (X: the key features, din = dv)
  float* E;
  int64_t ez;
  const void* V;
  int bf16;
  int64_t vz;  // V element stride per memory; V already offset to the chunk's first row
  int dv;
  const void* X;  // null unless residual: rows of dv elements, stride xz per memory
  int xbf16;
  int64_t xz;
  struct Pre {
    float vv, xv;
  };
  __device__ __forceinline__ Pre load(int z, int row, int col) const {
    return Pre{load_in(V, (int64_t)z * vz + (int64_t)row * dv + col, bf16),
               X ? load_in(X, (int64_t)z * xz + (int64_t)row * dv + col, xbf16) : 0.0f};
  }
  __device__ __forceinline__ void store(int z, int row, int col, float v, const Pre& p) const {
    E[(int64_t)z * ez + (int64_t)row * dv + col] = 2.0f * (v + p.xv - p.vv);
  }
};
struct EpiPD1 {  // P = acc, D1 = acc * silu'(Z)
  float* P;
  float* D1;
  const float* Z;
  int64_t pz, zz;
  int dh;
  struct Pre {
    float zv;
  };
  __device__ __forceinline__ Pre load(int z, int row, int col) const {
    return Pre{Z[(int64_t)z * zz + (int64_t)row * dh + col]};
  }
  __device__ __forceinline__ void store(int z, int row, int col, float v, const Pre& p) const {
    const int64_t o = (int64_t)z * pz + (int64_t)row * dh + col;
    P[o] = v;
    D1[o] = v * silu_primef_(p.zv);
  }
};
struct EpiEa {  // Ea = Eg + acc (in place), dV = -2 Ea
  float* Ea;
  int64_t ez;
  float* dV;
  int64_t vz;  // dV already offset to the chunk (acc = 0) or not (acc = 1)
  int dv;
  int64_t tau0;  // acc = 1: row r is token tau0 + r; tokens before 0 are dropped, the rest accumulate
  int acc;
  struct Pre {
    float ea, dv_old;
  };
  __device__ __forceinline__ Pre load(int z, int row, int col) const {
    return Pre{Ea[(int64_t)z * ez + (int64_t)row * dv + col],
               (acc && tau0 + row >= 0) ? dV[(int64_t)z * vz + (tau0 + row) * dv + col] : 0.0f};
  }
  __device__ __forceinline__ void store(int z, int row, int col, float v, const Pre& p) const {
    const float e = p.ea + v;
    Ea[(int64_t)z * ez + (int64_t)row * dv + col] = e;
    if (!acc) {
      dV[(int64_t)z * vz + (int64_t)row * dv + col] = -2.0f * e;
    } else if (tau0 + row >= 0) {
      dV[(int64_t)z * vz + (tau0 + row) * dv + col] = p.dv_old + -2.0f * e;
    }
  }
};
struct EpiZa {  // Za = Za1 + acc * silu'(Z) (in place)
  float* Za;
  const float* Z;
  int64_t pz, zz;
  int dh;
  struct Pre {
    float za, zv;
  };
  __device__ __forceinline__ Pre load(int z, int row, int col) const {
    return Pre{Za[(int64_t)z * pz + (int64_t)row * dh + col], Z[(int64_t)z * zz + (int64_t)row * dh + col]};
  }
  __device__ __forceinline__ void store(int z, int row, int col, float v, const Pre& p) const {
    Za[(int64_t)z * pz + (int64_t)row * dh + col] = p.za + v * silu_primef_(p.zv);
  }
};
struct EpiScaleSp {  // out = acc * silu'(Z[row + zr0])
  float* out;
  const float* Z;
  int64_t oz, zz;
  int zr0, dh;
  struct Pre {
    float zv;
  };
  __device__ __forceinline__ Pre load(int z, int row, int col) const {
    return Pre{Z[(int64_t)z * zz + (int64_t)(zr0 + row) * dh + col]};
  }
  __device__ __forceinline__ void store(int z, int row, int col, float v, const Pre& p) const {
    out[(int64_t)z * oz + (int64_t)row * dh + col] = v * silu_primef_(p.zv);
  }
};

struct EpiStAdd {  // out = acc (+ scale * add[z * az + row * ald + col] when add is given)
  float* out;
  int64_t sz;
  int ld;
  const float* add;
  int64_t az;
  int ald;
  float scale;
  int64_t tau0;  // acc = 1: row r goes to row tau0 + r of out, accumulated; rows before 0 dropped
  int acc;
  struct Pre {
    float addv, old;
  };
  __device__ __forceinline__ Pre load(int z, int row, int col) const {
    return Pre{add ? add[(int64_t)z * az + (int64_t)row * ald + col] : 0.0f,
               (acc && tau0 + row >= 0) ? out[(int64_t)z * sz + (tau0 + row) * ld + col] : 0.0f};
  }
  __device__ __forceinline__ void store(int z, int row, int col, float v, const Pre& p) const {
    if (add) v += scale * p.addv;
    if (!acc) {
      out[(int64_t)z * sz + (int64_t)row * ld + col] = v;
    } else if (tau0 + row >= 0) {
      out[(int64_t)z * sz + (tau0 + row) * ld + col] = p.old + v;
    }
  }
};

// Gated memory (rows of Z are [Z1 | Z3], dh each; a = silu(Z1)):
// b = acc (= E W2), D1 = b Z3 silu'(Z1), D3 = b a  -> B [row][dh], D [row][D1 | D3]
struct EpiPDg {
  float* B;
  float* D;
  const float* Z;
  int64_t bz, dzz, zz;
  int dh;
  struct Pre {
    float z1, z3;
  };
  __device__ __forceinline__ Pre load(int z, int row, int col) const {
    const float* zr = Z + (int64_t)z * zz + (int64_t)row * 2 * dh;
    return Pre{zr[col], zr[dh + col]};
  }
  __device__ __forceinline__ void store(int z, int row, int col, float v, const Pre& p) const {
    const float z1 = p.z1, z3 = p.z3;
    B[(int64_t)z * bz + (int64_t)row * dh + col] = v;
    float* dr = D + (int64_t)z * dzz + (int64_t)row * 2 * dh;
    dr[col] = v * z3 * silu_primef_(z1);
    dr[dh + col] = v * siluf_(z1);
  }
};
// H' = acc: Za1 += H' Z3 silu'(Z1), Za3 += H' a (in place)
struct EpiZag {
  float* Za;
  const float* Z;
  int64_t az, zz;
  int dh;
  struct Pre {
    float z1, z3, a1, a3;
  };
  __device__ __forceinline__ Pre load(int z, int row, int col) const {
    const float* zr = Z + (int64_t)z * zz + (int64_t)row * 2 * dh;
    const float* ar = Za + (int64_t)z * az + (int64_t)row * 2 * dh;
    return Pre{zr[col], zr[dh + col], ar[col], ar[dh + col]};
  }
  __device__ __forceinline__ void store(int z, int row, int col, float v, const Pre& p) const {
    const float z1 = p.z1, z3 = p.z3;
    float* ar = Za + (int64_t)z * az + (int64_t)row * 2 * dh;
    ar[col] = p.a1 + v * z3 * silu_primef_(z1);
    ar[dh + col] = p.a3 + v * siluf_(z1);
  }
};
// query rows: hq' = acc (= dY W2): Zq1' = hq' Zq3 silu'(Zq1), Zq3' = hq' silu(Zq1) (Zq: rows zr0..)
struct EpiScaleSpG {
  float* out;
  const float* Z;
  int64_t oz, zz;
  int zr0, dh;
  struct Pre {
    float z1, z3;
  };
  __device__ __forceinline__ Pre load(int z, int row, int col) const {
    const float* zr = Z + (int64_t)z * zz + (int64_t)(zr0 + row) * 2 * dh;
    return Pre{zr[col], zr[dh + col]};
  }
  __device__ __forceinline__ void store(int z, int row, int col, float v, const Pre& p) const {
    const float z1 = p.z1, z3 = p.z3;
    float* o = out + (int64_t)z * oz + (int64_t)row * 2 * dh;
    o[col] = v * z3 * silu_primef_(z1);
    o[dh + col] = v * siluf_(z1);
  }
};

struct EpiAxpy {  // out = alpha * x + beta * acc (out may alias x: same element, same thread)
  float* out;
  const float* x;
  int64_t sz;
  int ld;
  float alpha, beta;
  struct Pre {
    float xv;
  };
  __device__ __forceinline__ Pre load(int z, int row, int col) const {
    return Pre{x ? x[(int64_t)z * sz + (int64_t)row * ld + col] : 0.0f};
  }
  __device__ __forceinline__ void store(int z, int row, int col, float v, const Pre& p) const {
    out[(int64_t)z * sz + (int64_t)row * ld + col] = alpha * p.xv + beta * v;
  }
};
struct EpiAcc {  // out += acc
  float* out;
  int64_t sz;
  int ld;
  struct Pre {
    float old;
  };
  __device__ __forceinline__ Pre load(int z, int row, int col) const {
    return Pre{out[(int64_t)z * sz + (int64_t)row * ld + col]};
  }
  __device__ __forceinline__ void store(int z, int row, int col, float v, const Pre& p) const {
    out[(int64_t)z * sz + (int64_t)row * ld + col] = p.old + v;
  }
};

// ---------------------------------------------------------------------------- small kernels

__device__ __forceinline__ float silu_second(float z) {
  const float s = sigmoidf_(z);
  return s * (1.0f - s) * (2.0f + z * (1.0f - 2.0f * s));
}

// Per (row, memory): the coefficient adjoints and the elementwise adjoints (see the header).
// Each lane reads and then overwrites only its own elements.  With use_s = 0 (per-chunk gates:
// cS = 0, the momentum adjoint is folded into the gradient adjoint) U1s and U2s are not read.
__global__ void row_kernel(const float* __restrict__ Z, int64_t zz, float* __restrict__ Pz, const float* __restrict__ D1,
                           float* __restrict__ U1, float* __restrict__ U1s, const float* __restrict__ E,
                           float* __restrict__ U2, const float* __restrict__ U2s, int64_t hz, int64_t vz, int dh,
                           int dv, int C, const float* __restrict__ cW, const float* __restrict__ cS,
                           float* __restrict__ cWa, float* __restrict__ cSa, int use_s) {
  const int r = blockIdx.x, z = blockIdx.y, lane = threadIdx.x;
  const int64_t ho = (int64_t)z * hz + (int64_t)r * dh, vo = (int64_t)z * vz + (int64_t)r * dv;
  float s1 = 0.0f, s1s = 0.0f, s2 = 0.0f, s2s = 0.0f;
  for (int j = lane; j < dh; j += 64) {
    s1 += D1[ho + j] * U1[ho + j];
    if (use_s) s1s += D1[ho + j] * U1s[ho + j];
  }
  for (int j = lane; j < dv; j += 64) {
    s2 += E[vo + j] * U2[vo + j];
    if (use_s) s2s += E[vo + j] * U2s[vo + j];
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    s1 += __shfl_xor(s1, off, 64);
    s1s += __shfl_xor(s1s, off, 64);
    s2 += __shfl_xor(s2, off, 64);
    s2s += __shfl_xor(s2s, off, 64);
  }
  const float cw = cW[(int64_t)z * C + r], cs = cS[(int64_t)z * C + r];
  if (lane == 0) {
    cWa[(int64_t)z * C + r] = -(s1 + s2);
    cSa[(int64_t)z * C + r] = -(s1s + s2s);
  }
  for (int j = lane; j < dh; j += 64) {
    const float zv = Z[(int64_t)z * zz + (int64_t)r * dh + j];
    const float d1a = -(cw * U1[ho + j] + (use_s ? cs * U1s[ho + j] : 0.0f));
    const float p = Pz[ho + j];
    U1s[ho + j] = d1a * silu_primef_(zv);  // P'
    Pz[ho + j] = d1a * p * silu_second(zv);  // Z'_1
  }
  for (int j = lane; j < dv; j += 64) U2[vo + j] = -(cw * U2[vo + j] + (use_s ? cs * U2s[vo + j] : 0.0f));  // E'_g
}

// The linear memory's rows (g_r = E_r x_r^T, E = 2 (X W^T - V)): with U = X WA^T and Us = X SA^T,
// the coefficient adjoints -<E_r, U_r>, -<E_r, Us_r> and E'_r = -(oW_r U_r + oS_r Us_r) (in U), and
// dV = -2 E' (row r is token tau0 + r when acc, accumulated, tokens before 0 dropped; else row r
// of the chunk's dV).
__global__ void lin_row_kernel(const float* __restrict__ E, float* __restrict__ U, const float* __restrict__ Us,
                               int64_t vz, int dv, int ld, const float* __restrict__ rW, const float* __restrict__ rS,
                               float* __restrict__ cWa, float* __restrict__ cSa, float* __restrict__ dV, int64_t dvz,
                               int64_t tau0, int acc) {
  const int r = blockIdx.x, z = blockIdx.y, lane = threadIdx.x;
  const int64_t o = (int64_t)z * vz + (int64_t)r * dv;
  float a = 0.0f, b = 0.0f;
  for (int j = lane; j < dv; j += 64) {
    a += E[o + j] * U[o + j];
    b += E[o + j] * Us[o + j];
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    a += __shfl_xor(a, off, 64);
    b += __shfl_xor(b, off, 64);
  }
  if (lane == 0) {
    cWa[(int64_t)z * ld + r] = -a;
    cSa[(int64_t)z * ld + r] = -b;
  }
  const float w = rW[(int64_t)z * ld + r], sv = rS[(int64_t)z * ld + r];
  for (int j = lane; j < dv; j += 64) {
    const float ea = -(w * U[o + j] + sv * Us[o + j]);
    U[o + j] = ea;
    if (!acc) dV[(int64_t)z * dvz + (int64_t)r * dv + j] = -2.0f * ea;
    else if (tau0 + r >= 0) dV[(int64_t)z * dvz + (tau0 + r) * dv + j] += -2.0f * ea;
  }
}

// The gated memory's rows: coefficient adjoints -(<D, U1> + <E, U2>) (D = [D1 | D3], dz = 2 dh
// wide) and likewise with U1s, U2s; D' = -(cW U1 + cS U1s), then
//   b' = D1' Z3 s'(Z1) + D3' a                     (into U1s[:, :dh])
//   Za1 = D1' b Z3 s''(Z1) + D3' b s'(Z1),  Za3 = D1' b s'(Z1)   (into Za)
//   E'_g = -(cW U2 + cS U2s)                       (in U2)
// Each lane reads and then overwrites only its own elements (j and dh + j together).
__global__ void row_kernel_gated(const float* __restrict__ Z, int64_t zz, const float* __restrict__ B,
                                 int64_t bz, const float* __restrict__ D, float* __restrict__ U1,
                                 float* __restrict__ U1s, int64_t uz, float* __restrict__ Za,
                                 const float* __restrict__ E, float* __restrict__ U2, const float* __restrict__ U2s,
                                 int64_t vz, int dh, int dv, int C, const float* __restrict__ cW,
                                 const float* __restrict__ cS, float* __restrict__ cWa, float* __restrict__ cSa) {
  const int r = blockIdx.x, z = blockIdx.y, lane = threadIdx.x, dz = 2 * dh;
  const int64_t ho = (int64_t)z * uz + (int64_t)r * dz, vo = (int64_t)z * vz + (int64_t)r * dv;
  float s1 = 0.0f, s1s = 0.0f, s2 = 0.0f, s2s = 0.0f;
  for (int j = lane; j < dz; j += 64) {
    s1 += D[ho + j] * U1[ho + j];
    s1s += D[ho + j] * U1s[ho + j];
  }
  for (int j = lane; j < dv; j += 64) {
    s2 += E[vo + j] * U2[vo + j];
    s2s += E[vo + j] * U2s[vo + j];
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    s1 += __shfl_xor(s1, off, 64);
    s1s += __shfl_xor(s1s, off, 64);
    s2 += __shfl_xor(s2, off, 64);
    s2s += __shfl_xor(s2s, off, 64);
  }
  const float cw = cW[(int64_t)z * C + r], cs = cS[(int64_t)z * C + r];
  if (lane == 0) {
    cWa[(int64_t)z * C + r] = -(s1 + s2);
    cSa[(int64_t)z * C + r] = -(s1s + s2s);
  }
  const float* zr = Z + (int64_t)z * zz + (int64_t)r * dz;
  const float* br = B + (int64_t)z * bz + (int64_t)r * dh;
  for (int j = lane; j < dh; j += 64) {
    const float z1 = zr[j], z3 = zr[dh + j], b = br[j];
    const float sg = sigmoidf_(z1), a = z1 * sg;
    const float sp = sg * (1.0f + z1 * (1.0f - sg)), spp = silu_second(z1);
    const float d1a = -(cw * U1[ho + j] + cs * U1s[ho + j]);
    const float d3a = -(cw * U1[ho + dh + j] + cs * U1s[ho + dh + j]);
    U1s[ho + j] = d1a * z3 * sp + d3a * a;  // b'
    Za[ho + j] = d1a * b * z3 * spp + d3a * b * sp;
    Za[ho + dh + j] = d1a * b * sp;
  }
  for (int j = lane; j < dv; j += 64) U2[vo + j] = -(cw * U2[vo + j] + cs * U2s[vo + j]);  // E'_g
}

// beta' = <WA, W>, aS' = <WA, S>, PC' = <SA, S> per memory; ck: [M][2P] (W then S).
__global__ void __launch_bounds__(1024) scalar_adj_kernel(const float* __restrict__ WA, const float* __restrict__ SA,
                                  const float* __restrict__ ck, int64_t P, float* __restrict__ out) {
  __shared__ float red[3][16];  // one slot per wave (up to 1024 threads)
  const int z = blockIdx.x;
  const float* w = ck + (int64_t)z * 2 * P;
  const float* s = w + P;
  const float* wa = WA + (int64_t)z * P;
  const float* sa = SA + (int64_t)z * P;
  float b = 0.0f, a = 0.0f, p = 0.0f;
  int64_t i0 = 0;
  if (((P & 3) == 0) && ((((uintptr_t)w) | ((uintptr_t)wa) | ((uintptr_t)sa)) & 15) == 0) {
    // 16-byte loads, four per array in flight per thread
    const int64_t n4 = P / 4;
#pragma unroll 4
    for (int64_t q = threadIdx.x; q < n4; q += blockDim.x) {
      const float4 x = ((const float4*)w)[q], y = ((const float4*)s)[q];
      const float4 u = ((const float4*)wa)[q], v = ((const float4*)sa)[q];
      b += u.x * x.x + u.y * x.y + u.z * x.z + u.w * x.w;
      a += u.x * y.x + u.y * y.y + u.z * y.z + u.w * y.w;
      p += v.x * y.x + v.y * y.y + v.z * y.z + v.w * y.w;
    }
    i0 = P;
  }
  for (int64_t i = i0 + threadIdx.x; i < P; i += blockDim.x) {
    b += wa[i] * w[i];
    a += wa[i] * s[i];
    p += sa[i] * s[i];
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    b += __shfl_xor(b, off, 64);
    a += __shfl_xor(a, off, 64);
    p += __shfl_xor(p, off, 64);
  }
  const int wv = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    red[0][wv] = b;
    red[1][wv] = a;
    red[2][wv] = p;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    const int nw = blockDim.x >> 6;
    float s0 = 0.0f, s1 = 0.0f, s2 = 0.0f;
    for (int q = 0; q < nw; ++q) {
      s0 += red[2][q];
      s1 += red[0][q];
      s2 += red[1][q];
    }
    out[z * 3 + 0] = s0;  // PC'
    out[z * 3 + 1] = s1;  // beta'
    out[z * 3 + 2] = s2;  // aS'
  }
}

// Reverse of the gate scan for one chunk of every memory (thread 0 of a block per memory walks the
// chunk's two recurrences, the block's threads share out the per-step terms between them; e, b, w
// recomputed in LDS):  e_{C-1} = b_{C-1} = w_{C-1} = 1, e_r = eta_{r+1} e_{r+1},
// b_r = (1 - alpha_{r+1}) b_{r+1}, w_r = b_r + eta_{r+1} w_{r+1}, cS = theta e, cW = theta w,
// PC = eta_0 e_0, beta = (1 - alpha_0) b_0, aS = eta_0 w_0.
constexpr int kGateBwdMaxC = 1024;  // the largest chunk a configuration may ask for
__global__ void gate_bwd_kernel(const float* __restrict__ theta, const float* __restrict__ eta,
                                const float* __restrict__ alpha, int64_t ld, int64_t s0, int C,
                                const float* __restrict__ cWa, const float* __restrict__ cSa,
                                const float* __restrict__ sca, float* __restrict__ dth, float* __restrict__ det,
                                float* __restrict__ dal) {
  // e, b, w, ea, wa, the chunk's theta, the coefficient adjoints cw, cs and the output oth [C]
  // each in the dynamic LDS block; eta and alpha (which the two recurrences only read) and their
  // outputs oet, oal (which the second only writes) in arrays of their own, so that the compiler
  // may issue a step's LDS loads ahead of the previous steps' stores.  The block loads and stores
  // them in parallel, and thread 0 runs the recurrences without a global access.
  extern __shared__ float gb[];
  __shared__ float et[kGateBwdMaxC], al[kGateBwdMaxC], oet[kGateBwdMaxC], oal[kGateBwdMaxC];
  const int z = blockIdx.x;
  float* e = gb;
  float* b = gb + C;
  float* w = gb + 2 * C;
  float* ea = gb + 3 * C;
  float* wa = gb + 4 * C;
  float* th = gb + 5 * C;
  float* cwv = gb + 6 * C;
  float* csv = gb + 7 * C;
  float* oth = gb + 8 * C;
  for (int r = threadIdx.x; r < C; r += blockDim.x) {
    const int64_t o = (int64_t)z * ld + s0 + r;
    th[r] = theta[o];
    et[r] = eta[o];
    al[r] = alpha[o];
    cwv[r] = cWa[(int64_t)z * C + r];
    csv[r] = cSa[(int64_t)z * C + r];
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    // the recurrences carry their running values in registers; the loads they need do not
    // depend on the chain
    float ec = 1.0f, bc = 1.0f, wc = 1.0f;
    e[C - 1] = b[C - 1] = w[C - 1] = 1.0f;
#pragma unroll 4
    for (int r = C - 2; r >= 0; --r) {
      const float etn = et[r + 1], aln = al[r + 1];
      ec = etn * ec;
      bc = (1.0f - aln) * bc;
      wc = bc + etn * wc;
      e[r] = ec;
      b[r] = bc;
      w[r] = wc;
    }
  }
  __syncthreads();
  for (int r = threadIdx.x; r < C; r += blockDim.x) {  // per-step terms: every thread
    const float cw = cwv[r], cs = csv[r];
    oth[r] = cs * e[r] + cw * w[r];
    ea[r] = cs * th[r];
    wa[r] = cw * th[r];
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    const float PCa = sca[z * 3 + 0], betaa = sca[z * 3 + 1], aSa = sca[z * 3 + 2];
    oet[0] = PCa * e[0] + aSa * w[0];
    float ea_c = ea[0] + PCa * et[0];
    float wa_c = wa[0] + aSa * et[0];
    oal[0] = -betaa * b[0];
    float ba_c = betaa * (1.0f - al[0]);
#pragma unroll 4
    for (int r = 0; r + 1 < C; ++r) {
      const float w1 = w[r + 1], e1 = e[r + 1], et1 = et[r + 1], b1 = b[r + 1], al1 = al[r + 1];
      const float wan = wa[r + 1], ean = ea[r + 1];
      ba_c += wa_c;
      oet[r + 1] = wa_c * w1 + ea_c * e1;
      wa_c = wan + wa_c * et1;
      ea_c = ean + ea_c * et1;
      oal[r + 1] = -ba_c * b1;
      ba_c = ba_c * (1.0f - al1);
    }
  }
  __syncthreads();
  for (int r = threadIdx.x; r < C; r += blockDim.x) {
    const int64_t o = (int64_t)z * ld + s0 + r;
    dth[o] = oth[r];
    det[o] = oet[r];
    dal[o] = oal[r];
  }
}

// WA <- beta WA + Wb, SA <- aS WA + PC SA (per memory scalars sc = (PC, beta, aS)), into the other
// buffers of the ping-pong pair.
__global__ void state_adj_kernel(const float* __restrict__ WA, const float* __restrict__ SA,
                                 const float* __restrict__ Wb, const float* __restrict__ sc, int64_t P, int M,
                                 float* __restrict__ WAn, float* __restrict__ SAn) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)M * P) return;
  const int64_t z = i / P;
  const float pc = sc[z * 3 + 0], beta = sc[z * 3 + 1], aS = sc[z * 3 + 2];
  const float wa = WA[i];
  WAn[i] = beta * wa + Wb[i];
  SAn[i] = aS * wa + pc * SA[i];
}

// Omega window (per-token gates, window c): key row r of the chunk at token s is token
// tau = s - (c - 1) + r; rows before the call come from the window history the call started with
// (hv, hg: [M][c - 1][*], oldest first).  Values and gamma of the R rows to fp32 staging.
__global__ void stage_vg_kernel(const void* __restrict__ V, const float* __restrict__ gamma, int bf16, int64_t T,
                                int64_t s, int c, int R, int dv, const float* __restrict__ hv,
                                const float* __restrict__ hg, float* __restrict__ vs, float* __restrict__ gs) {
  const int r = blockIdx.x, z = blockIdx.y, H = c - 1;
  const int64_t tau = s - H + r;
  const int64_t row = (int64_t)z * R + r;
  for (int e = threadIdx.x; e < dv; e += blockDim.x)
    vs[row * dv + e] = tau >= 0 ? load_in(V, ((int64_t)z * T + tau) * dv + e, bf16)
                                : hv[((int64_t)z * H + H + tau) * dv + e];
  if (threadIdx.x == 0) gs[row] = tau >= 0 ? gamma[(int64_t)z * T + tau] : hg[(int64_t)z * H + H + tau];
}

// Feature rows phi(x) of `rows` consecutive tokens tau0 + r of every memory (identity for degree 1;
// degree 2: 1, x_i, x_i x_j / 2 for i <= j in combinations_with_replacement order), the raw row
// from X (tau >= 0) or from the window history hist ([M][H][dk], tau < 0), to out [M][rows][din].
__global__ void stage_feat_kernel(const void* __restrict__ X, int bf16, int64_t T, int64_t tau0, int rows, int dk,
                                  int din, int poly, const float* __restrict__ hist, int H, float* __restrict__ out) {
  extern __shared__ float xr[];  // the raw row
  const int r = blockIdx.x, z = blockIdx.y;
  const int64_t tau = tau0 + r;
  for (int e = threadIdx.x; e < dk; e += blockDim.x)
    xr[e] = tau >= 0 ? load_in(X, ((int64_t)z * T + tau) * dk + e, bf16) : hist[((int64_t)z * H + H + tau) * dk + e];
  __syncthreads();
  float* o = out + ((int64_t)z * rows + r) * din;
  for (int f = threadIdx.x; f < din; f += blockDim.x) {
    float v;
    if (poly == 1) {
      v = xr[f];
    } else if (f == 0) {
      v = 1.0f;
    } else if (f <= dk) {
      v = xr[f - 1];
    } else {
      int i, j;
      pair_of(f - 1 - dk, dk, i, j);
      v = 0.5f * (xr[i] * xr[j]);
    }
    o[f] = v;
  }
}

// The gradient of the raw rows from that of their degree-2 features: phi's monomials of degree 1
// give 1, x_i^2 / 2 gives x_i, x_i x_j / 2 (i < j) gives x_j / 2 to x_i, so
// dx_i = g_{1+i} + g_{ii} x_i + sum_{j != i} g_{ij} x_j / 2  (x_j read back from the features).
// Row r is token tau0 + r of out ([M][T][dk]); acc: accumulated (tokens before 0 dropped).
__global__ void feat_jac_kernel(const float* __restrict__ G, const float* __restrict__ F, int rows, int dk, int din,
                                int64_t T, int64_t tau0, int acc, float* __restrict__ out) {
  const int r = blockIdx.x, z = blockIdx.y;
  const int64_t tau = tau0 + r;
  if (tau < 0) return;
  const float* g = G + ((int64_t)z * rows + r) * din;
  const float* x = F + ((int64_t)z * rows + r) * din + 1;  // the degree-1 features are the raw row
  for (int i = threadIdx.x; i < dk; i += blockDim.x) {
    float v = g[1 + i];
    for (int j = 0; j < dk; ++j) {
      const int a = i < j ? i : j, b = i < j ? j : i;
      const float gp = g[1 + dk + pair_start(a, dk) + (b - a)];
      v += (i == j ? 1.0f : 0.5f) * gp * x[j];
    }
    float* o = out + ((int64_t)z * T + tau) * dk + i;
    if (acc) *o += v;
    else *o = v;
  }
}

// The coefficients of the key rows' gradients: g_r enters every step t of the chunk whose window
// holds it, so oW_r = gamma_r * sum_{t = max(j, 0)}^{min(j + c - 1, C - 1)} cW_t with j = r - (c - 1)
// (oS likewise); the window sums are kept for the adjoint.
__global__ void omega_coef_kernel(const float* __restrict__ cW, const float* __restrict__ cS,
                                  const float* __restrict__ gs, int C, int c, int R, int M, float* __restrict__ oW,
                                  float* __restrict__ oS, float* __restrict__ sW, float* __restrict__ sS) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)M * R) return;
  const int64_t z = i / R;
  const int r = (int)(i - z * R), j = r - (c - 1);
  const int t0 = j > 0 ? j : 0, t1 = j + c - 1 < C - 1 ? j + c - 1 : C - 1;
  float a = 0.0f, b = 0.0f;
  for (int t = t0; t <= t1; ++t) {
    a += cW[z * C + t];
    b += cS[z * C + t];
  }
  sW[i] = a;
  sS[i] = b;
  oW[i] = gs[i] * a;
  oS[i] = gs[i] * b;
}

// Its adjoint: cW'_t = sum_{r = t}^{t + c - 1} gamma_r oW'_r (cS' likewise) for the chunk's C tokens,
// and gamma'_r += oW'_r sW_r + oS'_r sS_r for the rows that are tokens of the call.
__global__ void omega_adj_kernel(const float* __restrict__ oWa, const float* __restrict__ oSa,
                                 const float* __restrict__ gs, const float* __restrict__ sW,
                                 const float* __restrict__ sS, int C, int c, int R, int M, int64_t T, int64_t s,
                                 float* __restrict__ cWa, float* __restrict__ cSa, float* __restrict__ dgamma) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)M * R) return;
  const int64_t z = i / R;
  const int r = (int)(i - z * R);
  const int64_t tau = s - (c - 1) + r;
  if (tau >= 0) dgamma[z * T + tau] += oWa[i] * sW[i] + oSa[i] * sS[i];
  if (r < C) {
    float a = 0.0f, b = 0.0f;
    for (int q = r; q < r + c; ++q) {
      a += gs[z * R + q] * oWa[z * R + q];
      b += gs[z * R + q] * oSa[z * R + q];
    }
    cWa[z * C + r] = a;
    cSa[z * C + r] = b;
  }
}

// Fill n floats with v.
__global__ void fill_kernel(float* __restrict__ p, int64_t n, float v) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

// The chunk-start state of memories m = y, y + gridDim.y, ... into the checkpoint rows:
// ck[m][0, P) = W[m], ck[m][P, 2P) = S[m] (one launch for both, in place of two strided copies).
__global__ void checkpoint_kernel(const float* __restrict__ W, const float* __restrict__ S, int64_t P, int64_t M,
                                  float* __restrict__ ck) {
  const int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (r >= P) return;
  for (int64_t m = blockIdx.y; m < M; m += gridDim.y) {
    ck[m * 2 * P + r] = W[m * P + r];
    ck[m * 2 * P + P + r] = S[m * P + r];
  }
}

// Per-chunk gates: SAt = SA + WA (S_end also feeds W_end); per memory the gate adjoints
// theta' = -<SAt, N>, eta' = <SAt, S0>, alpha' = -<WA, W0> at chunk k of the [M][ldg] gate arrays.
__global__ void chunk_gate_adj_kernel(const float* __restrict__ WA, const float* __restrict__ SA,
                                      const float* __restrict__ N, const float* __restrict__ ck, int64_t P,
                                      float* __restrict__ SAt, int64_t ldg, int64_t k, float* __restrict__ dth,
                                      float* __restrict__ det, float* __restrict__ dal) {
  __shared__ float red[3][4];
  const int z = blockIdx.x;
  const float* w0 = ck + (int64_t)z * 2 * P;
  const float* s0 = w0 + P;
  const int64_t o = (int64_t)z * P;
  float t = 0.0f, e = 0.0f, a = 0.0f;
  int64_t i0 = 0;
  if (((P & 3) == 0) && ((((uintptr_t)(WA + o)) | ((uintptr_t)(SA + o)) | ((uintptr_t)(N + o)) |
                          ((uintptr_t)(SAt + o)) | ((uintptr_t)w0)) & 15) == 0) {
    // 16-byte loads and stores, four iterations' loads in flight per thread (the SAt stores
    // would otherwise keep each iteration's loads behind the previous one's store)
    const int64_t n4 = P / 4;
    const float4* wa4 = (const float4*)(WA + o);
    const float4* sa4 = (const float4*)(SA + o);
    const float4* n_4 = (const float4*)(N + o);
    const float4* w04 = (const float4*)w0;
    const float4* s04 = (const float4*)s0;
    float4* st4 = (float4*)(SAt + o);
    for (int64_t q0 = threadIdx.x; q0 < n4; q0 += 4 * (int64_t)blockDim.x) {
      float4 u[4], v[4], nn[4], x[4], y[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t q = q0 + (int64_t)j * blockDim.x;
        if (q < n4) {
          u[j] = wa4[q];
          v[j] = sa4[q];
          nn[j] = n_4[q];
          x[j] = w04[q];
          y[j] = s04[q];
        }
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t q = q0 + (int64_t)j * blockDim.x;
        if (q < n4) {
          const float4 s = make_float4(v[j].x + u[j].x, v[j].y + u[j].y, v[j].z + u[j].z, v[j].w + u[j].w);
          st4[q] = s;
          t += s.x * nn[j].x + s.y * nn[j].y + s.z * nn[j].z + s.w * nn[j].w;
          e += s.x * y[j].x + s.y * y[j].y + s.z * y[j].z + s.w * y[j].w;
          a += u[j].x * x[j].x + u[j].y * x[j].y + u[j].z * x[j].z + u[j].w * x[j].w;
        }
      }
    }
    i0 = P;
  }
  for (int64_t i = i0 + threadIdx.x; i < P; i += blockDim.x) {
    const float sat = SA[o + i] + WA[o + i];
    SAt[o + i] = sat;
    t += sat * N[o + i];
    e += sat * s0[i];
    a += WA[o + i] * w0[i];
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    t += __shfl_xor(t, off, 64);
    e += __shfl_xor(e, off, 64);
    a += __shfl_xor(a, off, 64);
  }
  const int wv = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    red[0][wv] = t;
    red[1][wv] = e;
    red[2][wv] = a;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    dth[(int64_t)z * ldg + k] = -(red[0][0] + red[0][1] + red[0][2] + red[0][3]);
    det[(int64_t)z * ldg + k] = red[1][0] + red[1][1] + red[1][2] + red[1][3];
    dal[(int64_t)z * ldg + k] = -(red[2][0] + red[2][1] + red[2][2] + red[2][3]);
  }
}

// Per-chunk state carry: WA <- (1 - alpha_k) WA + Wb, SA <- eta_k SAt.
__global__ void chunk_state_adj_kernel(const float* __restrict__ WA, const float* __restrict__ SAt,
                                       const float* __restrict__ Wb, const float* __restrict__ eta,
                                       const float* __restrict__ alpha, int64_t ldg, int64_t k, int64_t P, int M,
                                       float* __restrict__ WAn, float* __restrict__ SAn) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)M * P) return;
  const int64_t z = i / P;
  const float om = 1.0f - alpha[z * ldg + k], et = eta[z * ldg + k];
  WAn[i] = om * WA[i] + Wb[i];
  SAn[i] = et * SAt[i];
}

// Per memory: <a, b> over n elements at a + z * za and b + z * zb (|G|_F^2 with a = b).
__global__ void dot_kernel(const float* __restrict__ a, int64_t za, const float* __restrict__ b, int64_t zb, int64_t n,
                           float* __restrict__ out) {
  __shared__ float red[4];
  const int z = blockIdx.x;
  float acc = 0.0f;
  for (int64_t i = threadIdx.x; i < n; i += blockDim.x) acc += a[(int64_t)z * za + i] * b[(int64_t)z * zb + i];
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) out[z] = red[0] + red[1] + red[2] + red[3];
}

// Geometry of one Newton-Schulz batch: slab z is matrix z / M (of nm <= 3 matrices that share the
// working shape r x c) of memory z % M.  Matrix i lies at goff[i] in a memory's P parameters as
// rows x cols; its working orientation is transposed when rows > cols.
struct NsGeo {
  int M, nm;
  int64_t P;
  int64_t goff[3];
  int rows[3], cols[3], tr[3];
};

// Element i of the batch (slab z, element e of the matrix in its own orientation): its index in
// the parameter layout and in a working slab of stride xz.
struct NsIdx {
  int64_t z, g, w;
};
__device__ __forceinline__ NsIdx ns_idx(const NsGeo& g, int64_t i, int64_t n, int64_t xz) {
  const int64_t z = i / n, e = i - z * n;
  const int mi = (int)(z / g.M);
  const int64_t zm = z - (int64_t)mi * g.M;
  const int r = (int)(e / g.cols[mi]), c = (int)(e - (int64_t)r * g.cols[mi]);
  return NsIdx{z, zm * g.P + g.goff[mi] + e, z * xz + (g.tr[mi] ? (int64_t)c * g.rows[mi] + r : e)};
}

// |G|^2 of every slab (one block each)
__global__ void ns_gsq_kernel(NsGeo g, const float* __restrict__ G, float* __restrict__ out) {
  __shared__ float red[4];
  const int z = blockIdx.x, mi = z / g.M;
  const float* p = G + (int64_t)(z - mi * g.M) * g.P + g.goff[mi];
  const int64_t n = (int64_t)g.rows[mi] * g.cols[mi];
  float acc = 0.0f;
  for (int64_t i = threadIdx.x; i < n; i += blockDim.x) acc += p[i] * p[i];
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) out[z] = red[0] + red[1] + red[2] + red[3];
}

// X0 = G / (|G| + eps) in the working orientation.
__global__ void ns_init_kernel(NsGeo g, const float* __restrict__ G, const float* __restrict__ sq, float eps,
                               float* __restrict__ X, int64_t xz, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)g.nm * g.M * n) return;
  const NsIdx x = ns_idx(g, i, n, xz);
  X[x.w] = G[x.g] * (1.0f / (sqrtf(sq[x.z]) + eps));
}

// G' = Xa0 / n - (<Xa0, G> / n^2) G / |G|, Xa0 taken back to G's orientation; n = |G| + eps.
// With G null the kernel copies a working slab back to G's orientation (Ga = Xa).
__global__ void ns_final_kernel(NsGeo g, const float* __restrict__ Xa, int64_t xz, const float* __restrict__ G,
                                const float* __restrict__ sq, const float* __restrict__ dotv, float eps,
                                float* __restrict__ Ga, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)g.nm * g.M * n) return;
  const NsIdx x = ns_idx(g, i, n, xz);
  const float xa = Xa[x.w];
  if (!G) {
    Ga[x.g] = xa;
    return;
  }
  const float gn = sqrtf(sq[x.z]), nn = gn + eps;
  const float corr = gn > 0.0f ? dotv[x.z] / (nn * gn) : 0.0f;  // dotv = <Xa0, X0> = <Xa0, G> / nn
  Ga[x.g] = xa / nn - corr * G[x.g];
}

// A parameter-layout matrix to its working slab (the adjoint of N entering the reverse).
__global__ void ns_to_work_kernel(NsGeo g, const float* __restrict__ in, float* __restrict__ out, int64_t xz,
                                  int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)g.nm * g.M * n) return;
  const NsIdx x = ns_idx(g, i, n, xz);
  out[x.w] = in[x.g];
}

// The other direction of the orientation change: out (working, [M][r][c]) from in (G's
// orientation, [rows][cols]), times `scale` per memory (scale[z] * mul), or a plain copy.
__global__ void to_work_kernel(const float* __restrict__ in, int64_t iz, int rows, int cols, int tr,
                               const float* __restrict__ scale, int64_t sld, int64_t sk, float mul,
                               float* __restrict__ out, int64_t oz, int M) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t n = (int64_t)rows * cols;
  if (i >= (int64_t)M * n) return;
  const int64_t z = i / n, e = i - z * n;
  const int r = (int)(e / cols), c = (int)(e - (int64_t)r * cols);
  const float f = scale ? scale[z * sld + sk] * mul : mul;
  const float v = in[z * iz + e] * f;
  if (tr) out[z * oz + (int64_t)c * rows + r] = v;
  else out[z * oz + e] = v;
}

}  // namespace bk

// ---------------------------------------------------------------------------- host

struct NsLay {  // Newton-Schulz buffers of g.nm matrices of one working shape r x c (r <= c), batched
  bk::NsGeo g;
  int r, c;
  int64_t x, a, b, xa0, xa1, ba, aa, sq, dot;
};

struct BwdLayout {
  int64_t ck, wa0, wa1, sa0, sa1, wb, zk, e, pz, d1, u1, u1s, u2, u2s, zqa, cw, cs, cwa, csa, sc, sca;
  int64_t R;  // key rows per chunk: C, or C + c - 1 with an Omega window
  int64_t ow, os, sw, ss, cwt, cst, ks, vs, gs, hk0, hv0, hg0;  // Omega window buffers
  int64_t qs, xg, qg;  // polynomial features: query features, feature-space gradients of keys / queries
  int64_t za;          // gated memory: the first-layer pre-activation adjoints [R][dz]
  int64_t gb, nb, nab, gab, sat;
  NsLay ns[3];
  int nns;  // Newton-Schulz batches: the matrices (W1, [W3,] W2) grouped by working shape
  int64_t end;
};

static BwdLayout bwd_layout(const Dims& d, int64_t nchunks) {
  const int64_t M = d.M, C = d.C, P = d.P, dh = d.dh, dv = d.dv;
  BwdLayout L;
  const int64_t R = d.c > 1 ? C + d.c - 1 : C;
  L.R = R;
  int64_t o = 0;
  auto take = [&](int64_t floats) {
    const int64_t r = o;
    o += (floats + 63) / 64 * 64;
    return r;
  };
  L.ck = take(nchunks * M * 2 * P);
  L.wa0 = take(M * P);
  L.wa1 = take(M * P);
  L.sa0 = take(M * P);
  L.sa1 = take(M * P);
  L.wb = take(M * P);
  const int64_t dz = d.dz;  // first-layer rows: dh, or 2 dh for the gated memory ([W1; W3])
  L.zk = take(M * (R + C) * dz);
  L.e = take(M * R * dv);
  L.pz = take(M * R * dh);
  L.d1 = take(M * R * dz);
  L.u1 = take(M * R * dz);
  L.u1s = take(M * R * dz);
  L.u2 = take(M * R * dv);
  L.u2s = take(M * R * dv);
  L.zqa = take(M * R * dz);
  L.za = d.gated ? take(M * R * dz) : 0;
  L.cw = take(M * C);
  L.cs = take(M * C);
  L.cwa = take(M * R);
  L.csa = take(M * R);
  L.ow = L.os = L.sw = L.ss = L.cwt = L.cst = L.ks = L.vs = L.gs = L.hk0 = L.hv0 = L.hg0 = 0;
  L.qs = L.xg = L.qg = 0;
  if (d.c > 1 || d.poly > 1) L.ks = take(M * R * d.din);  // staged key rows (features)
  if (d.poly > 1) {
    L.qs = take(M * C * d.din);
    L.xg = take(M * R * d.din);
    L.qg = take(M * C * d.din);
  }
  if (d.c > 1) {
    const int64_t H = d.c - 1;
    L.ow = take(M * R);
    L.os = take(M * R);
    L.sw = take(M * R);
    L.ss = take(M * R);
    L.cwt = take(M * C);
    L.cst = take(M * C);
    L.vs = take(M * R * dv);
    L.gs = take(M * R);
    L.hk0 = take(M * H * d.dk);
    L.hv0 = take(M * H * dv);
    L.hg0 = take(M * H);
  }
  L.sc = take(M * 3);
  L.sca = take(M * 3);
  L.gb = L.nb = L.nab = L.gab = L.sat = 0;
  L.nns = 0;
  for (int m = 0; m < 3; ++m) L.ns[m] = NsLay{};
  if (d.gate_mode == ATLASMEM_PER_CHUNK) {
    L.gb = take(M * P);
    L.nb = take(M * P);
    L.nab = take(M * P);
    L.gab = take(M * P);
    L.sat = take(M * P);
    if (d.ns_steps > 0) {
      const int steps = d.ns_steps;
      // the matrices: W1 [dh][din], W3 [dh][din] (gated, after W1), W2 [dv][dh] at P1
      int nmat = 0, shp[3][2];
      int64_t goff[3];
      shp[nmat][0] = (int)dh; shp[nmat][1] = d.din; goff[nmat++] = 0;
      if (d.gated) { shp[nmat][0] = (int)dh; shp[nmat][1] = d.din; goff[nmat++] = (int64_t)dh * d.din; }
      shp[nmat][0] = (int)dv; shp[nmat][1] = (int)dh; goff[nmat++] = d.P1;
      bool done[3] = {false, false, false};
      L.nns = 0;
      for (int m0 = 0; m0 < nmat; ++m0) {
        if (done[m0]) continue;
        NsLay& n = L.ns[L.nns++];
        n.r = shp[m0][0] < shp[m0][1] ? shp[m0][0] : shp[m0][1];
        n.c = shp[m0][0] < shp[m0][1] ? shp[m0][1] : shp[m0][0];
        n.g.M = (int)M;
        n.g.nm = 0;
        n.g.P = P;
        for (int m = m0; m < nmat; ++m) {  // every remaining matrix of this working shape
          const int wr = shp[m][0] < shp[m][1] ? shp[m][0] : shp[m][1];
          const int wc = shp[m][0] < shp[m][1] ? shp[m][1] : shp[m][0];
          if (done[m] || wr != n.r || wc != n.c) continue;
          done[m] = true;
          const int j = n.g.nm++;
          n.g.goff[j] = goff[m];
          n.g.rows[j] = shp[m][0];
          n.g.cols[j] = shp[m][1];
          n.g.tr[j] = shp[m][0] > shp[m][1];
        }
        const int64_t S = (int64_t)n.g.nm * M;  // slabs
        const int64_t rc = (int64_t)n.r * n.c, rr = (int64_t)n.r * n.r;
        n.x = take(S * (steps + 1) * rc);
        n.a = take(S * steps * rr);
        n.b = take(S * steps * rr);
        n.xa0 = take(S * rc);
        n.xa1 = take(S * rc);
        n.ba = take(S * rr);
        n.aa = take(S * rr);
        n.sq = take(S);
        n.dot = take(S);
      }
    }
  }
  L.end = o;
  return L;
}

static unsigned blocks_of(int64_t n) { return (unsigned)((n + 255) / 256); }

// Newton-Schulz forward of one batch (both matrices of every memory when they share a working
// shape, else one), keeping its iterates: X_0 = G / (|G| + eps)
// (working orientation), A_i = X_i X_i^T, B_i = b A_i + c A_i^2, X_{i+1} = a X_i + B_i X_i; the result
// goes back to G's orientation in N (at the matrix's offset).
// For the 64 x 128 working shape both directions run as one launch each, one workgroup per slab
// (k_nsbwd.hip), with the iterates in the same workspace in that kernel's own layout.
static NsSlabGeo slab_geo(const bk::NsGeo& g) {
  NsSlabGeo s;
  s.M = g.M;
  s.nm = g.nm;
  s.P = g.P;
  for (int i = 0; i < 3; ++i) {
    s.goff[i] = g.goff[i];
    s.tr[i] = g.tr[i];
  }
  return s;
}

static atlasmem_status ns_forward(const Dims& d, float* ws, const NsLay& n, const float* G, float* N, hipStream_t st) {
  const int steps = d.ns_steps, r = n.r, c = n.c, B = n.g.nm * d.M;  // B: slabs of the batch
  const int64_t rc = (int64_t)r * c, rr = (int64_t)r * r;
  const int64_t xz = (steps + 1) * rc, az = steps * rr;
  float *X = ws + n.x, *A = ws + n.a, *Bm = ws + n.b, *sq = ws + n.sq;
  if (ns_slab_supported(r, c, steps))
    return launch_ns_slab_forward(slab_geo(n.g), G, X, A, Bm, sq, N, steps, d.ns_a, d.ns_b, d.ns_c, d.ns_eps, st);
  hipLaunchKernelGGL(bk::ns_gsq_kernel, dim3(B), dim3(256), 0, st, n.g, G, sq);
  hipLaunchKernelGGL(bk::ns_init_kernel, dim3(blocks_of((int64_t)B * rc)), dim3(256), 0, st, n.g, G, sq, d.ns_eps, X,
                     xz, rc);
  AM_LAUNCH_CHECK();
  for (int i = 0; i < steps; ++i) {
    float *Xi = X + i * rc, *Xn = X + (i + 1) * rc, *Ai = A + i * rr, *Bi = Bm + i * rr;
    launch_gemm<false, false>(true, r, r, c, B, bk::cat1(bk::src(Xi, 0, xz, c, 1, r, c)),
                              bk::cat1(bk::src(Xi, 0, xz, c, 1, r, c)), bk::EpiSt{Ai, az, r}, st);
    launch_gemm<false, false>(true, r, r, r, B, bk::cat1(bk::src(Ai, 0, az, r, 1, r, r)),
                              bk::cat1(bk::src(Ai, 0, az, 1, r, r, r)), bk::EpiAxpy{Bi, Ai, az, r, d.ns_b, d.ns_c},
                              st);
    launch_gemm<false, false>(true, r, c, r, B, bk::cat1(bk::src(Bi, 0, az, r, 1, r, r)),
                              bk::cat1(bk::src(Xi, 0, xz, 1, c, c, r)), bk::EpiAxpy{Xn, Xi, xz, c, d.ns_a, 1.0f}, st);
  }
  hipLaunchKernelGGL(bk::ns_final_kernel, dim3(blocks_of((int64_t)B * rc)), dim3(256), 0, st, n.g, X + steps * rc,
                     xz, (const float*)nullptr, sq, sq, d.ns_eps, N, rc);
  AM_LAUNCH_CHECK();
  return ATLASMEM_OK;
}

// Its reverse: from Na (the adjoint of N, G's orientation) to Ga (the adjoint of G):
//   Ba = Xa X_i^T, Xa <- a Xa + B_i Xa + (Aa + Aa^T) X_i with Aa = b Ba + c (Ba A_i + A_i Ba),
//   then G' = Xa0 / n - (<Xa0, G> / n^2) G / |G|.
static atlasmem_status ns_backward(const Dims& d, float* ws, const NsLay& n, const float* G, const float* Na,
                                   float* Ga, hipStream_t st) {
  const int steps = d.ns_steps, r = n.r, c = n.c, B = n.g.nm * d.M;
  const int64_t rc = (int64_t)r * c, rr = (int64_t)r * r;
  const int64_t xz = (steps + 1) * rc, az = steps * rr;
  float *X = ws + n.x, *A = ws + n.a, *Bm = ws + n.b, *Ba = ws + n.ba, *Aa = ws + n.aa;
  if (ns_slab_supported(r, c, steps))
    return launch_ns_slab_reverse(slab_geo(n.g), G, Na, X, A, Bm, ws + n.sq, Ga, steps, d.ns_a, d.ns_b, d.ns_c,
                                  d.ns_eps, st);
  float* xa = ws + n.xa0;
  float* xn = ws + n.xa1;
  hipLaunchKernelGGL(bk::ns_to_work_kernel, dim3(blocks_of((int64_t)B * rc)), dim3(256), 0, st, n.g, Na, xa, rc, rc);
  AM_LAUNCH_CHECK();
  for (int i = steps - 1; i >= 0; --i) {
    float *Xi = X + i * rc, *Ai = A + i * rr, *Bi = Bm + i * rr;
    launch_gemm<false, false>(true, r, r, c, B, bk::cat1(bk::src(xa, 0, rc, c, 1, r, c)),
                              bk::cat1(bk::src(Xi, 0, xz, c, 1, r, c)), bk::EpiSt{Ba, rr, r}, st);
    launch_gemm<false, false>(true, r, c, r, B, bk::cat1(bk::src(Bi, 0, az, r, 1, r, r)),
                              bk::cat1(bk::src(xa, 0, rc, 1, c, c, r)), bk::EpiAxpy{xn, xa, rc, c, d.ns_a, 1.0f}, st);
    launch_gemm<false, false>(
        true, r, r, 2 * r, B, bk::cat2(bk::src(Ba, 0, rr, r, 1, r, r), bk::src(Ai, 0, az, r, 1, r, r), r),
        bk::cat2(bk::src(Ai, 0, az, 1, r, r, r), bk::src(Ba, 0, rr, 1, r, r, r), r),
        bk::EpiAxpy{Aa, Ba, rr, r, d.ns_b, d.ns_c}, st);
    launch_gemm<false, false>(
        true, r, c, 2 * r, B, bk::cat2(bk::src(Aa, 0, rr, r, 1, r, r), bk::src(Aa, 0, rr, 1, r, r, r), r),
        bk::cat2(bk::src(Xi, 0, xz, 1, c, c, r), bk::src(Xi, 0, xz, 1, c, c, r), r), bk::EpiAcc{xn, rc, c}, st);
    float* t = xa;
    xa = xn;
    xn = t;
  }
  hipLaunchKernelGGL(bk::dot_kernel, dim3(B), dim3(256), 0, st, xa, rc, X, xz, rc, ws + n.dot);  // <Xa0, X_0>
  AM_LAUNCH_CHECK();
  hipLaunchKernelGGL(bk::ns_final_kernel, dim3(blocks_of((int64_t)B * rc)), dim3(256), 0, st, n.g, xa, rc, G,
                     ws + n.sq, ws + n.dot, d.ns_eps, Ga, rc);
  AM_LAUNCH_CHECK();
  return ATLASMEM_OK;
}

bool backward_supported(const Dims& d) {
  if (d.kind == ATLASMEM_LINEAR) return !d.ptr && d.poly <= 2 && d.gate_mode == ATLASMEM_PER_TOKEN;
  if (d.prec == 2) return false;  // the 2-layer memories' backward products run in split bf16
  if (d.gated)
    return !d.ptr && d.poly <= 2 && (d.gate_mode == ATLASMEM_PER_CHUNK ? d.c == 1 && d.poly == 1 : d.ns_steps == 0);
  return d.kind == ATLASMEM_MLP2_SILU && !d.ptr && d.poly <= 2 &&
         (d.gate_mode == ATLASMEM_PER_CHUNK ? d.c == 1 && d.poly == 1 : d.ns_steps == 0);
}

int64_t backward_workspace_bytes(const Dims& d, int64_t T) {
  if (T % d.C != 0) return -1;
  return bwd_layout(d, T / d.C).end * (int64_t)sizeof(float);
}

atlasmem_status backward(Handle* h, const void* K, const void* Q, const void* V, const float* theta, const float* eta,
                         const float* alpha, const float* gamma, int64_t T, void* Y, const float* dY,
                         const float* dWT, const float* dST, void* workspace, float* dK, float* dQ, float* dV,
                         float* dth, float* det, float* dal, float* dgamma, float* dW0, float* dS0, hipStream_t st) {
  // split-K scratch for the products with few tiles and long k ranges (the concatenated-k
  // adjoint products), as on the forward path; null for a handle without one
  float* sk = h->d.no_splitk ? nullptr : h->sk;
  const int64_t skf = h->sk_floats;
  const Dims& d = h->d;
  const int M = d.M, C = d.C, dh = d.dh, dv = d.dv, din = d.din;
  const int64_t P = d.P, P1 = d.P1;
  const int64_t nch = T / C;
  const bool per_chunk = d.gate_mode == ATLASMEM_PER_CHUNK;
  const int bf = d.in_bf16;
  const size_t esz = bf ? 2 : 4;
  const BwdLayout L = bwd_layout(d, nch);
  float* ws = (float*)workspace;
  const int c = d.c;
  const bool win = c > 1;          // Omega window: key rows reach c - 1 tokens back, outputs accumulate
  const bool feat = d.poly > 1;    // polynomial features: the memory reads phi(k), phi(q)
  const bool staged = win || feat;  // key rows staged in fp32 (features, window history)
  if (win) {
    // the window history the call starts with (the forward below advances the handle's), and
    // zeroed gradients of the rows that several chunks touch
    const size_t H = (size_t)(c - 1) * M;
    if (hipMemcpyAsync(ws + L.hk0, h->hk[h->hcur], sizeof(float) * H * d.dk, hipMemcpyDeviceToDevice, st) !=
            hipSuccess ||
        hipMemcpyAsync(ws + L.hv0, h->hv[h->hcur], sizeof(float) * H * dv, hipMemcpyDeviceToDevice, st) !=
            hipSuccess ||
        hipMemcpyAsync(ws + L.hg0, h->hg[h->hcur], sizeof(float) * H, hipMemcpyDeviceToDevice, st) != hipSuccess ||
        hipMemsetAsync(dK, 0, sizeof(float) * M * T * d.dk, st) != hipSuccess ||
        hipMemsetAsync(dV, 0, sizeof(float) * M * T * dv, st) != hipSuccess ||
        hipMemsetAsync(dgamma, 0, sizeof(float) * M * T, st) != hipSuccess) {
      (void)hipGetLastError();
      return ATLASMEM_E_DEVICE;
    }
  }
  // ---- forward, saving the state at every chunk start
  for (int64_t k = 0; k < nch; ++k) {
    float* ck = ws + L.ck + k * M * 2 * P;
    hipLaunchKernelGGL(bk::checkpoint_kernel, dim3(blocks_of(P), (unsigned)(M < 65535 ? M : 65535)), dim3(256), 0, st,
                       (const float*)h->W[h->cur], (const float*)h->S[h->cur], (int64_t)P, (int64_t)M, ck);
    AM_LAUNCH_CHECK();
    const int64_t s = k * C;
    const int64_t go = per_chunk ? k : s;  // this chunk's gates
    const atlasmem_status stt =
        run_update(h, d, (const char*)K + s * d.dk * esz, (const char*)Q + s * d.dk * esz,
                   (const char*)V + s * dv * esz, theta + go, eta + go, alpha + go, win ? gamma + s : nullptr,
                   Span{C, T, per_chunk ? nch : T}, Y ? (void*)((char*)Y + s * dv * (d.out_bf16 ? 2 : 4)) : nullptr,
                   st);
    if (stt != ATLASMEM_OK) return stt;
  }
  // ---- adjoints of the final state
  float* WA = ws + L.wa0;
  float* SA = ws + L.sa0;
  float* WAn = ws + L.wa1;
  float* SAn = ws + L.sa1;
  const size_t pbytes = sizeof(float) * M * P;
  bool ok = (dWT ? hipMemcpyAsync(WA, dWT, pbytes, hipMemcpyDeviceToDevice, st) : hipMemsetAsync(WA, 0, pbytes, st)) ==
                hipSuccess &&
            (dST ? hipMemcpyAsync(SA, dST, pbytes, hipMemcpyDeviceToDevice, st) : hipMemsetAsync(SA, 0, pbytes, st)) ==
                hipSuccess;
  if (!ok) {
    (void)hipGetLastError();
    return ATLASMEM_E_DEVICE;
  }
  float *Zk = ws + L.zk, *E = ws + L.e, *Pz = ws + L.pz, *D1 = ws + L.d1, *U1 = ws + L.u1, *U1s = ws + L.u1s;
  float *U2 = ws + L.u2, *U2s = ws + L.u2s, *Zqa = ws + L.zqa, *Wb = ws + L.wb;
  float *cW = ws + L.cw, *cS = ws + L.cs, *cWa = ws + L.cwa, *cSa = ws + L.csa, *sc = ws + L.sc, *sca = ws + L.sca;
  const int R = (int)L.R;  // key rows per chunk (the queries are the chunk's C rows)
  const int64_t zz = (int64_t)(R + C) * dh, hz = (int64_t)R * dh, vz = (int64_t)R * dv;
  const int64_t inz = T * d.dk;  // input elements per memory (K, Q)
  // per key row: the coefficients of its gradient and their adjoints (window: oW / oS over R rows)
  const float* rW = win ? ws + L.ow : cW;
  const float* rS = win ? ws + L.os : cS;
  const int rld = win ? R : C;
  if (per_chunk) {
    // per-chunk gates: the per-token products take every row's gradient adjoint G' with cW = -1,
    // cS = 0 in place of the state adjoints; nothing in the chunk loop writes them, so once here
    hipLaunchKernelGGL(bk::fill_kernel, dim3(blocks_of((int64_t)M * C)), dim3(256), 0, st, cW, (int64_t)M * C, -1.0f);
    hipLaunchKernelGGL(bk::fill_kernel, dim3(blocks_of((int64_t)M * C)), dim3(256), 0, st, cS, (int64_t)M * C, 0.0f);
    AM_LAUNCH_CHECK();
  }
  for (int64_t k = nch - 1; k >= 0; --k) {
    const int64_t s = k * C;
    const float* ck = ws + L.ck + k * M * 2 * P;  // [M][W | S]
    const float* cW1 = ck;
    const float* cW2 = ck + P1;
    const char* Kc = (const char*)K + s * d.dk * esz;
    const char* Qc = (const char*)Q + s * d.dk * esz;
    // key rows: the chunk's keys (or the R staged feature rows); values, queries likewise
    const void* Kr = staged ? (const void*)(ws + L.ks) : (const void*)Kc;
    const int kbf = staged ? 0 : bf;
    const int64_t kz = staged ? (int64_t)R * din : inz;
    const void* Vr = win ? (const void*)(ws + L.vs) : (const void*)((const char*)V + s * dv * esz);
    const int vbf = win ? 0 : bf;
    const int64_t vrz = win ? (int64_t)R * dv : T * dv;
    const void* Qr = feat ? (const void*)(ws + L.qs) : (const void*)Qc;
    const int qbf = feat ? 0 : bf;
    const int64_t qz = feat ? (int64_t)C * din : inz;
    atlasmem_status stt = ATLASMEM_OK;
    if (!per_chunk) {
      stt = launch_gate_scan(theta, eta, alpha, M, T, s, 1, C, cW, cS, C, sc, 3, st);
      if (stt != ATLASMEM_OK) return stt;
    }
    if (staged) {
      hipLaunchKernelGGL(bk::stage_feat_kernel, dim3(R, M), dim3(256), sizeof(float) * d.dk, st, K, bf, T,
                         s - (c - 1), R, d.dk, din, d.poly, win ? ws + L.hk0 : nullptr, c - 1, ws + L.ks);
      AM_LAUNCH_CHECK();
    }
    if (feat) {
      hipLaunchKernelGGL(bk::stage_feat_kernel, dim3(C, M), dim3(256), sizeof(float) * d.dk, st, Q, bf, T, s, C,
                         d.dk, din, d.poly, (const float*)nullptr, 0, ws + L.qs);
      AM_LAUNCH_CHECK();
    }
    if (win) {
      hipLaunchKernelGGL(bk::stage_vg_kernel, dim3(R, M), dim3(64), 0, st, V, gamma, bf, T, s, c, R, dv,
                         ws + L.hv0, ws + L.hg0, ws + L.vs, ws + L.gs);
      hipLaunchKernelGGL(bk::omega_coef_kernel, dim3(blocks_of((int64_t)M * R)), dim3(256), 0, st, cW, cS,
                         ws + L.gs, C, c, R, M, ws + L.ow, ws + L.os, ws + L.sw, ws + L.ss);
      AM_LAUNCH_CHECK();
    }
    const bool lin = d.kind == ATLASMEM_LINEAR;
    if (lin) {
      // the linear memory M(x) = W x: E = 2 (X W^T - V), g_r = E_r x_r^T
      const float* cW0 = ck;
      const bk::Cat lk = bk::cat1(bk::src(Kr, kbf, kz, din, 1, R, din));
      launch_gemm<false, false>(true, R, dv, din, M, lk, bk::cat1(bk::src(cW0, 0, 2 * P, din, 1, dv, din)),
                                bk::EpiE{E, vz, Vr, vbf, vrz, dv, nullptr, 0, 0}, st, sk, skf);
      launch_gemm<false, false>(true, R, dv, din, M, lk, bk::cat1(bk::src(WA, 0, P, din, 1, dv, din)),
                                bk::EpiSt{U2, vz, dv}, st, sk, skf);
      launch_gemm<false, false>(true, R, dv, din, M, lk, bk::cat1(bk::src(SA, 0, P, din, 1, dv, din)),
                                bk::EpiSt{U2s, vz, dv}, st, sk, skf);
      hipLaunchKernelGGL(bk::lin_row_kernel, dim3(R, M), dim3(64), 0, st, E, U2, U2s, vz, dv, rld, rW, rS, cWa, cSa,
                         win ? dV : dV + s * dv, T * dv, s - (c - 1), win ? 1 : 0);
      AM_LAUNCH_CHECK();
      // X' = -(oW E) WA - (oS E) SA + 2 E' W   (B(k=v, j=f) = M[v][f])
      const bk::EpiStAdd out = feat ? bk::EpiStAdd{ws + L.xg, (int64_t)R * din, din, nullptr, 0, 0, 0.0f, 0, 0}
                               : win ? bk::EpiStAdd{dK, T * din, din, nullptr, 0, 0, 0.0f, s - (c - 1), 1}
                                     : bk::EpiStAdd{dK + s * din, T * din, din, nullptr, 0, 0, 0.0f, 0, 0};
      launch_gemm<false, false>(
          true, R, din, 3 * dv, M,
          bk::cat3(bk::src(E, 0, vz, dv, 1, R, dv, 2, rW, rld, -1.0f), bk::src(E, 0, vz, dv, 1, R, dv, 2, rS, rld, -1.0f),
                   bk::src(U2, 0, vz, dv, 1, R, dv, 0, nullptr, 0, 2.0f), dv, 2 * dv),
          bk::cat3(bk::src(WA, 0, P, 1, din, din, dv), bk::src(SA, 0, P, 1, din, din, dv),
                   bk::src(cW0, 0, 2 * P, 1, din, din, dv), dv, 2 * dv),
          out, st, sk, skf);
      // Q' = dY W
      launch_gemm<false, false>(true, C, din, dv, M, bk::cat1(bk::src(dY + s * dv, 0, T * dv, dv, 1, C, dv)),
                                bk::cat1(bk::src(cW0, 0, 2 * P, 1, din, din, dv)),
                                feat ? bk::EpiStAdd{ws + L.qg, (int64_t)C * din, din, nullptr, 0, 0, 0.0f, 0, 0}
                                     : bk::EpiStAdd{dQ + s * din, T * din, din, nullptr, 0, 0, 0.0f, 0, 0},
                                st, sk, skf);
      // W' = (2E')^T X + dY^T Q   (A(i=v, k=row), B(k=row, j=f))
      launch_gemm<false, false>(
          true, dv, din, R + C, M,
          bk::cat2(bk::src(U2, 0, vz, 1, dv, dv, R, 0, nullptr, 0, 2.0f), bk::src(dY + s * dv, 0, T * dv, 1, dv, dv, C),
                   R),
          bk::cat2(bk::src(Kr, kbf, kz, 1, din, din, R), bk::src(Qr, qbf, qz, 1, din, din, C), R),
          bk::EpiSt{Wb, P, din}, st, sk, skf);
      AM_LAUNCH_CHECK();
      if (feat) {
        hipLaunchKernelGGL(bk::feat_jac_kernel, dim3(R, M), dim3(64), 0, st, ws + L.xg, ws + L.ks, R, d.dk, din, T,
                           s - (c - 1), win ? 1 : 0, dK);
        hipLaunchKernelGGL(bk::feat_jac_kernel, dim3(C, M), dim3(64), 0, st, ws + L.qg, ws + L.qs, C, d.dk, din, T,
                           s, 0, dQ);
        AM_LAUNCH_CHECK();
      }
    } else if (d.gated) {
      // the gated memory M(x) = W2 (silu(Z1) * Z3): Z rows are [Z1 | Z3] (dz = 2 dh), first-layer
      // weights [W1; W3] one block; b = E W2, D = [b Z3 silu'(Z1) | b silu(Z1)]
      const int dzz = 2 * dh;
      const int64_t gzz = (int64_t)(R + C) * dzz, gz = (int64_t)R * dzz;
      float* Za = ws + L.za;
      {
        bk::Cat lk = bk::cat1(bk::src(Kr, kbf, kz, din, 1, R, din));
        bk::Cat lq = bk::cat1(bk::src(Qr, qbf, qz, din, 1, C, din));
        bk::Cat lb = bk::cat1(bk::src(cW1, 0, 2 * P, din, 1, dzz, din));
        launch_gemm<false, false>(true, R, dzz, din, M, lk, lb, bk::EpiSt{Zk, gzz, dzz}, st, sk, skf);
        launch_gemm<false, false>(true, C, dzz, din, M, lq, lb, bk::EpiSt{Zk + (int64_t)R * dzz, gzz, dzz}, st, sk, skf);
      }
      const bk::Src hk = bk::gated(Zk, gzz, dzz, 1, R, dh, dh);  // H of the key rows, A(i = row, k = h)
      launch_gemm<false, false>(true, R, dv, dh, M, bk::cat1(hk), bk::cat1(bk::src(cW2, 0, 2 * P, dh, 1, dv, dh)),
                                bk::EpiE{E, vz, Vr, vbf, vrz, dv, nullptr, 0, 0}, st, sk, skf);
      launch_gemm<false, false>(true, R, dh, dv, M, bk::cat1(bk::src(E, 0, vz, dv, 1, R, dv)),
                                bk::cat1(bk::src(cW2, 0, 2 * P, 1, dh, dh, dv)),
                                bk::EpiPDg{Pz, D1, Zk, hz, gz, gzz, dh}, st, sk, skf);
      // per-chunk gates: G = (Dz^T X, E^T H) over the chunk's rows, its Newton-Schulz image N, and
      // every row's gradient adjoint G' taken in place of the state adjoints (cW = -1, cS = 0)
      const float* WAg = WA;
      const float* SAg = SA;
      if (per_chunk) {
        float *Gb = ws + L.gb, *Nb = ws + L.nb, *NAb = ws + L.nab, *GAb = ws + L.gab, *SAt = ws + L.sat;
        launch_gemm<false, false>(true, dzz, din, C, M, bk::cat1(bk::src(D1, 0, gz, 1, dzz, dzz, C)),
                                  bk::cat1(bk::src(Kr, kbf, kz, 1, din, din, C)), bk::EpiSt{Gb, P, din}, st, sk, skf);
        launch_gemm<false, false>(true, dv, dh, C, M, bk::cat1(bk::src(E, 0, vz, 1, dv, dv, C)),
                                  bk::cat1(bk::gated(Zk, gzz, 1, dzz, dh, C, dh)), bk::EpiSt{Gb + P1, P, dh}, st, sk, skf);
        AM_LAUNCH_CHECK();
        const float* N = Gb;
        if (d.ns_steps > 0) {
          for (int m = 0; m < L.nns; ++m)
            if ((stt = ns_forward(d, ws, L.ns[m], Gb, Nb, st)) != ATLASMEM_OK) return stt;
          N = Nb;
        }
        hipLaunchKernelGGL(bk::chunk_gate_adj_kernel, dim3(M), dim3(256), 0, st, WA, SA, N, ck, P, SAt, nch, k, dth,
                           det, dal);
        hipLaunchKernelGGL(bk::to_work_kernel, dim3(blocks_of((int64_t)M * P)), dim3(256), 0, st, SAt, P, 1, (int)P,
                           0, theta, nch, k, -1.0f, NAb, P, M);  // N' = -theta_k SAt
        AM_LAUNCH_CHECK();
        if (d.ns_steps > 0) {
          for (int m = 0; m < L.nns; ++m)
            if ((stt = ns_backward(d, ws, L.ns[m], Gb, NAb, GAb, st)) != ATLASMEM_OK) return stt;
          WAg = SAg = GAb;
        } else {
          WAg = SAg = NAb;
        }
      }
      {  // U1 = X WAz^T, U1s = X SAz^T (dz wide), U2 = H WA2^T, U2s = H SA2^T
        bk::Cat lx = bk::cat1(bk::src(Kr, kbf, kz, din, 1, R, din));
        launch_gemm<false, false>(true, R, dzz, din, M, lx, bk::cat1(bk::src(WAg, 0, P, din, 1, dzz, din)),
                                  bk::EpiSt{U1, gz, dzz}, st, sk, skf);
        launch_gemm<false, false>(true, R, dzz, din, M, lx, bk::cat1(bk::src(SAg, 0, P, din, 1, dzz, din)),
                                  bk::EpiSt{U1s, gz, dzz}, st, sk, skf);
        launch_gemm<false, false>(true, R, dv, dh, M, bk::cat1(hk), bk::cat1(bk::src(WAg + P1, 0, P, dh, 1, dv, dh)),
                                  bk::EpiSt{U2, vz, dv}, st, sk, skf);
        launch_gemm<false, false>(true, R, dv, dh, M, bk::cat1(hk), bk::cat1(bk::src(SAg + P1, 0, P, dh, 1, dv, dh)),
                                  bk::EpiSt{U2s, vz, dv}, st, sk, skf);
      }
      hipLaunchKernelGGL(bk::row_kernel_gated, dim3(R, M), dim3(64), 0, st, Zk, gzz, Pz, hz, D1, U1, U1s, gz, Za, E,
                         U2, U2s, vz, dh, dv, rld, rW, rS, cWa, cSa);
      AM_LAUNCH_CHECK();
      {  // E' = E'_g + b' W2^T (b' in U1s[:, :dh]), dV = -2 E'
        const bk::EpiEa ep = win ? bk::EpiEa{U2, vz, dV, T * dv, dv, s - (c - 1), 1}
                                 : bk::EpiEa{U2, vz, dV + s * dv, T * dv, dv, 0, 0};
        launch_gemm<false, false>(true, R, dv, dh, M, bk::cat1(bk::src(U1s, 0, gz, dzz, 1, R, dh)),
                                  bk::cat1(bk::src(cW2, 0, 2 * P, dh, 1, dv, dh)), ep, st, sk, skf);
      }
      {  // W2' = E^T b' + (2E')^T H + dY^T Hq
        bk::Cat la = bk::cat3(bk::src(E, 0, vz, 1, dv, dv, R), bk::src(U2, 0, vz, 1, dv, dv, R, 0, nullptr, 0, 2.0f),
                              bk::src(dY + s * dv, 0, T * dv, 1, dv, dv, C), R, 2 * R);
        bk::Cat lb = bk::cat3(bk::src(U1s, 0, gz, 1, dzz, dh, R), bk::gated(Zk, gzz, 1, dzz, dh, R, dh),
                              bk::gated(Zk + (int64_t)R * dzz, gzz, 1, dzz, dh, C, dh), R, 2 * R);
        launch_gemm<false, false>(true, dv, dh, 2 * R + C, M, la, lb, bk::EpiSt{Wb + P1, P, dh}, st, sk, skf);
      }
      // H' = -(cW E) WA2 - (cS E) SA2 + (2E') W2, scattered into Za through the gate
      launch_gemm<false, false>(
          true, R, dh, 3 * dv, M,
          bk::cat3(bk::src(E, 0, vz, dv, 1, R, dv, 2, rW, rld, -1.0f), bk::src(E, 0, vz, dv, 1, R, dv, 2, rS, rld, -1.0f),
                   bk::src(U2, 0, vz, dv, 1, R, dv, 0, nullptr, 0, 2.0f), dv, 2 * dv),
          bk::cat3(bk::src(WAg + P1, 0, P, 1, dh, dh, dv), bk::src(SAg + P1, 0, P, 1, dh, dh, dv),
                   bk::src(cW2, 0, 2 * P, 1, dh, dh, dv), dv, 2 * dv),
          bk::EpiZag{Za, Zk, gz, gzz, dh}, st, sk, skf);
      {  // X' = -(cW D) WAz - (cS D) SAz + Za Wz
        const bk::EpiStAdd out = feat ? bk::EpiStAdd{ws + L.xg, (int64_t)R * din, din, nullptr, 0, 0, 0.0f, 0, 0}
                                 : win ? bk::EpiStAdd{dK, T * din, din, nullptr, 0, 0, 0.0f, s - (c - 1), 1}
                                       : bk::EpiStAdd{dK + s * din, T * din, din, nullptr, 0, 0, 0.0f, 0, 0};
        launch_gemm<false, false>(
            true, R, din, 3 * dzz, M,
            bk::cat3(bk::src(D1, 0, gz, dzz, 1, R, dzz, 2, rW, rld, -1.0f),
                     bk::src(D1, 0, gz, dzz, 1, R, dzz, 2, rS, rld, -1.0f), bk::src(Za, 0, gz, dzz, 1, R, dzz), dzz,
                     2 * dzz),
            bk::cat3(bk::src(WAg, 0, P, 1, din, din, dzz), bk::src(SAg, 0, P, 1, din, din, dzz),
                     bk::src(cW1, 0, 2 * P, 1, din, din, dzz), dzz, 2 * dzz),
            out, st, sk, skf);
      }
      {  // Zq' through the gate, Q' = Zq' Wz
        launch_gemm<false, false>(true, C, dh, dv, M, bk::cat1(bk::src(dY + s * dv, 0, T * dv, dv, 1, C, dv)),
                                  bk::cat1(bk::src(cW2, 0, 2 * P, 1, dh, dh, dv)),
                                  bk::EpiScaleSpG{Zqa, Zk, gz, gzz, R, dh}, st, sk, skf);
        launch_gemm<false, false>(true, C, din, dzz, M, bk::cat1(bk::src(Zqa, 0, gz, dzz, 1, C, dzz)),
                                  bk::cat1(bk::src(cW1, 0, 2 * P, 1, din, din, dzz)),
                                  feat ? bk::EpiStAdd{ws + L.qg, (int64_t)C * din, din, nullptr, 0, 0, 0.0f, 0, 0}
                                       : bk::EpiStAdd{dQ + s * din, T * din, din, nullptr, 0, 0, 0.0f, 0, 0},
                                  st, sk, skf);
      }
      {  // Wz' = Za^T X + Zq'^T Q -> Wb
        bk::Cat la = bk::cat2(bk::src(Za, 0, gz, 1, dzz, dzz, R), bk::src(Zqa, 0, gz, 1, dzz, dzz, C), R);
        bk::Cat lb = bk::cat2(bk::src(Kr, kbf, kz, 1, din, din, R), bk::src(Qr, qbf, qz, 1, din, din, C), R);
        launch_gemm<false, false>(true, dzz, din, R + C, M, la, lb, bk::EpiSt{Wb, P, din}, st, sk, skf);
      }
      AM_LAUNCH_CHECK();
      if (feat) {
        hipLaunchKernelGGL(bk::feat_jac_kernel, dim3(R, M), dim3(64), 0, st, ws + L.xg, ws + L.ks, R, d.dk, din, T,
                           s - (c - 1), win ? 1 : 0, dK);
        hipLaunchKernelGGL(bk::feat_jac_kernel, dim3(C, M), dim3(64), 0, st, ws + L.qg, ws + L.qs, C, d.dk, din, T,
                           s, 0, dQ);
        AM_LAUNCH_CHECK();
      }
    } else {
    // Z of key and query rows
    {  // rows [0, R) keys, [R, R + C) queries (two launches into the two parts)
      bk::Cat lk = bk::cat1(bk::src(Kr, kbf, kz, din, 1, R, din));
      bk::Cat lq = bk::cat1(bk::src(Qr, qbf, qz, din, 1, C, din));
      bk::Cat lb = bk::cat1(bk::src(cW1, 0, 2 * P, din, 1, dh, din));
      launch_gemm<false, false>(true, R, dh, din, M, lk, lb, bk::EpiSt{Zk, zz, dh}, st, sk, skf);
      launch_gemm<false, false>(true, C, dh, din, M, lq, lb, bk::EpiSt{Zk + (int64_t)R * dh, zz, dh}, st, sk, skf);
    }
    // E = 2 (H W2^T - V)
    {
      bk::Cat la = bk::cat1(bk::src(Zk, 0, zz, dh, 1, R, dh, 1));
      bk::Cat lb = bk::cat1(bk::src(cW2, 0, 2 * P, dh, 1, dv, dh));
      launch_gemm<false, false>(true, R, dv, dh, M, la, lb,
                                bk::EpiE{E, vz, Vr, vbf, vrz, dv, d.residual ? Kr : nullptr, kbf, kz}, st, sk, skf);
    }
    // P = E W2, D1 = P silu'(Z)
    {
      bk::Cat la = bk::cat1(bk::src(E, 0, vz, dv, 1, R, dv));
      bk::Cat lb = bk::cat1(bk::src(cW2, 0, 2 * P, 1, dh, dh, dv));  // B(k=v, j=h) = W2[v][h]
      launch_gemm<false, false>(true, R, dh, dv, M, la, lb, bk::EpiPD1{Pz, D1, Zk, hz, zz, dh}, st, sk, skf);
    }
    // Per-chunk gates: G = (D1^T X, E^T H), N = NS(G) or G, S_end = eta S - theta N,
    // W_end = (1 - alpha) W + S_end.  The adjoint of every row's gradient is G' (from N' = -theta
    // (SA + WA) through the orthogonalisation), which the per-token products below take with
    // cW = -1, cS = 0 in place of the state adjoints.
    const float* WAg = WA;
    const float* SAg = SA;
    if (per_chunk) {
      float *Gb = ws + L.gb, *Nb = ws + L.nb, *NAb = ws + L.nab, *GAb = ws + L.gab, *SAt = ws + L.sat;
      launch_gemm<false, false>(true, dh, din, C, M, bk::cat1(bk::src(D1, 0, hz, 1, dh, dh, C)),
                                bk::cat1(bk::src(Kc, bf, inz, 1, din, din, C)), bk::EpiSt{Gb, P, din}, st, sk, skf);
      launch_gemm<false, false>(true, dv, dh, C, M, bk::cat1(bk::src(E, 0, vz, 1, dv, dv, C)),
                                bk::cat1(bk::src(Zk, 0, zz, 1, dh, dh, C, 1)), bk::EpiSt{Gb + P1, P, dh}, st, sk, skf);
      AM_LAUNCH_CHECK();
      const float* N = Gb;
      if (d.ns_steps > 0) {
        for (int m = 0; m < L.nns; ++m)
          if ((stt = ns_forward(d, ws, L.ns[m], Gb, Nb, st)) != ATLASMEM_OK) return stt;
        N = Nb;
      }
      hipLaunchKernelGGL(bk::chunk_gate_adj_kernel, dim3(M), dim3(256), 0, st, WA, SA, N, ck, P, SAt, nch, k, dth,
                         det, dal);
      // N' = -theta_k SAt (G's orientation, whole parameter vector)
      hipLaunchKernelGGL(bk::to_work_kernel, dim3(blocks_of((int64_t)M * P)), dim3(256), 0, st, SAt, P, 1, (int)P, 0,
                         theta, nch, k, -1.0f, NAb, P, M);
      AM_LAUNCH_CHECK();
      if (d.ns_steps > 0) {
        for (int m = 0; m < L.nns; ++m)
          if ((stt = ns_backward(d, ws, L.ns[m], Gb, NAb, GAb, st)) != ATLASMEM_OK) return stt;
        WAg = SAg = GAb;
      } else {
        WAg = SAg = NAb;
      }
    }
    // U1 = X WA1^T, U1s = X SA1^T, U2 = H WA2^T, U2s = H SA2^T
    {
      bk::Cat lx = bk::cat1(bk::src(Kr, kbf, kz, din, 1, R, din));
      bk::Cat lh = bk::cat1(bk::src(Zk, 0, zz, dh, 1, R, dh, 1));
      launch_gemm<false, false>(true, R, dh, din, M, lx, bk::cat1(bk::src(WAg, 0, P, din, 1, dh, din)),
                                bk::EpiSt{U1, hz, dh}, st, sk, skf);
      if (!per_chunk)
        launch_gemm<false, false>(true, R, dh, din, M, lx, bk::cat1(bk::src(SAg, 0, P, din, 1, dh, din)),
                                  bk::EpiSt{U1s, hz, dh}, st, sk, skf);
      launch_gemm<false, false>(true, R, dv, dh, M, lh, bk::cat1(bk::src(WAg + P1, 0, P, dh, 1, dv, dh)),
                                bk::EpiSt{U2, vz, dv}, st, sk, skf);
      if (!per_chunk)
        launch_gemm<false, false>(true, R, dv, dh, M, lh, bk::cat1(bk::src(SAg + P1, 0, P, dh, 1, dv, dh)),
                                  bk::EpiSt{U2s, vz, dv}, st, sk, skf);
    }
    hipLaunchKernelGGL(bk::row_kernel, dim3(R, M), dim3(64), 0, st, Zk, zz, Pz, D1, U1, U1s, E, U2, U2s, hz, vz, dh,
                       dv, rld, rW, rS, cWa, cSa, per_chunk ? 0 : 1);
    AM_LAUNCH_CHECK();
    // now: U1s = P', Pz = Z'_1, U2 = E'_g.  E' = E'_g + P' W2^T (in U2), dV = -2 E'
    {
      bk::Cat la = bk::cat1(bk::src(U1s, 0, hz, dh, 1, R, dh));
      bk::Cat lb = bk::cat1(bk::src(cW2, 0, 2 * P, dh, 1, dv, dh));  // B(k=h, j=v) = W2[v][h]
      const bk::EpiEa ep = win ? bk::EpiEa{U2, vz, dV, T * dv, dv, s - (c - 1), 1}
                               : bk::EpiEa{U2, vz, dV + s * dv, T * dv, dv, 0, 0};
      launch_gemm<false, false>(true, R, dv, dh, M, la, lb, ep, st, sk, skf);
    }
    // W2' = E^T P' + (2E')^T H + dY^T Hq  -> Wb + P1   (A(i=v, k=row), B(k=row, j=h))
    {
      bk::Cat la = bk::cat3(bk::src(E, 0, vz, 1, dv, dv, R), bk::src(U2, 0, vz, 1, dv, dv, R, 0, nullptr, 0, 2.0f),
                            bk::src(dY + s * dv, 0, T * dv, 1, dv, dv, C), R, 2 * R);
      bk::Cat lb = bk::cat3(bk::src(U1s, 0, hz, 1, dh, dh, R), bk::src(Zk, 0, zz, 1, dh, dh, R, 1),
                            bk::src(Zk + (int64_t)R * dh, 0, zz, 1, dh, dh, C, 1), R, 2 * R);
      launch_gemm<false, false>(true, dv, dh, 2 * R + C, M, la, lb, bk::EpiSt{Wb + P1, P, dh}, st, sk, skf);
    }
    // H' = -(cW E) WA2 - (cS E) SA2 + (2E') W2;  Z' = Z'_1 + H' silu'(Z)  (in Pz)
    {
      const bk::Src ea = bk::src(E, 0, vz, dv, 1, R, dv, 2, rW, rld, -1.0f);
      const bk::Src e2 = bk::src(U2, 0, vz, dv, 1, R, dv, 0, nullptr, 0, 2.0f);
      const bk::Src wa = bk::src(WAg + P1, 0, P, 1, dh, dh, dv);  // B(k=v, j=h) = M[v][h]
      const bk::Src w2 = bk::src(cW2, 0, 2 * P, 1, dh, dh, dv);
      if (per_chunk) {
        launch_gemm<false, false>(true, R, dh, 2 * dv, M, bk::cat2(ea, e2, dv), bk::cat2(wa, w2, dv),
                                  bk::EpiZa{Pz, Zk, hz, zz, dh}, st, sk, skf);
      } else {
        launch_gemm<false, false>(true, R, dh, 3 * dv, M,
                                  bk::cat3(ea, bk::src(E, 0, vz, dv, 1, R, dv, 2, rS, rld, -1.0f), e2, dv, 2 * dv),
                                  bk::cat3(wa, bk::src(SAg + P1, 0, P, 1, dh, dh, dv), w2, dv, 2 * dv),
                                  bk::EpiZa{Pz, Zk, hz, zz, dh}, st, sk, skf);
      }
    }
    // X' = -(cW D1) WA1 - (cS D1) SA1 + Z' W1 -> dK rows
    {
      const bk::Src da = bk::src(D1, 0, hz, dh, 1, R, dh, 2, rW, rld, -1.0f);
      const bk::Src za = bk::src(Pz, 0, hz, dh, 1, R, dh);
      const bk::Src wa = bk::src(WAg, 0, P, 1, din, din, dh);  // B(k=h, j=f) = M[h][f]
      const bk::Src w1 = bk::src(cW1, 0, 2 * P, 1, din, din, dh);
      // the residual memory's keys also enter E directly: + 2 E' (E' in U2, din = dv)
      // with features the rows' feature-space gradient goes to xg and through phi's Jacobian below
      const bk::EpiStAdd out = feat ? bk::EpiStAdd{ws + L.xg, (int64_t)R * din, din, d.residual ? U2 : nullptr, vz,
                                                   dv, 2.0f, 0, 0}
                               : win ? bk::EpiStAdd{dK, T * din, din, d.residual ? U2 : nullptr, vz, dv, 2.0f,
                                                    s - (c - 1), 1}
                                     : bk::EpiStAdd{dK + s * din, T * din, din, d.residual ? U2 : nullptr, vz, dv,
                                                    2.0f, 0, 0};
      if (per_chunk) {
        launch_gemm<false, false>(true, R, din, 2 * dh, M, bk::cat2(da, za, dh), bk::cat2(wa, w1, dh), out, st, sk, skf);
      } else {
        launch_gemm<false, false>(true, R, din, 3 * dh, M,
                                  bk::cat3(da, bk::src(D1, 0, hz, dh, 1, R, dh, 2, rS, rld, -1.0f), za, dh, 2 * dh),
                                  bk::cat3(wa, bk::src(SAg, 0, P, 1, din, din, dh), w1, dh, 2 * dh), out, st, sk, skf);
      }
    }
    // Zq' = (dY W2) silu'(Zq); Q' = Zq' W1 -> dQ rows
    {
      bk::Cat la = bk::cat1(bk::src(dY + s * dv, 0, T * dv, dv, 1, C, dv));
      bk::Cat lb = bk::cat1(bk::src(cW2, 0, 2 * P, 1, dh, dh, dv));
      launch_gemm<false, false>(true, C, dh, dv, M, la, lb, bk::EpiScaleSp{Zqa, Zk, hz, zz, R, dh}, st, sk, skf);
      bk::Cat la2 = bk::cat1(bk::src(Zqa, 0, hz, dh, 1, C, dh));
      bk::Cat lb2 = bk::cat1(bk::src(cW1, 0, 2 * P, 1, din, din, dh));
      // the residual memory's retrieval adds the query: + dY
      launch_gemm<false, false>(true, C, din, dh, M, la2, lb2,
                                feat ? bk::EpiStAdd{ws + L.qg, (int64_t)C * din, din,
                                                    d.residual ? dY + s * dv : nullptr, T * dv, dv, 1.0f, 0, 0}
                                     : bk::EpiStAdd{dQ + s * din, T * din, din, d.residual ? dY + s * dv : nullptr,
                                                    T * dv, dv, 1.0f, 0, 0},
                                st, sk, skf);
    }
    if (feat) {  // the raw rows' gradients through the feature map
      hipLaunchKernelGGL(bk::feat_jac_kernel, dim3(R, M), dim3(64), 0, st, ws + L.xg, ws + L.ks, R, d.dk, din, T,
                         s - (c - 1), win ? 1 : 0, dK);
      hipLaunchKernelGGL(bk::feat_jac_kernel, dim3(C, M), dim3(64), 0, st, ws + L.qg, ws + L.qs, C, d.dk, din, T, s,
                         0, dQ);
      AM_LAUNCH_CHECK();
    }
    // W1' = Z'^T X + Zq'^T Q -> Wb   (A(i=h, k=row), B(k=row, j=f))
    {
      bk::Cat la = bk::cat2(bk::src(Pz, 0, hz, 1, dh, dh, R), bk::src(Zqa, 0, hz, 1, dh, dh, C), R);
      bk::Cat lb = bk::cat2(bk::src(Kr, kbf, kz, 1, din, din, R), bk::src(Qr, qbf, qz, 1, din, din, C), R);
      launch_gemm<false, false>(true, dh, din, R + C, M, la, lb, bk::EpiSt{Wb, P, din}, st, sk, skf);
    }
    }  // MLP memory
    AM_LAUNCH_CHECK();
    const int64_t n = (int64_t)M * P;
    if (per_chunk) {
      hipLaunchKernelGGL(bk::chunk_state_adj_kernel, dim3(blocks_of(n)), dim3(256), 0, st, WA, ws + L.sat, Wb, eta,
                         alpha, nch, k, P, M, WAn, SAn);
      AM_LAUNCH_CHECK();
    } else {
      // one block per memory (eight memories in the per-token workloads): 1024 threads keep more of
      // the memory's loads in flight (5.0 us per chunk, 5.5 with 256)
      hipLaunchKernelGGL(bk::scalar_adj_kernel, dim3(M), dim3(1024), 0, st, WA, SA, ck, P, sca);
      AM_LAUNCH_CHECK();
      const float* cWt = cWa;  // the per-token coefficient adjoints entering the gate scan's reverse
      const float* cSt = cSa;
      if (win) {
        hipLaunchKernelGGL(bk::omega_adj_kernel, dim3(blocks_of((int64_t)M * R)), dim3(256), 0, st, cWa, cSa,
                           ws + L.gs, ws + L.sw, ws + L.ss, C, c, R, M, T, s, ws + L.cwt, ws + L.cst, dgamma);
        AM_LAUNCH_CHECK();
        cWt = ws + L.cwt;
        cSt = ws + L.cst;
      }
      if (C > bk::kGateBwdMaxC) return ATLASMEM_E_UNSUPPORTED;
      hipLaunchKernelGGL(bk::gate_bwd_kernel, dim3(M), dim3(64), (size_t)9 * C * sizeof(float), st, theta, eta,
                         alpha, T, s, C, cWt, cSt, sca, dth, det, dal);
      AM_LAUNCH_CHECK();
      hipLaunchKernelGGL(bk::state_adj_kernel, dim3(blocks_of(n)), dim3(256), 0, st, WA, SA, Wb, sc, P, M, WAn, SAn);
      AM_LAUNCH_CHECK();
    }
    float* t;
    t = WA, WA = WAn, WAn = t;
    t = SA, SA = SAn, SAn = t;
  }
  if (hipMemcpyAsync(dW0, WA, pbytes, hipMemcpyDeviceToDevice, st) != hipSuccess ||
      hipMemcpyAsync(dS0, SA, pbytes, hipMemcpyDeviceToDevice, st) != hipSuccess) {
    (void)hipGetLastError();
    return ATLASMEM_E_DEVICE;
  }
  return ATLASMEM_OK;
}

}  // namespace am
