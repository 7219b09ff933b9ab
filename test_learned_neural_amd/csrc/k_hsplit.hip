// Hidden-split chunk kernel: the 2-layer SiLU memory with per-token gates, an Omega window and
// polynomial key / query features, one launch per chunk.
//
// The chunk-wise form (ATLAS ... | Summary, section 3.3 "Parallelizing Omega Rule"; the gradient
// as delta^T activation products, titans-pytorch-mlx README, "MLX Optimizations - Gradient
// Computation") splits along the hidden units: with workgroup g owning the hidden units
// [16 g, 16 g + 16) of a memory, it owns rows [16 g, 16 g + 16) of W1 and S1 and the same columns
// of W2 and S2, and every product of the chunk except one stays inside the workgroup:
//   Z_g = phi(X) W1_g^T, H_g = silu(Z_g)                (the workgroup's pre-activations)
//   Yhat = sum_g H_g W2_g^T                             (the one sum over workgroups)
//   E = 2 (Yhat - V), D1_g = (E W2_g) * silu'(Z_g)
//   W1_g, S1_g <- coefficient form with sum_r c_r D1_g[r]^T phi(x_r)
//   W2_g, S2_g <- coefficient form with sum_r c_r E[r]^T H_g[r]
// The sum over workgroups is carried by the kernel boundary: a launch finishes chunk k (reads the
// G partial Yhat of every workgroup of its memory, written by the previous launch, forms E, the
// gradients and the update) and then runs the forward of chunk k + 1 at the new weights, writing
// its own partial Yhat.  No workgroup waits for another inside a launch.
//
// Products: v_mfma_f32_16x16x32_bf16 (v_mfma_f32_16x16x16_bf16 for the k = 16 output product),
// every fp32 operand split into bf16 hi + lo, terms hi*hi + hi*lo + lo*hi; features of bf16 inputs
// of degree 1 are exact and contribute no lo word.  The features are evaluated from the raw rows
// staged in LDS, through a table of (i, j, half) per feature (phi_f = x_i x_j, times 1/2 for the
// degree-2 monomials; a constant-one and a zero column give the constant feature and padding).
#include "internal.h"
#include "common.h"

namespace am {
namespace hsk {

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;
constexpr int HS = 16;  // hidden units per workgroup
constexpr int kMaxG = 8;
constexpr int kMaxLds = 160 * 1024;
// per-thread (per-wave) register staging of a launch's global loads; hsplit_supported checks the
// shapes against them
constexpr int kStage = 3;    // 8-element raw-row pieces: (rows) * d_key / 8 <= kStage * kThreads
constexpr int kEItems = 3;   // (key row, 4 outputs) items of E: RkK * d_value / 4 <= kEItems * kThreads
constexpr int kYItems = 1;   // (query row, 4 outputs) items of the outputs owned by a workgroup
constexpr int kZTiles = 2;   // key-row tiles of 16 per wave: RkK <= 16 * kZTiles * kWaves
constexpr int kT1 = 5;       // first-layer tiles of 16 features per wave: din <= 16 * kT1 * kWaves
constexpr int kT2 = 2;       // second-layer tiles of 16 outputs per wave: d_value <= 16 * kT2 * kWaves
constexpr int kW2Items = 8;  // W2 slice elements per thread: 16 d_value <= kW2Items * kThreads

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ f32x4 mfma16k16(u32x2 a, u32x2 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a), __builtin_bit_cast(s16x4, b), c, 0,
                                                  0, 0);
}

struct Args {
  const uint16_t* K;  // bf16 rows [M][ld][dk]
  const uint16_t* Q;
  const uint16_t* V;  // [M][ld][dv]
  int64_t ld;         // token stride per memory of K, Q, V and Y
  const float* hk;    // window history [M][c-1][dk], [M][c-1][dv] (fp32)
  const float* hv;
  const float* Win;   // state at the start of the finished chunk [M][P] (or of the forwarded one)
  const float* Sin;
  float* Wout;
  float* Sout;
  int64_t P, P1;
  const float* cw;    // the finished chunk's key-row coefficients: cw[m * ldc + r], r < Rk
  const float* cs;
  int64_t ldc;
  const float* scal;  // its (P, beta, a_S) at scal[m * lds]
  int64_t lds;
  const float* Yp_rd;  // partial outputs [M][G][Rk + nq][dv] of the finished chunk
  float* Yp_wr;        // ... of the forwarded chunk
  const float* Z_rd;   // key-row pre-activations [M][Rk][dh] of the finished chunk
  float* Z_wr;         // ... of the forwarded chunk
  void* Y;
  int out_bf16;
  int64_t s_fin, s_fwd;  // first token of the finished / forwarded chunk, -1 for none
  int M, G, dk, din, dh, dv, Rk, nq, c, poly;
  int* flag;
};

// LDS layout (byte offsets), the same on the host (launch size) and the device.
struct Layout {
  int dinP, RkT, RkK, nqT;
  int xs, xts, w1s, w2s, w2ts, ers, ets, hrs;
  int tab, w1h, w1l, w2h, w2l, w2th, w2tl;
  int w1c;                                                   // the constant feature's weights (fp32)
  int xr, hh, hl;                                            // forward
  int xrT, eh, el, eth, etl, dwh, dwl, dsh, dsl, hwh, hwl, hsh, hsl, cwL, csL;  // finish
  int total;
};

__host__ __device__ inline int up(int x, int a) { return (x + a - 1) / a * a; }

// Degree-2 features of d_key = QB (16 or 32) in the forward product are laid out in blocks of
// 4 x 8 monomials x_i x_j (i in [4 ib, 4 ib + 4), j in [8 jb, 8 jb + 8)), one block per k-step of
// 32: lane group lg of a wave takes i = 4 ib + lg and all lanes the same eight j, so every
// feature is a product of two registers of the lane's raw row.  Blocks with some i <= j are kept
// (jb >= ib / 2), the slots with i > j carry zero weights.  Step 0 holds the degree-1 features;
// the constant feature's weight is added to the product in fp32.
__host__ __device__ constexpr int quad_blocks(int D) {
  int n = 0;
  for (int ib = 0; ib < D / 4; ++ib) n += D / 8 - ib / 2;
  return n;
}
// first block of i-block ib
__host__ __device__ constexpr int quad_block0(int D, int ib) {
  return ib * (D / 8) - ((ib / 2) * (ib / 2 - 1) + (ib % 2) * (ib / 2));
}
__host__ __device__ constexpr int block_slots(int D) { return 32 * (1 + quad_blocks(D)); }

__host__ __device__ inline Layout make_layout(int dk, int din, int dv, int Rk, int nq, int qb) {
  Layout L;
  L.dinP = up(din, 32);
  L.RkT = up(Rk, 16);
  L.RkK = up(Rk, 32);
  L.nqT = up(nq, 16);
  L.xs = dk + 4;        // raw row: dk values, a one, three zeros (16-byte rows)
  L.xts = L.RkK + 4;    // transposed raw rows: (dk + 2) rows of RkK (+4) floats
  L.w1s = (qb ? block_slots(qb) : L.dinP) + 8;  // W1 slice [16][w1s] bf16 (block layout when qb)
  L.w2s = HS + 4;       // W2 slice [dv][w2s] bf16
  L.w2ts = dv + 8;      // W2 slice transposed [16][w2ts] bf16
  L.ers = dv + 8;       // E [RkK][ers] bf16
  L.ets = L.RkK + 8;    // E^T [dv][ets], scaled D1^T and H^T [16][ets] bf16
  L.hrs = HS + 4;       // H [rows][hrs] bf16
  int o = 0;
  auto take = [&](int bytes) {
    const int r = o;
    o += up(bytes, 16);
    return r;
  };
  L.tab = take(4 * L.dinP);
  L.w1h = take(2 * HS * L.w1s);
  L.w1l = take(2 * HS * L.w1s);
  L.w2h = take(2 * dv * L.w2s);
  L.w2l = take(2 * dv * L.w2s);
  L.w2th = take(2 * HS * L.w2ts);
  L.w2tl = take(2 * HS * L.w2ts);
  L.w1c = take(4 * HS);
  const int u = o;
  // forward
  L.xr = take(4 * (L.RkT + L.nqT) * L.xs);
  L.hh = take(2 * (L.RkT + L.nqT) * L.hrs);
  L.hl = take(2 * (L.RkT + L.nqT) * L.hrs);
  const int endA = o;
  o = u;
  // finish
  L.xrT = take(4 * (dk + 2) * L.xts);
  L.eh = take(2 * L.RkK * L.ers);
  L.el = take(2 * L.RkK * L.ers);
  L.eth = take(2 * dv * L.ets);
  L.etl = take(2 * dv * L.ets);
  L.dwh = take(2 * HS * L.ets);
  L.dwl = take(2 * HS * L.ets);
  L.dsh = take(2 * HS * L.ets);
  L.dsl = take(2 * HS * L.ets);
  L.hwh = take(2 * HS * L.ets);
  L.hwl = take(2 * HS * L.ets);
  L.hsh = take(2 * HS * L.ets);
  L.hsl = take(2 * HS * L.ets);
  L.cwL = take(4 * L.RkK);
  L.csL = take(4 * L.RkK);
  L.total = o > endA ? o : endA;
  return L;
}

// Feature f of the map as (i, j, half): phi_f = x_i x_j (times 1/2 when half), where column dk
// of a raw row holds 1 and column dk + 1 holds 0.  Order: degree 1, the raw elements; degree 2,
// [1, x_0 .. x_{dk-1}, x_i x_j / 2 for i <= j in combinations-with-replacement order].
__device__ __forceinline__ uint32_t feature_entry(int f, int din, int dk, int poly) {
  const uint32_t one = (uint32_t)dk, zero = (uint32_t)dk + 1;
  if (f >= din) return zero | (one << 8);
  if (poly == 1) return (uint32_t)f | (one << 8);
  if (f == 0) return one | (one << 8);
  if (f <= dk) return (uint32_t)(f - 1) | (one << 8);
  int i, j;
  pair_of(f - 1 - dk, dk, i, j);
  return (uint32_t)i | ((uint32_t)j << 8) | (1u << 16);
}
// The block-layout slot of canonical feature f (0x7FFF for the constant, f == 0) and its weight
// scale (1/2 of the degree-2 monomials goes into the weight: x_i x_j (w / 2) = (x_i x_j / 2) w
// exactly).
__device__ __forceinline__ int slot_of(int f, int dk) {
  if (f == 0) return 0x7FFF;
  if (f <= dk) return f - 1;
  int i, j;
  pair_of(f - 1 - dk, dk, i, j);
  const int ib = i >> 2, jb = j >> 3;
  return 32 * (1 + quad_block0(dk, ib) + jb - ib / 2) + (i & 3) * 8 + (j & 7);
}
__device__ __forceinline__ float feat_eval(uint32_t e, float xi, float xj) {
  return (e >> 16) & 1u ? (0.5f * xi) * xj : xi * xj;
}

// Split v into hi / lo and store both at element `idx` of two bf16 arrays.
__device__ __forceinline__ void st_split1(uint16_t* hi, uint16_t* lo, int idx, float v) {
  uint32_t h, l;
  split_bf16(v, h, l);
  hi[idx] = (uint16_t)h;
  lo[idx] = (uint16_t)l;
}
// Four consecutive elements (8-byte aligned).
__device__ __forceinline__ void st_split4(uint16_t* hi, uint16_t* lo, int idx, float a, float b, float c, float d) {
  uint32_t h0, l0, h1, l1;
  split2(a, b, h0, l0);
  split2(c, d, h1, l1);
  *(u32x2*)&hi[idx] = u32x2{h0, h1};
  *(u32x2*)&lo[idx] = u32x2{l0, l1};
}

// Byte offset that lies outside every buffer resource here (each covers less than 2 GB): loads
// there return zeros, so a load that does not apply is issued anyway and adds nothing.  Loads
// stay branch-free, and a wait for one of them never becomes a wait for everything in flight.
constexpr int kOut = (int)0x80000000u;

// Per-memory buffer resources of a launch.
struct Res {
  rsrc_t K, Q, V, hk, hv, W, S, yp, Z, cw, cs;
};

// A piece of a raw row: elements [8q, 8q + 8) of key row r (token s - (c - 1) + r, from the
// window history before the call) or of query row r - Rk (token s + r - Rk), as bf16 bits; the
// sources that do not apply are read out of range.  HIST: the row may be a history row (only a
// thread's first piece can be: the first c - 1 rows); QRY: it may be a query row.  The history
// holds the same bf16 values as fp32, so the conversion back is exact.
template <bool HIST, bool QRY>
__device__ __forceinline__ u32x4 load_piece(const Args& a, const Res& R, int64_t s, int r, int q, bool valid) {
  const int tau = (int)(s - (a.c - 1)) + r;
  const bool key = valid && r < a.Rk;
  u32x4 x = buf_ld16(R.K, key && tau >= 0 ? tau * a.dk * 2 + 16 * q : kOut, 0);
  if (QRY) {
    const u32x4 qb = buf_ld16(R.Q, valid && r >= a.Rk ? ((int)s + r - a.Rk) * a.dk * 2 + 16 * q : kOut, 0);
    x = u32x4{x[0] | qb[0], x[1] | qb[1], x[2] | qb[2], x[3] | qb[3]};
  }
  if (HIST) {
    const int oh = key && tau < 0 ? ((a.c - 1) + tau) * a.dk * 4 + 32 * q : kOut;
    const u32x4 h0 = buf_ld16(R.hk, oh, 0), h1 = buf_ld16(R.hk, oh + 16, 0);
    x = u32x4{x[0] | (h0[0] >> 16) | (h0[1] & 0xFFFF0000u), x[1] | (h0[2] >> 16) | (h0[3] & 0xFFFF0000u),
              x[2] | (h1[0] >> 16) | (h1[1] & 0xFFFF0000u), x[3] | (h1[2] >> 16) | (h1[3] & 0xFFFF0000u)};
  }
  return x;
}
__device__ __forceinline__ float lo_bf16(uint32_t x) { return __uint_as_float(x << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t x) { return __uint_as_float(x & 0xFFFF0000u); }

// EXACT: degree-1 features of bf16 inputs (no lo word on their side); QB: d_key of the block
// layout of degree-2 features in the forward product (0: features gathered through the table).
template <bool EXACT, int QB>
__global__ void __launch_bounds__(kThreads) hsplit_kernel(Args a) {
  extern __shared__ __attribute__((aligned(16))) char sm[];
  const Layout L = make_layout(a.dk, a.din, a.dv, a.Rk, a.nq, QB);
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  // the G workgroups of a memory on one XCD (dispatch places workgroup i on XCD i mod 8), so the
  // partial outputs they exchange stay in one L2
  const int nwg = a.M * a.G;
  int lin = blockIdx.x;
  if ((nwg & 7) == 0) lin = (blockIdx.x & 7) * (nwg >> 3) + (blockIdx.x >> 3);
  const int m = lin / a.G, g = lin - m * a.G;
  const int hs = g * HS;
  const int Rr = a.Rk + a.nq;  // logical rows of a partial output
  const bool fin = a.s_fin >= 0, fwd = a.s_fwd >= 0;
  const int dq = a.dk >> 3;     // 8-element pieces per raw row
  const int nv4 = a.dv >> 2;
  const int nft = L.dinP / 16;  // first-layer tiles of 16 features
  const int nvt = a.dv / 16;    // second-layer tiles of 16 outputs

  uint32_t* tab = (uint32_t*)(sm + L.tab);
  uint16_t* w1h = (uint16_t*)(sm + L.w1h);
  uint16_t* w1l = (uint16_t*)(sm + L.w1l);
  uint16_t* w2h = (uint16_t*)(sm + L.w2h);
  uint16_t* w2l = (uint16_t*)(sm + L.w2l);
  uint16_t* w2th = (uint16_t*)(sm + L.w2th);
  uint16_t* w2tl = (uint16_t*)(sm + L.w2tl);
  float* w1c = (float*)(sm + L.w1c);

  // ------------------------------------------------ every global load of the launch, issued first
  // (one memory latency for the launch instead of one per staging step)
  const float* Wm = a.Win + (int64_t)m * a.P;
  const float* Sm = a.Sin + (int64_t)m * a.P;
  u32x4 kt[kStage];             // key rows of the finished chunk
  float4 ys[kEItems];           // sum over workgroups of its partial outputs (key rows)
  float vv[kEItems][4];         // its values
  float4 yq[kYItems];           // ... and of its query rows owned by this workgroup
  float zp[kZTiles][4];         // its key-row pre-activations
  float w1p[kT1][4], s1p[kT1][4];
  float4 w2p[kT2], s2p[kT2];
  float w2s[kW2Items];          // W2 slice at the chunk start (the product E W2_g)
  u32x4 kx[kStage];             // raw rows of the forwarded chunk
  const float* yp = a.Yp_rd + (int64_t)m * a.G * Rr * a.dv;
  const int mine = (a.Y && a.nq > g) ? (a.nq - g + a.G - 1) / a.G : 0;
  Res R;
  {
    const uint32_t rowb = (uint32_t)(a.ld * a.dk * 2);
    R.K = make_rsrc(a.K + (int64_t)m * a.ld * a.dk, rowb);
    R.Q = make_rsrc((a.Q ? a.Q : a.K) + (int64_t)m * a.ld * a.dk, a.Q ? rowb : 0u);
    R.V = make_rsrc(a.V + (int64_t)m * a.ld * a.dv, (uint32_t)(a.ld * a.dv * 2));
    R.hk = make_rsrc(a.hk + (int64_t)m * (a.c - 1) * a.dk, (uint32_t)((a.c - 1) * a.dk * 4));
    R.hv = make_rsrc(a.hv + (int64_t)m * (a.c - 1) * a.dv, (uint32_t)((a.c - 1) * a.dv * 4));
    R.W = make_rsrc(Wm, (uint32_t)(a.P * 4));
    R.S = make_rsrc(Sm, (uint32_t)(a.P * 4));
    R.yp = make_rsrc(fin ? yp : Wm, fin ? (uint32_t)(a.G * Rr * a.dv * 4) : 0u);
    R.Z = make_rsrc(fin ? a.Z_rd + (int64_t)m * a.Rk * a.dh : Wm, fin ? (uint32_t)(a.Rk * a.dh * 4) : 0u);
    R.cw = make_rsrc(fin ? a.cw + (int64_t)m * a.ldc : Wm, fin ? (uint32_t)(a.Rk * 4) : 0u);
    R.cs = make_rsrc(fin ? a.cs + (int64_t)m * a.ldc : Wm, fin ? (uint32_t)(a.Rk * 4) : 0u);
  }
  // the forwarded chunk's raw rows (key rows, then query rows)
  auto load_rows = [&]() {
    kx[0] = load_piece<true, true>(a, R, a.s_fwd, t / dq, t % dq, fwd && t < (a.Rk + a.nq) * dq);
#pragma unroll
    for (int it = 1; it < kStage; ++it) {
      const int e = t + it * kThreads;
      kx[it] = load_piece<false, true>(a, R, a.s_fwd, e / dq, e % dq, fwd && e < (a.Rk + a.nq) * dq);
    }
  };
  float cwr = 0.0f, csr = 0.0f;  // the coefficient of key row t (t < RkK)
  float cP = 0.0f, cB = 0.0f, cA = 0.0f;  // the finished chunk's (P, beta, a_S)
  if (fin) {
    const int oc = t < a.Rk ? 4 * t : kOut;
    cwr = buf_ld(R.cw, oc, 0);
    csr = buf_ld(R.cs, oc, 0);
    const float* sc = a.scal + (int64_t)m * a.lds;
    cP = sc[0];
    cB = sc[1];
    cA = sc[2];
    kt[0] = load_piece<true, false>(a, R, a.s_fin, t / dq, t % dq, t < a.Rk * dq);
#pragma unroll
    for (int it = 1; it < kStage; ++it) {
      const int e = t + it * kThreads;
      kt[it] = load_piece<false, false>(a, R, a.s_fin, e / dq, e % dq, e < a.Rk * dq);
    }
#pragma unroll
    for (int it = 0; it < kEItems; ++it) {
      const int e = t + it * kThreads;
      const int r = e / nv4, v = (e - r * nv4) * 4;
      const bool ok = r < a.Rk;
      // every workgroup's partial in flight at once (workgroups past G read out of range: zero),
      // summed in workgroup order
      float4 q[kMaxG];
#pragma unroll
      for (int gg = 0; gg < kMaxG; ++gg) q[gg] = buf_ld4(R.yp, ok ? ((gg * Rr + r) * a.dv + v) * 4 : kOut, 0);
      float4 sum = q[0];
#pragma unroll
      for (int gg = 1; gg < kMaxG; ++gg) {
        sum.x += q[gg].x;
        sum.y += q[gg].y;
        sum.z += q[gg].z;
        sum.w += q[gg].w;
      }
      ys[it] = sum;
      const int tau = (int)(a.s_fin - (a.c - 1)) + r;
      const uint2 b = buf_ld8(R.V, ok && tau >= 0 ? (tau * a.dv + v) * 2 : kOut, 0);
      const float4 h4 = buf_ld4(R.hv, ok && tau < 0 ? (((a.c - 1) + tau) * a.dv + v) * 4 : kOut, 0);
      vv[it][0] = lo_bf16(b.x) + h4.x;  // one of the two is zero
      vv[it][1] = hi_bf16(b.x) + h4.y;
      vv[it][2] = lo_bf16(b.y) + h4.z;
      vv[it][3] = hi_bf16(b.y) + h4.w;
    }
#pragma unroll
    for (int it = 0; it < kYItems; ++it) {
      const int e = t + it * kThreads;
      const int j = e / nv4, v = (e - j * nv4) * 4;
      const int row = a.Rk + g + j * a.G;
      float4 q[kMaxG];
#pragma unroll
      for (int gg = 0; gg < kMaxG; ++gg) q[gg] = buf_ld4(R.yp, j < mine ? ((gg * Rr + row) * a.dv + v) * 4 : kOut, 0);
      float4 sum = q[0];
#pragma unroll
      for (int gg = 1; gg < kMaxG; ++gg) {
        sum.x += q[gg].x;
        sum.y += q[gg].y;
        sum.z += q[gg].z;
        sum.w += q[gg].w;
      }
      yq[it] = sum;
    }
#pragma unroll
    for (int j = 0; j < kZTiles; ++j) {
      const int rt = w + j * kWaves;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = rt * 16 + lg * 4 + i;  // rows past Rk read out of range
        zp[j][i] = buf_ld(R.Z, (r * a.dh + hs + lr) * 4, 0);
      }
    }
  }
  if (fin || fwd) {
    // W2 slice at the start of the finished chunk, or of the forwarded one when nothing is finished
#pragma unroll
    for (int it = 0; it < kW2Items; ++it) {
      const int e = t + it * kThreads;
      w2s[it] = buf_ld(R.W, e < a.dv * HS ? ((int)a.P1 + (e >> 4) * a.dh + hs + (e & 15)) * 4 : kOut, 0);
    }
  }

  // ------------------------------------------------ LDS: feature table and the W2 slice
  for (int f = t; f < L.dinP; f += kThreads)
    tab[f] = feature_entry(f, a.din, a.dk, a.poly) | (QB && f < a.din ? (uint32_t)slot_of(f, a.dk) << 17 : 0u);
  if (QB) {  // the block layout's zero slots: the whole slice is cleared before any weight is written
    u32x4* wz = (u32x4*)(sm + L.w1h);
    const int n16 = 2 * (2 * HS * L.w1s) / 16;  // hi and lo arrays, adjacent
    for (int e = t; e < n16; e += kThreads) wz[e] = u32x4{0u, 0u, 0u, 0u};
  }
#pragma unroll
  for (int it = 0; it < kW2Items; ++it) {
    const int e = t + it * kThreads;
    if ((fin || fwd) && e < a.dv * HS) {
      const int v = e >> 4, h = e & 15;
      uint32_t hi, lo;
      split_bf16(w2s[it], hi, lo);
      w2h[v * L.w2s + h] = (uint16_t)hi;
      w2l[v * L.w2s + h] = (uint16_t)lo;
      w2th[h * L.w2ts + v] = (uint16_t)hi;
      w2tl[h * L.w2ts + v] = (uint16_t)lo;
    }
  }

  bool bad = false;

  if (fin) {
    // ---------------------------------------------------------------- finish chunk at s_fin
    float* xT = (float*)(sm + L.xrT);
    uint16_t* eh = (uint16_t*)(sm + L.eh);
    uint16_t* el = (uint16_t*)(sm + L.el);
    uint16_t* eth = (uint16_t*)(sm + L.eth);
    uint16_t* etl = (uint16_t*)(sm + L.etl);
    float* cwL = (float*)(sm + L.cwL);
    float* csL = (float*)(sm + L.csL);
    if (t < L.RkK) {
      cwL[t] = cwr;
      csL[t] = csr;
    }
    // key rows transposed: xT[i][r]; row dk holds ones, row dk + 1 zeros, rows past Rk zeros
#pragma unroll
    for (int it = 0; it < kStage; ++it) {
      const int e = t + it * kThreads;
      if (e < a.Rk * dq) {
        const int r = e / dq, q = e % dq;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          xT[(8 * q + 2 * u) * L.xts + r] = lo_bf16(kt[it][u]);
          xT[(8 * q + 2 * u + 1) * L.xts + r] = hi_bf16(kt[it][u]);
        }
      }
    }
    for (int e = t; e < 2 * L.RkK; e += kThreads) {
      const bool one = e < L.RkK;
      xT[(a.dk + (one ? 0 : 1)) * L.xts + (one ? e : e - L.RkK)] = one ? 1.0f : 0.0f;
    }
    for (int e = t; e < a.dk * 32; e += kThreads) {  // columns Rk .. RkK - 1 (fewer than 32)
      const int i = e >> 5, c = e & 31;
      if (a.Rk + c < L.RkK) xT[i * L.xts + a.Rk + c] = 0.0f;
    }
    // E = 2 (sum_g Yhat_g - V) over the key rows, hi / lo in [r][v] and [v][r]
#pragma unroll
    for (int it = 0; it < kEItems; ++it) {
      const int e = t + it * kThreads;
      if (e < L.RkK * nv4) {
        const int r = e / nv4, v = (e - r * nv4) * 4;
        const bool ok = r < a.Rk;
        const float o0 = ok ? 2.0f * (ys[it].x - vv[it][0]) : 0.0f;
        const float o1 = ok ? 2.0f * (ys[it].y - vv[it][1]) : 0.0f;
        const float o2 = ok ? 2.0f * (ys[it].z - vv[it][2]) : 0.0f;
        const float o3 = ok ? 2.0f * (ys[it].w - vv[it][3]) : 0.0f;
        st_split4(eh, el, r * L.ers + v, o0, o1, o2, o3);
        st_split1(eth, etl, (v + 0) * L.ets + r, o0);
        st_split1(eth, etl, (v + 1) * L.ets + r, o1);
        st_split1(eth, etl, (v + 2) * L.ets + r, o2);
        st_split1(eth, etl, (v + 3) * L.ets + r, o3);
      }
    }
    // the finished chunk's outputs: query rows g, g + G, ... of this memory
#pragma unroll
    for (int it = 0; it < kYItems; ++it) {
      const int e = t + it * kThreads;
      const int j = e / nv4, v = (e - j * nv4) * 4;
      if (j < mine) {
        const int64_t yo = ((int64_t)m * a.ld + a.s_fin + g + j * a.G) * a.dv + v;
        const float4 s4 = yq[it];
        if (a.out_bf16) *(uint2*)((uint16_t*)a.Y + yo) = uint2{cvt_pk_bf16(s4.x, s4.y), cvt_pk_bf16(s4.z, s4.w)};
        else *(float4*)((float*)a.Y + yo) = s4;
      }
    }
    // second batch of loads: the state slices of the update and the forwarded chunk's raw rows,
    // their latency covered by the D1 product
#pragma unroll
      for (int j = 0; j < kT1; ++j) {
        const int f = (w + j * kWaves) * 16 + lr;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int o = f < a.din ? ((hs + lg * 4 + i) * a.din + f) * 4 : kOut;
          w1p[j][i] = buf_ld(R.W, o, 0);
          s1p[j][i] = buf_ld(R.S, o, 0);
        }
      }
#pragma unroll
      for (int j = 0; j < kT2; ++j) {
        const int vt = w + j * kWaves;
        const int o = vt < nvt ? ((int)a.P1 + (vt * 16 + lr) * a.dh + hs + lg * 4) * 4 : kOut;
        w2p[j] = buf_ld4(R.W, o, 0);
        s2p[j] = buf_ld4(R.S, o, 0);
      }
    load_rows();  // out of range when nothing is forwarded: no branch around the loads
    __syncthreads();

    // D1 = (E W2_g) * silu'(Z_g) and H_g over the key rows, scaled by the row coefficients,
    // transposed: [h][r]
    uint16_t* dwh = (uint16_t*)(sm + L.dwh);
    uint16_t* dwl = (uint16_t*)(sm + L.dwl);
    uint16_t* dsh = (uint16_t*)(sm + L.dsh);
    uint16_t* dsl = (uint16_t*)(sm + L.dsl);
    uint16_t* hwh = (uint16_t*)(sm + L.hwh);
    uint16_t* hwl = (uint16_t*)(sm + L.hwl);
    uint16_t* hsh_ = (uint16_t*)(sm + L.hsh);
    uint16_t* hsl_ = (uint16_t*)(sm + L.hsl);
#pragma unroll
    for (int j = 0; j < kZTiles; ++j) {
      const int rt = w + j * kWaves;
      if (rt < L.RkK / 16) {
        f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
        for (int v0 = 0; v0 < a.dv; v0 += 32) {
          const int ia = (rt * 16 + lr) * L.ers + v0 + lg * 8;
          const int ib = lr * L.w2ts + v0 + lg * 8;
          const u32x4 ah = *(const u32x4*)&eh[ia], al = *(const u32x4*)&el[ia];
          const u32x4 bh = *(const u32x4*)&w2th[ib], bl = *(const u32x4*)&w2tl[ib];
          acc = mfma16(ah, bh, acc);
          acc = mfma16(ah, bl, acc);
          acc = mfma16(al, bh, acc);
        }
        float dw[4], ds[4], hw[4], hs4[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = rt * 16 + lg * 4 + i;
          const float z = zp[j][i];
          const float sg = sigmoidf_(z);
          const float d1 = r < a.Rk ? acc[i] * (sg * (1.0f + z * (1.0f - sg))) : 0.0f;
          const float hv = r < a.Rk ? z * sg : 0.0f;
          dw[i] = cwL[r] * d1;
          ds[i] = csL[r] * d1;
          hw[i] = cwL[r] * hv;
          hs4[i] = csL[r] * hv;
        }
        const int io = lr * L.ets + rt * 16 + lg * 4;
        st_split4(dwh, dwl, io, dw[0], dw[1], dw[2], dw[3]);
        st_split4(dsh, dsl, io, ds[0], ds[1], ds[2], ds[3]);
        st_split4(hwh, hwl, io, hw[0], hw[1], hw[2], hw[3]);
        st_split4(hsh_, hsl_, io, hs4[0], hs4[1], hs4[2], hs4[3]);
      }
    }
    // the update's state values and the forwarded chunk's rows are taken here, in one wait: the
    // gradient tiles and the staging below then wait for nothing (a wait there would also wait for
    // the stores issued before it)
#pragma unroll
    for (int j = 0; j < kT1; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) asm volatile("" ::"v"(w1p[j][i]), "v"(s1p[j][i]));
#pragma unroll
    for (int j = 0; j < kT2; ++j) asm volatile("" ::"v"(w2p[j].x), "v"(w2p[j].y), "v"(w2p[j].z), "v"(w2p[j].w),
                                            "v"(s2p[j].x), "v"(s2p[j].y), "v"(s2p[j].z), "v"(s2p[j].w));
    asm volatile("" ::"v"(cP), "v"(cB), "v"(cA));
#pragma unroll
    for (int it = 0; it < kStage; ++it) asm volatile("" ::"v"(kx[it][0]), "v"(kx[it][1]), "v"(kx[it][2]), "v"(kx[it][3]));
    __syncthreads();

    // W1_g, S1_g: G1^W = (c^W D1)^T phi, G1^S = (c^S D1)^T phi; tiles of 16 features, the k-step
    // outermost so that its D1 fragments are read once for all of the wave's tiles
    f32x4 aw[kT1], as[kT1];
    uint32_t ents[kT1];
    const float* xi[kT1];
    const float* xj[kT1];
    float hf[kT1];
#pragma unroll
    for (int j = 0; j < kT1; ++j) {
      const int ft = w + j * kWaves;
      const uint32_t ent = tab[ft < nft ? ft * 16 + lr : lr];
      ents[j] = ent;
      xi[j] = xT + (ent & 255u) * L.xts;
      xj[j] = xT + ((ent >> 8) & 255u) * L.xts;
      hf[j] = (ent >> 16) & 1u ? 0.5f : 1.0f;
      aw[j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
      as[j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    }
    for (int r0 = 0; r0 < L.RkK; r0 += 32) {
      const int rr = r0 + lg * 8;
      const int ia = lr * L.ets + rr;
      const u32x4 awh = *(const u32x4*)&dwh[ia], awl = *(const u32x4*)&dwl[ia];
      const u32x4 ash = *(const u32x4*)&dsh[ia], asl = *(const u32x4*)&dsl[ia];
#pragma unroll
      for (int j = 0; j < kT1; ++j) {
        if (w + j * kWaves < nft) {
          const float4 i0 = *(const float4*)&xi[j][rr], i1 = *(const float4*)&xi[j][rr + 4];
          const float4 j0 = *(const float4*)&xj[j][rr], j1 = *(const float4*)&xj[j][rr + 4];
          const float h = hf[j];
          float v[8] = {(h * i0.x) * j0.x, (h * i0.y) * j0.y, (h * i0.z) * j0.z, (h * i0.w) * j0.w,
                        (h * i1.x) * j1.x, (h * i1.y) * j1.y, (h * i1.z) * j1.z, (h * i1.w) * j1.w};
          u32x4 bh, bl;
          if (EXACT) pack8_hi(v, bh);
          else pack8(v, bh, bl);
          aw[j] = mfma16(awh, bh, aw[j]);
          aw[j] = mfma16(awl, bh, aw[j]);
          as[j] = mfma16(ash, bh, as[j]);
          as[j] = mfma16(asl, bh, as[j]);
          if (!EXACT) {
            aw[j] = mfma16(awh, bl, aw[j]);
            as[j] = mfma16(ash, bl, as[j]);
          }
        }
      }
    }
#pragma unroll
    for (int j = 0; j < kT1; ++j) {
      const int ft = w + j * kWaves;
      if (ft < nft) {
        const int f = ft * 16 + lr;
        const bool fok = f < a.din;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int h = lg * 4 + i;
          // explicit fused multiply-adds, as in the other update epilogues
          const float wn = fmaf(cB, w1p[j][i], fmaf(cA, s1p[j][i], -aw[j][i]));
          const float sn = fmaf(cP, s1p[j][i], -as[j][i]);
          if (fok) {
            const int64_t e = (int64_t)m * a.P + (int64_t)(hs + h) * a.din + f;
            a.Wout[e] = wn;
            a.Sout[e] = sn;
            if (!isfinite(wn) || !isfinite(sn)) bad = true;
          }
          if (fwd) {
            if (QB) {  // into the block layout: its slot, the constant's fp32 weight apart
              const int slot = (int)(ents[j] >> 17);
              if (fok && slot == 0x7FFF) w1c[h] = wn;
              else if (fok) st_split1(w1h, w1l, h * L.w1s + slot, (ents[j] >> 16) & 1u ? 0.5f * wn : wn);
            } else {
              st_split1(w1h, w1l, h * L.w1s + f, fok ? wn : 0.0f);
            }
          }
        }
      }
    }
    // W2_g, S2_g: G2^T = (c H_g)^T E, tiles of 16 output columns
#pragma unroll
    for (int j = 0; j < kT2; ++j) {
      const int vt = w + j * kWaves;
      if (vt < nvt) {
        const int v = vt * 16 + lr;
        const int64_t e0 = (int64_t)m * a.P + a.P1 + (int64_t)v * a.dh + hs + lg * 4;
        f32x4 aw = {0.0f, 0.0f, 0.0f, 0.0f}, as = {0.0f, 0.0f, 0.0f, 0.0f};
        for (int r0 = 0; r0 < L.RkK; r0 += 32) {
          const int rr = r0 + lg * 8;
          const int ia = lr * L.ets + rr, ib = v * L.ets + rr;
          const u32x4 bh = *(const u32x4*)&eth[ib], bl = *(const u32x4*)&etl[ib];
          const u32x4 awh = *(const u32x4*)&hwh[ia], awl = *(const u32x4*)&hwl[ia];
          const u32x4 ash = *(const u32x4*)&hsh_[ia], asl = *(const u32x4*)&hsl_[ia];
          aw = mfma16(awh, bh, aw);
          aw = mfma16(awh, bl, aw);
          aw = mfma16(awl, bh, aw);
          as = mfma16(ash, bh, as);
          as = mfma16(ash, bl, as);
          as = mfma16(asl, bh, as);
        }
        const float wv[4] = {w2p[j].x, w2p[j].y, w2p[j].z, w2p[j].w};
        const float sv[4] = {s2p[j].x, s2p[j].y, s2p[j].z, s2p[j].w};
        float wn[4], sn[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          wn[i] = fmaf(cB, wv[i], fmaf(cA, sv[i], -aw[i]));
          sn[i] = fmaf(cP, sv[i], -as[i]);
          if (!isfinite(wn[i]) || !isfinite(sn[i])) bad = true;
        }
        *(float4*)(a.Wout + e0) = float4{wn[0], wn[1], wn[2], wn[3]};
        *(float4*)(a.Sout + e0) = float4{sn[0], sn[1], sn[2], sn[3]};
        if (fwd) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int h = lg * 4 + i;
            uint32_t hi, lo;
            split_bf16(wn[i], hi, lo);
            w2h[v * L.w2s + h] = (uint16_t)hi;
            w2l[v * L.w2s + h] = (uint16_t)lo;
            w2th[h * L.w2ts + v] = (uint16_t)hi;
            w2tl[h * L.w2ts + v] = (uint16_t)lo;
          }
        }
      }
    }
    __syncthreads();
  }

  if (fwd) {
    // ---------------------------------------------------------------- forward of chunk at s_fwd
    if (!fin) {
      load_rows();
      const float* b1 = Wm + (int64_t)hs * a.din;
      if (QB) {
        __syncthreads();  // the slice's zero slots are cleared first
        for (int e = t; e < HS * a.din; e += kThreads) {
          const int h = e / a.din, f = e - h * a.din;
          const uint32_t ent = tab[f];
          const float x = b1[(int64_t)h * a.din + f];
          const int slot = (int)(ent >> 17);
          if (slot == 0x7FFF) w1c[h] = x;
          else st_split1(w1h, w1l, h * L.w1s + slot, (ent >> 16) & 1u ? 0.5f * x : x);
        }
      } else {
        for (int e = t; e < HS * L.dinP; e += kThreads) {
          const int h = e / L.dinP, f = e - h * L.dinP;
          st_split1(w1h, w1l, h * L.w1s + f, f < a.din ? b1[(int64_t)h * a.din + f] : 0.0f);
        }
      }
    }
    float* xr = (float*)(sm + L.xr);
    uint16_t* hh = (uint16_t*)(sm + L.hh);
    uint16_t* hl = (uint16_t*)(sm + L.hl);
    const int nrow = L.RkT + L.nqT;
#pragma unroll
    for (int it = 0; it < kStage; ++it) {
      const int e = t + it * kThreads;
      if (e < (a.Rk + a.nq) * dq) {
        const int r = e / dq, q = e % dq;
        const int row = r < a.Rk ? r : L.RkT + (r - a.Rk);
        float* x = xr + row * L.xs + 8 * q;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          x[2 * u] = lo_bf16(kx[it][u]);
          x[2 * u + 1] = hi_bf16(kx[it][u]);
        }
      }
    }
    // the one and zero columns (dk .. dk + 3) of every row, then the padding rows (key rows
    // Rk .. RkT - 1, query rows nq .. nqT - 1: fewer than 32) as float4s, d_key / 4 <= 16 per row
    for (int e = t; e < nrow; e += kThreads) *(float4*)(xr + e * L.xs + a.dk) = float4{1.0f, 0.0f, 0.0f, 0.0f};
    {
      const int pk = L.RkT - a.Rk, pq = L.nqT - a.nq;
      const int p = t >> 4, q = t & 15;
      if (q < (a.dk >> 2) && p < pk + pq) {
        const int row = p < pk ? a.Rk + p : L.RkT + a.nq + (p - pk);
        *(float4*)(xr + row * L.xs + 4 * q) = float4{0.0f, 0.0f, 0.0f, 0.0f};
      }
    }
    __syncthreads();
    // Z_g = phi W1_g^T over key and query rows; H_g = silu(Z_g) into [row][h]
    for (int rt = w; rt < nrow / 16; rt += kWaves) {
      const float* xrow = xr + (rt * 16 + lr) * L.xs;
      f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
      if constexpr (QB > 0) {
        // the lane's raw row in registers; every feature of a step is a register product
        float xv[QB];
#pragma unroll
        for (int q = 0; q < QB / 4; ++q) {
          const float4 x4 = *(const float4*)(xrow + 4 * q);
          xv[4 * q] = x4.x;
          xv[4 * q + 1] = x4.y;
          xv[4 * q + 2] = x4.z;
          xv[4 * q + 3] = x4.w;
        }
        {  // step 0: the degree-1 features x_{8 lg + u} (exact bf16 values), zero past d_key
          const bool in = lg * 8 < QB;
          const float4 l0 = *(const float4*)(xrow + (in ? lg * 8 : 0));
          const float4 l1 = *(const float4*)(xrow + (in ? lg * 8 + 4 : 0));
          const float v[8] = {in ? l0.x : 0.0f, in ? l0.y : 0.0f, in ? l0.z : 0.0f, in ? l0.w : 0.0f,
                              in ? l1.x : 0.0f, in ? l1.y : 0.0f, in ? l1.z : 0.0f, in ? l1.w : 0.0f};
          u32x4 ah;
          pack8_hi(v, ah);
          const int ib = lr * L.w1s + lg * 8;
          const u32x4 bh = *(const u32x4*)&w1h[ib], bl = *(const u32x4*)&w1l[ib];
          acc = mfma16(ah, bh, acc);
          acc = mfma16(ah, bl, acc);
        }
        float xs4[QB / 4];  // x_{4 ib + lg}
#pragma unroll
        for (int ib = 0; ib < QB / 4; ++ib)
          xs4[ib] = lg == 0 ? xv[4 * ib] : lg == 1 ? xv[4 * ib + 1] : lg == 2 ? xv[4 * ib + 2] : xv[4 * ib + 3];
#pragma unroll
        for (int ib = 0; ib < QB / 4; ++ib) {
#pragma unroll
          for (int jb = ib / 2; jb < QB / 8; ++jb) {
            const int blk = quad_block0(QB, ib) + jb - ib / 2;
            float v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) v[u] = xs4[ib] * xv[8 * jb + u];  // exact: 16 significant bits
            u32x4 ah, al;
            pack8(v, ah, al);
            const int ib2 = lr * L.w1s + 32 * (1 + blk) + lg * 8;
            const u32x4 bh = *(const u32x4*)&w1h[ib2], bl = *(const u32x4*)&w1l[ib2];
            acc = mfma16(ah, bh, acc);
            acc = mfma16(ah, bl, acc);
            acc = mfma16(al, bh, acc);
          }
        }
        const float c0 = w1c[lr];
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] += c0;
      } else
      for (int f0 = 0; f0 < L.dinP; f0 += 32) {
        const int fb = f0 + lg * 8;
        const u32x4 e0 = *(const u32x4*)&tab[fb], e1 = *(const u32x4*)&tab[fb + 4];
        const uint32_t ent[8] = {e0[0], e0[1], e0[2], e0[3], e1[0], e1[1], e1[2], e1[3]};
        float v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = feat_eval(ent[u], xrow[ent[u] & 255u], xrow[(ent[u] >> 8) & 255u]);
        u32x4 ah, al;
        if (EXACT) pack8_hi(v, ah);
        else pack8(v, ah, al);
        const int ib = lr * L.w1s + fb;
        const u32x4 bh = *(const u32x4*)&w1h[ib], bl = *(const u32x4*)&w1l[ib];
        acc = mfma16(ah, bh, acc);
        acc = mfma16(ah, bl, acc);
        if (!EXACT) acc = mfma16(al, bh, acc);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = rt * 16 + lg * 4 + i;
        if (row < a.Rk) a.Z_wr[((int64_t)m * a.Rk + row) * a.dh + hs + lr] = acc[i];
        st_split1(hh, hl, row * L.hrs + lr, siluf_(acc[i]));
      }
    }
    __syncthreads();
    // partial outputs Yhat_g = H_g W2_g^T (k = 16)
    float* yw = a.Yp_wr + (int64_t)(m * a.G + g) * Rr * a.dv;
    for (int tile = w; tile < (nrow / 16) * nvt; tile += kWaves) {
      const int rt = tile / nvt, vt = tile - rt * nvt;
      const int ia = (rt * 16 + lr) * L.hrs + lg * 4;
      const int ib = (vt * 16 + lr) * L.w2s + lg * 4;
      const u32x2 ah = *(const u32x2*)&hh[ia], al = *(const u32x2*)&hl[ia];
      const u32x2 bh = *(const u32x2*)&w2h[ib], bl = *(const u32x2*)&w2l[ib];
      f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
      acc = mfma16k16(ah, bh, acc);
      acc = mfma16k16(ah, bl, acc);
      acc = mfma16k16(al, bh, acc);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = rt * 16 + lg * 4 + i;
        int lrow = -1;
        if (row < L.RkT) {
          if (row < a.Rk) lrow = row;
        } else if (row - L.RkT < a.nq) {
          lrow = a.Rk + (row - L.RkT);
        }
        if (lrow >= 0) yw[(int64_t)lrow * a.dv + vt * 16 + lr] = acc[i];
      }
    }
  }
  if (bad) a.flag[0] = 1;
}

// d_key of the block layout of degree-2 features, 0 when the table path runs
inline int block_qb(const Dims& d) { return d.poly == 2 && (d.dk == 16 || d.dk == 32) ? d.dk : 0; }

}  // namespace hsk

bool hsplit_supported(const Dims& d) {
  if (d.kind != ATLASMEM_MLP2_SILU || d.gated || d.residual || d.ptr || d.conv) return false;
  if (d.gate_mode != ATLASMEM_PER_TOKEN || d.ns_steps != 0 || d.prec != 1 || !d.in_bf16) return false;
  if (d.poly != 1 && d.poly != 2) return false;
  if (d.dh % hsk::HS != 0 || d.dh / hsk::HS > hsk::kMaxG) return false;
  if (d.dv % 32 != 0 || d.dk % 8 != 0 || d.dk > 64) return false;
  using namespace hsk;
  const int G = d.dh / HS;
  const Layout L = make_layout(d.dk, d.din, d.dv, d.Rk, d.C, block_qb(d));
  if ((d.Rk + d.C) * (d.dk / 8) > kStage * kThreads || (d.c - 1) * (d.dk / 8) > kThreads) return false;
  if (L.RkK * d.dv / 4 > kEItems * kThreads || L.RkK > 16 * kZTiles * kWaves) return false;
  if ((d.C + G - 1) / G * (d.dv / 4) > kYItems * kThreads) return false;
  if (L.dinP > 16 * kT1 * kWaves || d.dv > 16 * kT2 * kWaves || 16 * d.dv > kW2Items * kThreads) return false;
  return L.total <= kMaxLds;
}

int64_t hsplit_workspace_floats(const Dims& d) {
  const int G = d.dh / hsk::HS;
  return 2 * ((int64_t)d.M * G * (d.Rk + d.C) * d.dv + (int64_t)d.M * d.Rk * d.dh);
}

atlasmem_status launch_hsplit(Handle* h, const Dims& d, const void* K, const void* Q, const void* V, int64_t kb0,
                              int nb, int64_t ld, void* Y, hipStream_t st) {
  using namespace hsk;
  const int G = d.dh / HS;
  const int nq = Y ? d.C : 0;
  const int c = d.c;
  const int qb = block_qb(d);
  const Layout L = make_layout(d.dk, d.din, d.dv, d.Rk, nq, qb);
  if (L.total > kMaxLds || !h->hsw) return ATLASMEM_E_UNSUPPORTED;
  const int64_t ypf = (int64_t)d.M * G * (d.Rk + nq) * d.dv, zf = (int64_t)d.M * d.Rk * d.dh;
  float* yp[2] = {h->hsw, h->hsw + ypf};
  float* zb[2] = {h->hsw + 2 * ypf, h->hsw + 2 * ypf + zf};
  const bool exact = d.poly == 1;
  const void* kern = exact ? (const void*)hsplit_kernel<true, 0>
                           : qb == 32 ? (const void*)hsplit_kernel<false, 32>
                                      : qb == 16 ? (const void*)hsplit_kernel<false, 16> : (const void*)hsplit_kernel<false, 0>;
  if (hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, L.total) != hipSuccess)
    return ATLASMEM_E_DEVICE;
  Args a;
  a.K = (const uint16_t*)K;
  a.Q = (const uint16_t*)Q;
  a.V = (const uint16_t*)V;
  a.ld = ld;
  a.hk = h->hk[h->hcur];
  a.hv = h->hv[h->hcur];
  a.P = d.P;
  a.P1 = d.P1;
  a.ldc = c > 1 ? (int64_t)h->ncb * d.Rk : (int64_t)h->ncb * d.C;
  a.lds = (int64_t)h->ncb * 3;
  a.Y = Y;
  a.out_bf16 = d.out_bf16;
  a.M = d.M;
  a.G = G;
  a.dk = d.dk;
  a.din = d.din;
  a.dh = d.dh;
  a.dv = d.dv;
  a.Rk = d.Rk;
  a.nq = nq;
  a.c = c;
  a.poly = d.poly;
  a.flag = h->flag;
  // nb + 1 launches: the forward of the block's first chunk, then (finish k, forward k + 1), and
  // the finish of its last chunk
  for (int j = 0; j <= nb; ++j) {
    const int64_t kf = kb0 + j - 1;  // chunk finished by this launch (j >= 1)
    const int64_t kw = kb0 + j;      // chunk forwarded by this launch (j < nb)
    a.s_fin = j >= 1 ? kf * d.C : -1;
    a.s_fwd = j < nb ? kw * d.C : -1;
    const int kb = j - 1;
    a.cw = j >= 1 ? (c > 1 ? h->oW + (int64_t)kb * d.Rk : h->cW + (int64_t)kb * d.C) : nullptr;
    a.cs = j >= 1 ? (c > 1 ? h->oS + (int64_t)kb * d.Rk : h->cS + (int64_t)kb * d.C) : nullptr;
    a.scal = j >= 1 ? h->scal + (int64_t)kb * 3 : nullptr;
    a.Yp_rd = yp[kf & 1];
    a.Yp_wr = yp[kw & 1];
    a.Z_rd = zb[kf & 1];
    a.Z_wr = zb[kw & 1];
    a.Win = h->W[h->cur];
    a.Sin = h->S[h->cur];
    a.Wout = h->W[1 - h->cur];
    a.Sout = h->S[1 - h->cur];
    if (exact) hipLaunchKernelGGL((hsplit_kernel<true, 0>), dim3(d.M * G), dim3(kThreads), L.total, st, a);
    else if (qb == 32) hipLaunchKernelGGL((hsplit_kernel<false, 32>), dim3(d.M * G), dim3(kThreads), L.total, st, a);
    else if (qb == 16) hipLaunchKernelGGL((hsplit_kernel<false, 16>), dim3(d.M * G), dim3(kThreads), L.total, st, a);
    else hipLaunchKernelGGL((hsplit_kernel<false, 0>), dim3(d.M * G), dim3(kThreads), L.total, st, a);
    AM_LAUNCH_CHECK();
    if (j >= 1) h->cur = 1 - h->cur;
  }
  return ATLASMEM_OK;
}

}  // namespace am
