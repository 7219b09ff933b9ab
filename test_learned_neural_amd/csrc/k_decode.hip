// Streaming calls of a few tokens (decoding): one launch per call answers the call's queries from
// the current state and appends its key and value rows (and per-token gates) to the unfinished
// chunk, in place of the GEMM-engine retrieval and the strided copies.
//
// Retrieval of an MLP memory (titans-pytorch-mlx README, MAC Eq. 21: the memory is read without
// an update; the unfinished chunk's queries read the weights of its start, as inside a chunk;
// ATLAS summary, section 5.1: the residual and gated memories):
//   Z = W1 q (and Z3 = W3 q for the gated memory), H = silu(Z) (or silu(Z) * Z3),
//   y = W2 H (+ q for the residual memory).
// The products keep the library's precision policy: every fp32 operand is split into bf16
// hi + lo and a product is summed as hi*hi + hi*lo + lo*hi in fp32 (a bf16 input is exact and
// contributes no lo term; without the split only hi*hi), so answers do not depend on how the
// sequence is cut into calls beyond the order of fp32 accumulation.
//
// One 256-thread workgroup per memory: the queries go to LDS in fp32; a row of W1 q (and then of
// W2 H) is split over up to 64 lanes, each reading its segment of the weight row as 16-byte
// vectors, all issued before the products, and the partial sums meet by cross-lane reduction.
#include "common.h"
#include "internal.h"

namespace am {
namespace dk {

struct Args {
  const void* Q;   // the call's first token of memory 0; memory m at + m * ld rows
  const void* K;
  const void* V;
  int64_t ld;      // tokens per memory in the caller's arrays
  int n;           // tokens of this call
  int in_bf16;
  const float* W;  // state [M][P]
  int64_t P, P1;
  int din, dh, dv, dz;
  int gated, residual, split;
  void* Y;         // the call's first output row of memory 0 (null: no retrieval)
  int out_bf16;
  // the unfinished chunk: rows r0 .. r0 + n of [M][C][width] buffers (append = 0: retrieval only)
  int append;
  void* pK;
  void* pV;
  int C;
  int64_t r0;
  const float* th;  // per-token gates and gamma of the call (null: none), [M][ld]
  const float* et;
  const float* al;
  const float* gm;
  float* pth;
  float* pet;
  float* pal;
  float* pg;
  // One-token calls whose W1 (W2) product takes every thread once (dz (dv) rows x p lanes = 256)
  // with a segment of at most 32 floats: each thread loads its own W1 and W2 segments (w1v, w2v
  // float4) at the start, right after the query, so that every load of the call is in flight
  // at once and the call costs one memory latency.
  int w1v, w2v;
  // One-token calls on the matrix cores (mf): each wave takes whole 16-row tiles of W1 (then W2),
  // its segments loaded at the start in the A-operand layout of v_mfma_f32_16x16x32_bf16, and the
  // query (then H) is column 0 of the B operand; at most four tile-steps of a wave per product.
  int mf;
};

__device__ __forceinline__ void split1(float x, float& hi, float& lo) {
  uint32_t h, l;
  split_bf16(x, h, l);
  hi = bf16_value(h);
  lo = bf16_value(l);
}

// sum_i w[i] x[i] over a segment of one fp32 weight row (16-byte aligned, length a multiple of
// 4) and an fp32 vector in LDS whose bf16 halves are xh / xl (xl unused when x_exact).  The
// segment is read 64 floats at a time with every load issued before the products, so a
// segment of up to 64 floats costs one memory latency.
__device__ __forceinline__ float seg_dot(const float* __restrict__ w, const float* xh, const float* xl, int len,
                                         bool x_exact, bool split) {
  float ah[4] = {0.0f, 0.0f, 0.0f, 0.0f}, al[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int i0 = 0; i0 < len; i0 += 64) {
    float4 v[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) v[u] = (i0 + 4 * u < len) ? *(const float4*)(w + i0 + 4 * u) : float4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      if (i0 + 4 * u >= len) break;
      const float wv[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int i = i0 + 4 * u + c;
        float wh, wl;
        split1(wv[c], wh, wl);
        const float a = xh[i];
        ah[c] = fmaf(a, wh, ah[c]);
        if (split) {
          al[c] = fmaf(a, wl, al[c]);
          if (!x_exact) al[c] = fmaf(xl[i], wh, al[c]);
        }
      }
    }
  }
  return ((ah[0] + ah[1]) + (ah[2] + ah[3])) + ((al[0] + al[1]) + (al[2] + al[3]));
}

// sum_i w[i] x[i] over the lane's segment held in registers (nv float4, nv <= 8) and an fp32
// vector in LDS (hi / lo halves xh, xl): eight independent accumulators (the four elements of a
// vector, times the hi*hi and the lo-word terms), so the multiply-add chains stay short.
__device__ __forceinline__ float reg_dot(const float4* w, int nv, const float* xh, const float* xl, bool x_exact,
                                         bool split) {
  float ah[4] = {0.0f, 0.0f, 0.0f, 0.0f}, al[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    if (u >= nv) break;
    const float4 x4 = *(const float4*)(xh + 4 * u);
    const float4 l4 = x_exact ? float4{0.0f, 0.0f, 0.0f, 0.0f} : *(const float4*)(xl + 4 * u);
    const float wv[4] = {w[u].x, w[u].y, w[u].z, w[u].w};
    const float xv[4] = {x4.x, x4.y, x4.z, x4.w};
    const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      float wh, wl;
      split1(wv[c], wh, wl);
      ah[c] = fmaf(xv[c], wh, ah[c]);
      if (split) {
        al[c] = fmaf(xv[c], wl, al[c]);
        if (!x_exact) al[c] = fmaf(lv[c], wh, al[c]);
      }
    }
  }
  return ((ah[0] + ah[1]) + (ah[2] + ah[3])) + ((al[0] + al[1]) + (al[2] + al[3]));
}

// Lanes per output row: the most (a power of two up to 64) that keeps every lane busy with a
// segment of whole 16-byte vectors.
__device__ __forceinline__ int lanes_per_row(int rows, int len) {
  int p = 1;
  while (p < 64 && rows * p * 2 <= 256 && len % (8 * p) == 0) p *= 2;
  return p;
}

__device__ __forceinline__ void retrieve(const Args& a, int z, int t, int n, int64_t row0) {
  extern __shared__ float ds[];
  // the query first, then the weight segments: waiting for the query waits for nothing younger
  const bool q_exact = a.in_bf16;
  float qv = 0.0f;
  const bool q1 = n * a.din <= 256;  // one query element per thread
  if (q1 && t < n * a.din) qv = load_in(a.Q, row0 * a.din + t, a.in_bf16);
  float4 w1r[8];
  const int lane = t & 63, wv = t >> 6, lr = lane & 15, lg = lane >> 4;
  if (a.mf) {  // tile-step s of this wave: row tile wv + 4 (s / KS1), k-step s % KS1
    const int KS1 = a.din / 32, nts = (a.dz / 64) * KS1;
    const float* w1 = a.W + (int64_t)z * a.P;
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) {
      if (s4 >= nts) break;
      const int row = (wv + 4 * (s4 / KS1)) * 16 + lr, k0 = (s4 % KS1) * 32 + lg * 8;
      w1r[2 * s4] = *(const float4*)(w1 + (int64_t)row * a.din + k0);
      w1r[2 * s4 + 1] = *(const float4*)(w1 + (int64_t)row * a.din + k0 + 4);
    }
  }
  if (a.w1v) {
    const int p = lanes_per_row(a.dz, a.din), seg = a.din / p;
    const float4* w1 = (const float4*)(a.W + (int64_t)z * a.P + (int64_t)(t / p) * a.din + (t % p) * seg);
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (u < a.w1v) w1r[u] = w1[u];
  }
  float4 w2r[8];
  if (a.mf) {
    const int KS2 = a.dh / 32, nts = (a.dv / 64) * KS2;
    const float* w2 = a.W + (int64_t)z * a.P + a.P1;
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) {
      if (s4 >= nts) break;
      const int row = (wv + 4 * (s4 / KS2)) * 16 + lr, k0 = (s4 % KS2) * 32 + lg * 8;
      w2r[2 * s4] = *(const float4*)(w2 + (int64_t)row * a.dh + k0);
      w2r[2 * s4 + 1] = *(const float4*)(w2 + (int64_t)row * a.dh + k0 + 4);
    }
  }
  if (a.w2v) {
    const int p = lanes_per_row(a.dv, a.dh), seg = a.dh / p;
    const float4* w2 = (const float4*)(a.W + (int64_t)z * a.P + a.P1 + (int64_t)(t / p) * a.dh + (t % p) * seg);
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (u < a.w2v) w2r[u] = w2[u];
  }
  // LDS: q hi, q lo [n][din]; Z [n][dz]; H hi, H lo [n][dh]
  float* qh = ds;
  float* ql = qh + n * a.din;
  float* zs = ql + n * a.din;
  float* hh = zs + n * a.dz;
  float* hl = hh + n * a.dh;
  for (int e = t; e < n * a.din; e += 256) {
    const float x = q1 ? qv : load_in(a.Q, row0 * a.din + e, a.in_bf16);
    float h, l;
    split1(x, h, l);
    qh[e] = q_exact ? x : h;
    ql[e] = q_exact ? 0.0f : l;
  }
  __syncthreads();
  const float* W1 = a.W + (int64_t)z * a.P;
  const float* W2 = W1 + a.P1;
  if (a.mf) {  // Z = W1 q on the matrix cores
    const int KS1 = a.din / 32, nts = (a.dz / 64) * KS1;
    f32x4 acc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) {
      if (s4 >= nts) break;
      const float wv8[8] = {w1r[2 * s4].x, w1r[2 * s4].y, w1r[2 * s4].z, w1r[2 * s4].w,
                            w1r[2 * s4 + 1].x, w1r[2 * s4 + 1].y, w1r[2 * s4 + 1].z, w1r[2 * s4 + 1].w};
      u32x4 ah, al;
      pack8(wv8, ah, al);
      const int k0 = (s4 % KS1) * 32 + lg * 8;
      float xh8[8], xl8[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        xh8[u] = lr == 0 ? qh[k0 + u] : 0.0f;
        xl8[u] = lr == 0 && !q_exact ? ql[k0 + u] : 0.0f;
      }
      u32x4 bh, bl;
      pack8_hi(xh8, bh);
      pack8_hi(xl8, bl);
      const int i = s4 / KS1;
      acc[i] = mfma16(ah, bh, acc[i]);
      if (a.split) {
        acc[i] = mfma16(al, bh, acc[i]);
        if (!q_exact) acc[i] = mfma16(ah, bl, acc[i]);
      }
    }
    if (lr == 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (i >= a.dz / 64) break;
#pragma unroll
        for (int r = 0; r < 4; ++r) zs[(wv + 4 * i) * 16 + lg * 4 + r] = acc[i][r];
      }
    }
  } else {  // Z = W1 q: p lanes per (token, row), partial sums reduced across the p lanes
    const int p = lanes_per_row(n * a.dz, a.din), seg = a.din / p;
    for (int e0 = 0; e0 < n * a.dz * p; e0 += 256) {
      const int e = e0 + t, task = e / p, part = e - task * p;
      float acc = 0.0f;
      if (a.w1v) {  // n = 1, one task per thread: row t / p, segment t % p, weights in registers
        const int i0 = part * seg;
        acc = reg_dot(w1r, a.w1v, qh + i0, ql + i0, q_exact, a.split);
      } else if (task < n * a.dz) {
        const int tt = task / a.dz, j = task - tt * a.dz, i0 = part * seg;
        acc = seg_dot(W1 + (int64_t)j * a.din + i0, qh + tt * a.din + i0, ql + tt * a.din + i0, seg, q_exact,
                      a.split);
      }
      for (int off = 1; off < p; off <<= 1) acc += __shfl_xor(acc, off, 64);
      if (task < n * a.dz && part == 0) zs[task] = acc;
    }
  }
  __syncthreads();
  for (int e = t; e < n * a.dh; e += 256) {
    const int tt = e / a.dh, j = e - tt * a.dh;
    const float zv = zs[tt * a.dz + j];
    const float hv = a.gated ? siluf_(zv) * zs[tt * a.dz + a.dh + j] : siluf_(zv);
    float h, l;
    split1(hv, h, l);
    hh[e] = h;
    hl[e] = l;
  }
  __syncthreads();
  if (a.mf) {  // y = W2 H (+ q) on the matrix cores
    const int KS2 = a.dh / 32, nts = (a.dv / 64) * KS2;
    f32x4 acc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) {
      if (s4 >= nts) break;
      const float wv8[8] = {w2r[2 * s4].x, w2r[2 * s4].y, w2r[2 * s4].z, w2r[2 * s4].w,
                            w2r[2 * s4 + 1].x, w2r[2 * s4 + 1].y, w2r[2 * s4 + 1].z, w2r[2 * s4 + 1].w};
      u32x4 ah, al;
      pack8(wv8, ah, al);
      const int k0 = (s4 % KS2) * 32 + lg * 8;
      float xh8[8], xl8[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        xh8[u] = lr == 0 ? hh[k0 + u] : 0.0f;
        xl8[u] = lr == 0 ? hl[k0 + u] : 0.0f;
      }
      u32x4 bh, bl;
      pack8_hi(xh8, bh);
      pack8_hi(xl8, bl);
      const int i = s4 / KS2;
      acc[i] = mfma16(ah, bh, acc[i]);
      if (a.split) {
        acc[i] = mfma16(al, bh, acc[i]);
        acc[i] = mfma16(ah, bl, acc[i]);
      }
    }
    if (lr == 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (i >= a.dv / 64) break;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int v = (wv + 4 * i) * 16 + lg * 4 + r;
          float y = acc[i][r];
          if (a.residual) y += load_in(a.Q, row0 * a.din + v, a.in_bf16);  // din = dv
          const int64_t o = row0 * a.dv + v;
          if (a.out_bf16) ((uint16_t*)a.Y)[o] = (uint16_t)bf16_bits(y);
          else ((float*)a.Y)[o] = y;
        }
      }
    }
  } else {  // y = W2 H (+ q)
    const int p = lanes_per_row(n * a.dv, a.dh), seg = a.dh / p;
    for (int e0 = 0; e0 < n * a.dv * p; e0 += 256) {
      const int e = e0 + t, task = e / p, part = e - task * p;
      float y = 0.0f;
      if (a.w2v) {  // n = 1, one task per thread: row t / p, segment t % p, weights in registers
        const int i0 = part * seg;
        y = reg_dot(w2r, a.w2v, hh + i0, hl + i0, false, a.split);
      } else if (task < n * a.dv) {
        const int tt = task / a.dv, v = task - tt * a.dv, i0 = part * seg;
        y = seg_dot(W2 + (int64_t)v * a.dh + i0, hh + tt * a.dh + i0, hl + tt * a.dh + i0, seg, false, a.split);
      }
      for (int off = 1; off < p; off <<= 1) y += __shfl_xor(y, off, 64);
      if (task < n * a.dv && part == 0) {
        const int tt = task / a.dv, v = task - tt * a.dv;
        if (a.residual) y += load_in(a.Q, (row0 + tt) * a.din + v, a.in_bf16);  // din = dv
        const int64_t o = (row0 + tt) * a.dv + v;
        if (a.out_bf16) ((uint16_t*)a.Y)[o] = (uint16_t)bf16_bits(y);
        else ((float*)a.Y)[o] = y;
      }
    }
  }
}


__global__ void __launch_bounds__(256) decode_kernel(Args a) {
  const int z = blockIdx.x, t = threadIdx.x, n = a.n;
  const size_t esz = a.in_bf16 ? 2 : 4;
  // the call's rows of this memory: token tt of memory z is row z * ld + tt
  const int64_t row0 = (int64_t)z * a.ld;
  // The append (keys, values and per-token gates into the unfinished chunk) is loaded first and
  // stored after the retrieval: every load of the call is then in flight at once, and the call
  // costs one memory latency.  Rows of whole 16-byte pieces that fit one piece per thread take
  // that path; others are copied at the end.
  const int64_t kw = (int64_t)a.din * esz, vw = (int64_t)a.dv * esz;  // row bytes (identity features: din = dk)
  const char* ks = (const char*)a.K + row0 * kw;
  const char* vs = (const char*)a.V + row0 * vw;
  char* kd = (char*)a.pK + ((int64_t)z * a.C + a.r0) * kw;
  char* vd = (char*)a.pV + ((int64_t)z * a.C + a.r0) * vw;
  const bool wide = a.append &&
                    ((kw | vw | (uintptr_t)ks | (uintptr_t)vs | (uintptr_t)kd | (uintptr_t)vd) & 15) == 0 &&
                    n * kw / 16 <= 256 && n * vw / 16 <= 256;
  uint4 kp = {0u, 0u, 0u, 0u}, vp = {0u, 0u, 0u, 0u};
  if (wide) {
    if (t < n * kw / 16) kp = ((const uint4*)ks)[t];
    if (t < n * vw / 16) vp = ((const uint4*)vs)[t];
  }
  float g4[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  const int64_t src = row0 + t, dst = (int64_t)z * a.C + a.r0 + t;
  if (a.append && t < n) {
    if (a.th) {
      g4[0] = a.th[src];
      g4[1] = a.et[src];
      g4[2] = a.al[src];
    }
    if (a.gm) g4[3] = a.gm[src];
  }
  if (a.Y) retrieve(a, z, t, n, row0);
  if (a.append) {
    if (wide) {
      if (t < n * kw / 16) ((uint4*)kd)[t] = kp;
      if (t < n * vw / 16) ((uint4*)vd)[t] = vp;
    } else {
      for (int64_t e = t; e < n * kw / 2; e += 256) ((uint16_t*)kd)[e] = ((const uint16_t*)ks)[e];
      for (int64_t e = t; e < n * vw / 2; e += 256) ((uint16_t*)vd)[e] = ((const uint16_t*)vs)[e];
    }
    if (t < n) {
      if (a.th) {
        a.pth[dst] = g4[0];
        a.pet[dst] = g4[1];
        a.pal[dst] = g4[2];
      }
      if (a.gm) a.pg[dst] = g4[3];
    }
  }
}

}  // namespace dk

constexpr int kDecodeMaxTokens = 8;
constexpr int kDecodeMaxLds = 64 * 1024;

static size_t decode_lds(const Dims& d, int64_t n) {
  return sizeof(float) * (size_t)n * (2 * (size_t)d.din + (size_t)d.dz + 2 * (size_t)d.dh);
}

bool decode_supported(const Dims& d, int64_t n) {
  return d.kind == ATLASMEM_MLP2_SILU && d.poly == 1 && !d.ptr && d.prec != 2 && n >= 1 && n <= kDecodeMaxTokens &&
         d.din % 4 == 0 && d.dh % 4 == 0 && decode_lds(d, n) <= (size_t)kDecodeMaxLds;
}

atlasmem_status launch_decode(Handle* h, const void* Q, const void* K, const void* V, const float* theta,
                              const float* eta, const float* alpha, const float* gamma, int64_t ld, int64_t n,
                              void* Y, bool append, hipStream_t st) {
  const Dims& d = h->d;
  if (!decode_supported(d, n)) return ATLASMEM_E_UNSUPPORTED;
  if (append && (h->pending + n > d.C || !K || !V || (d.c > 1 && !gamma) ||
                 (d.gate_mode == ATLASMEM_PER_TOKEN && (!theta || !eta || !alpha))))
    return ATLASMEM_E_UNSUPPORTED;
  if (!append && !Y) return ATLASMEM_OK;
  dk::Args a;
  a.Q = Q;
  a.K = K;
  a.V = V;
  a.ld = ld;
  a.n = (int)n;
  a.in_bf16 = d.in_bf16;
  a.W = h->W[h->cur];
  a.P = d.P;
  a.P1 = d.P1;
  a.din = d.din;
  a.dh = d.dh;
  a.dv = d.dv;
  a.dz = d.dz;
  a.gated = d.gated;
  a.residual = d.residual;
  a.split = d.split;
  a.Y = Y;
  a.out_bf16 = d.out_bf16;
  a.append = append;
  a.pK = h->pK;
  a.pV = h->pV;
  a.C = d.C;
  a.r0 = h->pending;
  const bool per_token = d.gate_mode == ATLASMEM_PER_TOKEN;
  a.th = per_token ? theta : nullptr;
  a.et = per_token ? eta : nullptr;
  a.al = per_token ? alpha : nullptr;
  a.gm = d.c > 1 ? gamma : nullptr;
  a.pth = h->pth;
  a.pet = h->pet;
  a.pal = h->pal;
  a.pg = h->pg;
  a.w1v = a.w2v = 0;
  a.mf = Y && n == 1 && d.P % 4 == 0 && d.P1 % 4 == 0 && d.din % 32 == 0 && d.dz % 64 == 0 && d.dz * d.din <= 8192 &&
         d.dh % 32 == 0 && d.dv % 64 == 0 && d.dv * d.dh <= 8192;
  if (Y && n == 1 && !a.mf && d.P % 4 == 0 && d.P1 % 4 == 0) {  // the kernel's lane splits of the two products
    int p = 1;
    while (p < 64 && d.dv * p * 2 <= 256 && d.dh % (8 * p) == 0) p *= 2;
    if (d.dv * p == 256 && (d.dh / p) % 4 == 0 && d.dh / p <= 32) a.w2v = d.dh / p / 4;
    p = 1;
    while (p < 64 && d.dz * p * 2 <= 256 && d.din % (8 * p) == 0) p *= 2;
    if (d.dz * p == 256 && (d.din / p) % 4 == 0 && d.din / p <= 32) a.w1v = d.din / p / 4;
  }
  hipLaunchKernelGGL(dk::decode_kernel, dim3(d.M), dim3(256), Y ? decode_lds(d, n) : 0, st, a);
  AM_LAUNCH_CHECK();
  if (append) h->pending += n;
  return ATLASMEM_OK;
}

}  // namespace am
