// Gate scan, Omega-window coefficients, window history and the stand-alone feature map.
//
// Gate scan.  Inside a chunk every gradient g_j is taken at the chunk-start weights, so the
// per-token momentum / forgetting recurrence (titans-pytorch-mlx README, Core Equations,
// Eq. 13-14) unrolls to S_end = P S0 - sum_j cS_j g_j, W_end = beta W0 + a_S S0 - sum_j cW_j g_j.
// The pair (b_j, w_j) of forgetting product and W-weight obeys
//   [b_j; w_j] = M_{j+1} [b_{j+1}; w_{j+1}],  M_l = [[1 - alpha_l, 0], [1 - alpha_l, eta_l]],
// with b_C = w_C = 1, so [b_j; w_j] = L_j [1; 1] where L_j = M_{j+1} ... M_C is a suffix product
// of 2x2 lower-triangular matrices; e_j = prod_{l>j} eta_l is L_j's lower-right entry.  One wave64
// computes the suffix products of 64 tokens in six shuffle steps (division free), carrying the
// product of later 64-token blocks for chunks longer than a wave.
#include "common.h"
#include "internal.h"

namespace am {

struct Lt {  // [[a, 0], [c, d]]
  float a, c, d;
};
__device__ __forceinline__ Lt lt_mul(Lt x, Lt y) { return Lt{x.a * y.a, x.c * y.a + x.d * y.c, x.d * y.d}; }
__device__ __forceinline__ Lt lt_shfl_down(Lt x, int off) {
  return Lt{__shfl_down(x.a, off, 64), __shfl_down(x.c, off, 64), __shfl_down(x.d, off, 64)};
}

__global__ void __launch_bounds__(256) gate_scan_kernel(const float* __restrict__ theta, const float* __restrict__ eta,
                                                        const float* __restrict__ alpha, int M, int64_t ld_gate,
                                                        int64_t t0, int nchunks, int C, float* __restrict__ cW,
                                                        float* __restrict__ cS, int64_t ld_c,
                                                        float* __restrict__ scal, int64_t ld_s) {
  const int64_t wave = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  const int lane = threadIdx.x & 63;
  if (wave >= (int64_t)M * nchunks) return;  // uniform per wave
  const int m = (int)(wave / nchunks), kc = (int)(wave % nchunks);
  const int64_t g0 = (int64_t)m * ld_gate + t0 + (int64_t)kc * C;
  const int64_t o0 = (int64_t)m * ld_c + (int64_t)kc * C;
  Lt carry{1.0f, 0.0f, 1.0f};
  for (int b0 = ((C - 1) / 64) * 64; b0 >= 0; b0 -= 64) {
    const int j = b0 + lane;
    const bool valid = j < C;
    const float et = valid ? eta[g0 + j] : 1.0f;
    const float al = valid ? alpha[g0 + j] : 0.0f;
    const float th = valid ? theta[g0 + j] : 0.0f;
    Lt U = valid ? Lt{1.0f - al, 1.0f - al, et} : Lt{1.0f, 0.0f, 1.0f};
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {  // inclusive suffix product inside the block
      Lt o = lt_shfl_down(U, off);
      if (lane + off < 64) U = lt_mul(U, o);
    }
    U = lt_mul(U, carry);  // ... times every later block: U_j = M_j ... M_C
    Lt L = lt_shfl_down(U, 1);
    if (lane == 63) L = carry;  // L_j = U_{j+1}
    if (valid) {
      cS[o0 + j] = th * L.d;
      cW[o0 + j] = th * (L.c + L.d);
    }
    if (b0 == 0 && lane == 0) {
      float* sc = scal + (int64_t)m * ld_s + (int64_t)kc * 3;
      sc[0] = U.d;                  // prod eta
      sc[1] = U.a;                  // prod (1 - alpha)
      sc[2] = et * (L.c + L.d);     // a_S = eta_1 w_1
    }
    carry = Lt{__shfl(U.a, 0, 64), __shfl(U.c, 0, 64), __shfl(U.d, 0, 64)};
  }
}

atlasmem_status launch_gate_scan(const float* theta, const float* eta, const float* alpha, int M, int64_t ld_gate,
                                 int64_t t0, int nchunks, int C, float* cW, float* cS, int64_t ld_c, float* scal,
                                 int64_t ld_s, hipStream_t st) {
  const int64_t waves = (int64_t)M * nchunks;
  if (waves == 0) return ATLASMEM_OK;
  const int64_t blocks = (waves + 3) / 4;
  hipLaunchKernelGGL(gate_scan_kernel, dim3((unsigned)blocks), dim3(256), 0, st, theta, eta, alpha, M, ld_gate, t0,
                     nchunks, C, cW, cS, ld_c, scal, ld_s);
  AM_LAUNCH_CHECK();
  return ATLASMEM_OK;
}

// Omega window (ATLAS summary, section 3.2): the step-t gradient sums gamma_i g_i over the last c
// tokens, so g_i's coefficient in the chunk is gamma_i times the sum of the per-step coefficients
// c_t over the steps t in [i, i + c - 1] that fall inside the chunk.  Row r of chunk [s, s + C)
// is token i = s - (c - 1) + r; tokens before the call come from the window history.
__global__ void __launch_bounds__(256) omega_kernel(const float* __restrict__ cW, const float* __restrict__ cS,
                                                    int64_t ld_c, const float* __restrict__ gamma, int64_t ld_g,
                                                    const float* __restrict__ ghist, int M, int64_t s0, int nchunks,
                                                    int C, int c, float* __restrict__ oW, float* __restrict__ oS,
                                                    int64_t ld_o) {
  const int Rk = C + c - 1;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t total = (int64_t)M * nchunks * Rk;
  if (idx >= total) return;
  const int r = (int)(idx % Rk);
  const int kc = (int)((idx / Rk) % nchunks);
  const int m = (int)(idx / ((int64_t)Rk * nchunks));
  const int64_t s = s0 + (int64_t)kc * C;
  const int64_t i = s - (c - 1) + r;
  float g = 0.0f;
  if (i >= 0) g = gamma[(int64_t)m * ld_g + i];
  else if (ghist) g = ghist[(int64_t)m * (c - 1) + (c - 1) + i];
  const int64_t t_lo = i > s ? i : s;
  const int64_t t_hi = (i + c - 1) < (s + C - 1) ? (i + c - 1) : (s + C - 1);
  float sw = 0.0f, ss = 0.0f;
  for (int64_t t = t_lo; t <= t_hi; ++t) {
    sw += cW[(int64_t)m * ld_c + (t - s0)];
    ss += cS[(int64_t)m * ld_c + (t - s0)];
  }
  const int64_t o = (int64_t)m * ld_o + (int64_t)kc * Rk + r;
  oW[o] = g * sw;
  oS[o] = g * ss;
}

atlasmem_status launch_omega(const float* cW, const float* cS, int64_t ld_c, const float* gamma, int64_t ld_g,
                             const float* ghist, int M, int64_t s0, int nchunks, int C, int c, float* oW, float* oS,
                             int64_t ld_o, hipStream_t st) {
  const int64_t total = (int64_t)M * nchunks * (C + c - 1);
  if (total == 0) return ATLASMEM_OK;
  hipLaunchKernelGGL(omega_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st, cW, cS, ld_c, gamma, ld_g,
                     ghist, M, s0, nchunks, C, c, oW, oS, ld_o);
  AM_LAUNCH_CHECK();
  return ATLASMEM_OK;
}

// Per-token retrieval reads W_t, the state right after token t's update.  Inside a chunk that
// starts from (W0, S0) with per-token gates (titans-pytorch-mlx README, Eq. 13-14), every
// gradient taken at the chunk-start weights,
//   S_t = P_t S0 - sum_{l<=t} E_{t,l} theta_l G_l,  E_{t,l} = prod_{n=l+1..t} eta_n, P_t = prod_{n<=t} eta_n
//   W_t = beta_t W0 + a_t S0 - sum_{l<=t} w_{t,l} theta_l G_l,  beta_t = prod_{l<=t} (1 - alpha_l),
// with a_t = (1 - alpha_t) a_{t-1} + P_t and w_{t,l} = (1 - alpha_t) w_{t-1,l} + E_{t,l}, w_{l,l} = 1.
// With the Omega window G_l = sum_{i=l-c+1..l} gamma_i g_i (ATLAS summary, section 3.2), so g_i
// enters W_t with Om_{t,i} = gamma_i sum_{l in [max(i, s), min(i + c - 1, t)]} w_{t,l} theta_l.
// One block per memory walks the chunk's tokens in order; w and E live in LDS, one column per l.
// Om[t][r] = gamma_r * sum over the tokens l of key row r's window (l <= t) of theta_l w_{t,l}, with
// w_{l,l} = E_{l,l} = 1 and, for t > l, E_{t,l} = eta_t E_{t-1,l}, w_{t,l} = (1 - alpha_t) w_{t-1,l}
// + E_{t,l}: each (t, l) sequence is its own scalar recurrence in t, so thread r carries the
// w and E of its window's (at most PTR_MAXC) tokens in registers through the chunk, with no
// barrier per token.  beta_t and a_t follow from the gates alone (the block's last thread, so
// that this scan runs beside the key rows of the first waves).
constexpr int PTR_MAXC = 8;
__global__ void ptr_coeff_kernel(const float* __restrict__ theta, const float* __restrict__ eta,
                                 const float* __restrict__ alpha, const float* __restrict__ gamma, int64_t ld,
                                 const float* __restrict__ ghist, int64_t s0, int C, int c, float* __restrict__ bA,
                                 float* __restrict__ Om) {
  extern __shared__ float pc[];  // the chunk's gates th, et, al [C]
  float* th = pc;
  float* et = pc + C;
  float* al = pc + 2 * C;
  const int m = blockIdx.x;
  const int Rk = C + c - 1;
  for (int l = threadIdx.x; l < C; l += blockDim.x) {
    const int64_t o = (int64_t)m * ld + s0 + l;
    th[l] = theta[o];
    et[l] = eta[o];
    al[l] = alpha[o];
  }
  __syncthreads();
  if (threadIdx.x == blockDim.x - 1) {  // the last wave: the key rows start on wave 0
    float beta = 1.0f, a = 0.0f, P = 1.0f;
    for (int t = 0; t < C; ++t) {
      const float om = 1.0f - al[t], e = et[t];
      P *= e;
      a = om * a + P;
      beta *= om;
      bA[((int64_t)m * C + t) * 2] = beta;
      bA[((int64_t)m * C + t) * 2 + 1] = a;
    }
  }
  for (int r = threadIdx.x; r < Rk; r += blockDim.x) {
    const int i = r - (c - 1);  // chunk-relative token of key row r (negative: window history)
    float g = 1.0f;
    if (c > 1) {  // gamma of token s0 + i of the call, or of the history before the call
      const int64_t tau = s0 + i;
      g = (tau >= 0) ? gamma[(int64_t)m * ld + tau] : ghist[(int64_t)m * (c - 1) + (c - 1) + tau];
    }
    const int lo = i > 0 ? i : 0;             // first window token inside the chunk
    const int hi = (i + c - 1) < C ? (i + c - 1) : C - 1;
    float w[PTR_MAXC], E[PTR_MAXC];
#pragma unroll
    for (int q = 0; q < PTR_MAXC; ++q) w[q] = E[q] = 0.0f;
    float* col = Om + (int64_t)m * C * Rk + r;
#pragma unroll 4
    for (int t = 0; t < C; ++t) {  // unrolled: four tokens' gate loads from LDS issued together
      const float om = 1.0f - al[t], e = et[t];
      float v = 0.0f;
#pragma unroll
      for (int q = 0; q < PTR_MAXC; ++q) {
        const int l = lo + q;
        if (l > hi) break;
        if (l < t) {
          E[q] = e * E[q];
          w[q] = om * w[q] + E[q];
        } else if (l == t) {
          E[q] = 1.0f;
          w[q] = 1.0f;
        }
        if (l <= t) v += th[l] * w[q];
      }
      col[(int64_t)t * Rk] = (i <= t) ? ((c > 1) ? v * g : v) : 0.0f;
    }
  }
}

// Windows wider than PTR_MAXC: the same coefficients token by token, the block walking the
// chunk with two barriers per token.
__global__ void ptr_coeff_seq_kernel(const float* __restrict__ theta, const float* __restrict__ eta,
                                 const float* __restrict__ alpha, const float* __restrict__ gamma, int64_t ld,
                                 const float* __restrict__ ghist, int64_t s0, int C, int c, float* __restrict__ bA,
                                 float* __restrict__ Om) {
  // w[C], E[C], tw[C], then the chunk's gates th, et, al [C] and the key rows' gamma [Rk], staged
  // once so that the sequential loop over the chunk's tokens makes no global loads
  extern __shared__ float pc[];
  float* w = pc;
  float* E = pc + C;
  float* tw = pc + 2 * C;
  float* th = pc + 3 * C;
  float* et = pc + 4 * C;
  float* al = pc + 5 * C;
  float* gr = pc + 6 * C;
  const int m = blockIdx.x;
  const int Rk = C + c - 1;
  for (int l = threadIdx.x; l < C; l += blockDim.x) {
    const int64_t o = (int64_t)m * ld + s0 + l;
    th[l] = theta[o];
    et[l] = eta[o];
    al[l] = alpha[o];
  }
  if (c > 1) {
    for (int r = threadIdx.x; r < Rk; r += blockDim.x) {  // gamma of token s0 + r - (c - 1)
      const int64_t tau = s0 + r - (c - 1);
      gr[r] = (tau >= 0) ? gamma[(int64_t)m * ld + tau] : ghist[(int64_t)m * (c - 1) + (c - 1) + tau];
    }
  }
  __syncthreads();
  float beta = 1.0f, a = 0.0f, P = 1.0f;
  for (int t = 0; t < C; ++t) {
    const float om = 1.0f - al[t], e = et[t];
    for (int l = threadIdx.x; l < C; l += blockDim.x) {
      float wl, El;
      if (l < t) {
        El = e * E[l];
        wl = om * w[l] + El;
      } else {
        El = 1.0f;
        wl = 1.0f;
      }
      if (l <= t) {
        E[l] = El;
        w[l] = wl;
      }
      tw[l] = (l <= t) ? th[l] * wl : 0.0f;
    }
    P *= e;
    a = om * a + P;
    beta *= om;
    __syncthreads();
    float* orow = Om + ((int64_t)m * C + t) * Rk;
    for (int r = threadIdx.x; r < Rk; r += blockDim.x) {
      const int i = r - (c - 1);  // chunk-relative token of key row r (negative: window history)
      float v = 0.0f;
      if (i <= t) {
        const int lo = i > 0 ? i : 0;
        const int hi = (i + c - 1) < t ? (i + c - 1) : t;
        for (int l = lo; l <= hi; ++l) v += tw[l];
        if (c > 1) v *= gr[r];  // gamma of token s0 + i of the call, or of the history before it
      }
      orow[r] = v;
    }
    if (threadIdx.x == 0) {
      bA[((int64_t)m * C + t) * 2] = beta;
      bA[((int64_t)m * C + t) * 2 + 1] = a;
    }
    __syncthreads();
  }
}

atlasmem_status launch_ptr_coeffs(const float* theta, const float* eta, const float* alpha, const float* gamma,
                                  int64_t ld, const float* ghist, int M, int64_t s0, int C, int c, float* bA,
                                  float* Om, hipStream_t st) {
  if (M == 0) return ATLASMEM_OK;
  if (c > PTR_MAXC) {
    const size_t lds = ((size_t)6 * C + C + c - 1) * sizeof(float);
    hipLaunchKernelGGL(ptr_coeff_seq_kernel, dim3(M), dim3(256), lds, st, theta, eta, alpha, gamma, ld, ghist, s0, C,
                       c, bA, Om);
  } else {
    const size_t lds = (size_t)3 * C * sizeof(float);
    hipLaunchKernelGGL(ptr_coeff_kernel, dim3(M), dim3(256), lds, st, theta, eta, alpha, gamma, ld, ghist, s0, C, c,
                       bA, Om);
  }
  AM_LAUNCH_CHECK();
  return ATLASMEM_OK;
}

// Window history: after a call of T tokens, keep the last c - 1 (key, value, gamma) rows of
// (old history ++ this call), oldest first.  Rows that do not exist (fewer than c - 1 tokens
// seen since the sequence start) keep gamma = 0 and zero vectors.
__global__ void history_kernel(const void* __restrict__ K, const void* __restrict__ V,
                               const float* __restrict__ gamma, int in_bf16, int M, int64_t T, int64_t ld, int c,
                               int dk, int dv,
                               const float* __restrict__ hk, const float* __restrict__ hv,
                               const float* __restrict__ hg, float* __restrict__ nk, float* __restrict__ nv,
                               float* __restrict__ ng) {
  const int H = c - 1;
  const int width = dk + dv + 1;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)M * H * width) return;
  const int e = (int)(idx % width);
  const int hrow = (int)((idx / width) % H);
  const int m = (int)(idx / ((int64_t)width * H));
  const int64_t tau = T - H + hrow;
  if (e < dk) {
    float x = (tau >= 0) ? load_in(K, ((int64_t)m * ld + tau) * dk + e, in_bf16)
                         : hk[((int64_t)m * H + hrow + T) * dk + e];
    nk[((int64_t)m * H + hrow) * dk + e] = x;
  } else if (e < dk + dv) {
    const int ev = e - dk;
    float x = (tau >= 0) ? load_in(V, ((int64_t)m * ld + tau) * dv + ev, in_bf16)
                         : hv[((int64_t)m * H + hrow + T) * dv + ev];
    nv[((int64_t)m * H + hrow) * dv + ev] = x;
  } else {
    float x = (tau >= 0) ? gamma[(int64_t)m * ld + tau] : hg[(int64_t)m * H + hrow + T];
    ng[(int64_t)m * H + hrow] = x;
  }
}

atlasmem_status launch_history_update(const Handle* h, const void* K, const void* V, const float* gamma, int64_t T,
                                      int64_t ld, hipStream_t st) {
  const Dims& d = h->d;
  if (d.c <= 1 || T == 0) return ATLASMEM_OK;
  const int64_t total = (int64_t)d.M * (d.c - 1) * (d.dk + d.dv + 1);
  const int src = h->hcur, dst = 1 - h->hcur;
  hipLaunchKernelGGL(history_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st, K, V, gamma, d.in_bf16,
                     d.M, T, ld, d.c, d.dk, d.dv, h->hk[src], h->hv[src], h->hg[src], h->hk[dst], h->hv[dst],
                     h->hg[dst]);
  AM_LAUNCH_CHECK();
  return ATLASMEM_OK;
}

// Stand-alone feature map: rows of width d -> C(d+2, 2) fp32 features.  The map is bound by the
// output bytes (C(d+2, 2) / (d / 2) times the input), so a block writes the contiguous feature
// rows of kPolyRows input rows as one stream of 16-byte stores: each store's four features are
// looked up in an LDS table of (i, j) index pairs built once per block (constant: both 0xFFFF,
// linear x_i: j = 0xFFFF, quadratic x_i x_j / 2: both set).  For widths whose table does not fit
// in LDS (TAB = false) the pair is recomputed per feature.
constexpr int kPolyRows = 32;  // a multiple of 4: each block's output starts 16-byte aligned
template <bool TAB>
__global__ void __launch_bounds__(256) poly_kernel(const void* __restrict__ X, int in_bf16, int64_t n, int d,
                                                   float* __restrict__ F) {
  extern __shared__ float xs[];  // [kPolyRows][d] inputs, then the pair table [nf]
  const int nf = poly_count(d);
  uint32_t* tab = (uint32_t*)(xs + kPolyRows * d);
  const int64_t r0 = (int64_t)blockIdx.x * kPolyRows;
  const int nr = (int)((n - r0) < kPolyRows ? (n - r0) : kPolyRows);
  for (int e = threadIdx.x; e < nr * d; e += blockDim.x) xs[e] = load_in(X, r0 * d + e, in_bf16);
  auto code_of = [&](int f) -> uint32_t {
    if (f == 0) return 0xFFFFFFFFu;
    if (f <= d) return 0xFFFF0000u | (uint32_t)(f - 1);
    int i, j;
    pair_of(f - 1 - d, d, i, j);
    return ((uint32_t)j << 16) | (uint32_t)i;
  };
  if (TAB)
    for (int f = threadIdx.x; f < nf; f += blockDim.x) tab[f] = code_of(f);
  __syncthreads();
  auto feature = [&](int e) -> float {  // element e of the block's contiguous output
    const int r = e / nf, f = e - r * nf;
    const uint32_t code = TAB ? tab[f] : code_of(f);
    const uint32_t i = code & 0xFFFFu, j = code >> 16;
    const float* x = xs + r * d;
    if (i == 0xFFFFu) return 1.0f;
    if (j == 0xFFFFu) return x[i];
    return 0.5f * (x[i] * x[j]);
  };
  float* out = F + r0 * nf;
  const int total = nr * nf;
  const int n4 = ((uintptr_t)out & 15) ? 0 : total >> 2;  // scalar stores for a misaligned F
  for (int e4 = threadIdx.x; e4 < n4; e4 += blockDim.x) {
    const int e = 4 * e4;
    *(float4*)(out + e) = float4{feature(e), feature(e + 1), feature(e + 2), feature(e + 3)};
  }
  for (int e = 4 * n4 + threadIdx.x; e < total; e += blockDim.x) out[e] = feature(e);
}

atlasmem_status launch_poly(const void* X, int in_bf16, int64_t n, int d, float* F, hipStream_t st) {
  if (n == 0) return ATLASMEM_OK;
  const int64_t blocks = (n + kPolyRows - 1) / kPolyRows;
  const size_t lds_x = (size_t)kPolyRows * d * sizeof(float);
  const size_t lds_t = lds_x + (size_t)(1 + d + (d * (d + 1)) / 2) * sizeof(uint32_t);
  const bool tab = lds_t <= 64 * 1024;
  const size_t lds = tab ? lds_t : lds_x;
  const void* fn = tab ? (const void*)poly_kernel<true> : (const void*)poly_kernel<false>;
  if (lds > 64 * 1024 && hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess)
    return ATLASMEM_E_DEVICE;
  if (tab)
    hipLaunchKernelGGL(poly_kernel<true>, dim3((unsigned)blocks), dim3(256), lds, st, X, in_bf16, n, d, F);
  else
    hipLaunchKernelGGL(poly_kernel<false>, dim3((unsigned)blocks), dim3(256), lds, st, X, in_bf16, n, d, F);
  AM_LAUNCH_CHECK();
  return ATLASMEM_OK;
}

}  // namespace am
