// Linear memory M_W(x) = W x: the exact recurrence in fp32, one wave64 per memory.
//
// The gradient of ||W x - v||^2 is 2 (W x - v) x^T (Atlas-Torch README, "How the memory
// works": the delta rule).  Lane r owns row r of W (and of the momentum S and of the
// chunk-start copy W_start) in registers, so a step needs no cross-lane traffic: the
// prediction error of row r is e_r = 2 (W_start[r] . x - v_r), the step's gradient row is
// sum over the window of gamma_i e_i[r] x_i, and the momentum / forgetting update of
// titans-pytorch-mlx README Eq. 13-14 is applied in place.  Tokens are staged 64 at a time
// into an LDS ring that also keeps the c - 1 previous tokens of the Omega window (ATLAS
// summary, section 3.2), whose errors are re-taken at each chunk's start weights.
#include "common.h"
#include "internal.h"

namespace am {

constexpr int kRing = 128;   // ring of staged tokens (power of two >= 64 + window history)
constexpr int kBlockTok = 64;
constexpr int kMaxWindow = 8;

struct LinArgs {
  const void* K;
  const void* Q;
  const void* V;
  int in_bf16;
  const float* theta;
  const float* eta;
  const float* alpha;
  const float* gamma;
  int per_chunk;
  int64_t T;         // tokens
  int64_t ld, ldg;   // per memory: token stride of the row arrays, stride of per-chunk gates
  int C, c, dk, din, dv, poly;
  const float* Win;
  const float* Sin;
  float* Wout;
  float* Sout;
  int64_t P;
  const float* hk;
  const float* hv;
  const float* hg;
  void* Y;
  int out_bf16;
  int ptr;           // per-token retrieval: y_t from the state right after token t's update
  int* flag;
};

// phi(x)[f] of a raw row x (width dk) read from global memory.
__device__ __forceinline__ float feature_of(const void* base, int64_t row_off, int in_bf16, int f, int dk, int poly,
                                            const float* frow = nullptr) {
  auto xat = [&](int i) { return frow ? frow[i] : load_in(base, row_off + i, in_bf16); };
  if (poly == 1) return xat(f);
  if (f == 0) return 1.0f;
  if (f <= dk) return xat(f - 1);
  int i, j;
  pair_of(f - 1 - dk, dk, i, j);
  return 0.5f * (xat(i) * xat(j));
}

template <int D>
__device__ __forceinline__ float dot_row(const float (&w)[D], const float* x) {
  float acc = 0.0f;
#pragma unroll
  for (int l = 0; l < D; l += 4) {
    const f32x4 xv = *(const f32x4*)(x + l);
    acc = fmaf(w[l], xv[0], acc);
    acc = fmaf(w[l + 1], xv[1], acc);
    acc = fmaf(w[l + 2], xv[2], acc);
    acc = fmaf(w[l + 3], xv[3], acc);
  }
  return acc;
}

template <int D>
__global__ void __launch_bounds__(64) lin_kernel(LinArgs a) {
  extern __shared__ __attribute__((aligned(16))) float sm[];
  float* Xr = sm;                       // [kRing][D]   phi(k) rows
  float* Vr = Xr + kRing * D;           // [kRing][D]   values
  float* Gr = Vr + kRing * D;           // [kRing]      window weights
  float* Qb = Gr + kRing;               // [kBlockTok][D] phi(q) rows
  float* Th = Qb + kBlockTok * D;       // [kBlockTok] gates of the staged block
  float* Et = Th + kBlockTok;
  float* Al = Et + kBlockTok;

  const int m = blockIdx.x;
  const int r = threadIdx.x;
  const bool own = r < a.dv;
  const int H = a.c - 1;

  float W[D], Wb[D], S[D], G[D], E[kMaxWindow];
#pragma unroll
  for (int l = 0; l < D; ++l) {
    const bool in = own && l < a.din;
    W[l] = in ? a.Win[(int64_t)m * a.P + (int64_t)r * a.din + l] : 0.0f;
    S[l] = in ? a.Sin[(int64_t)m * a.P + (int64_t)r * a.din + l] : 0.0f;
    Wb[l] = W[l];
    G[l] = 0.0f;
  }
#pragma unroll
  for (int u = 0; u < kMaxWindow; ++u) E[u] = 0.0f;

  // window history rows (tokens -H .. -1)
  for (int hrow = 0; hrow < H; ++hrow) {
    const int slot = (hrow - H) & (kRing - 1);
    const float* hkr = a.hk + ((int64_t)m * H + hrow) * a.dk;
    for (int f = r; f < D; f += 64)
      Xr[slot * D + f] = f < a.din ? feature_of(nullptr, 0, 0, f, a.dk, a.poly, hkr) : 0.0f;
    for (int f = r; f < D; f += 64) Vr[slot * D + f] = f < a.dv ? a.hv[((int64_t)m * H + hrow) * a.dv + f] : 0.0f;
    if (r == 0) Gr[slot] = a.hg[(int64_t)m * H + hrow];
  }

  for (int64_t b0 = 0; b0 < a.T; b0 += kBlockTok) {
    const int nb = (int)((a.T - b0) < kBlockTok ? (a.T - b0) : kBlockTok);
    __syncthreads();
    for (int idx = r; idx < nb * D; idx += 64) {
      const int j = idx / D, f = idx % D;
      const int64_t tau = b0 + j;
      const int slot = (int)(tau & (kRing - 1));
      const int64_t krow = ((int64_t)m * a.ld + tau) * a.dk;
      Xr[slot * D + f] = f < a.din ? feature_of(a.K, krow, a.in_bf16, f, a.dk, a.poly) : 0.0f;
      // queries are read only when Y is asked for (Q may be null otherwise)
      Qb[j * D + f] = (a.Y && f < a.din) ? feature_of(a.Q, krow, a.in_bf16, f, a.dk, a.poly) : 0.0f;
      Vr[slot * D + f] = f < a.dv ? load_in(a.V, ((int64_t)m * a.ld + tau) * a.dv + f, a.in_bf16) : 0.0f;
    }
    for (int j = r; j < nb; j += 64) {
      const int64_t tau = b0 + j;
      Gr[tau & (kRing - 1)] = a.c > 1 ? a.gamma[(int64_t)m * a.ld + tau] : 1.0f;
      if (!a.per_chunk) {
        Th[j] = a.theta[(int64_t)m * a.ld + tau];
        Et[j] = a.eta[(int64_t)m * a.ld + tau];
        Al[j] = a.alpha[(int64_t)m * a.ld + tau];
      }
    }
    __syncthreads();

    for (int j = 0; j < nb; ++j) {
      const int64_t t = b0 + j;
      if (t % a.C == 0) {  // chunk start: freeze the weights, re-take the history errors
#pragma unroll
        for (int l = 0; l < D; ++l) {
          Wb[l] = W[l];
          G[l] = 0.0f;
        }
#pragma unroll
        for (int u = 1; u < kMaxWindow; ++u) {
          if (u <= H) {
            const int slot = (int)((t - u) & (kRing - 1));
            E[kMaxWindow - u] = 2.0f * (dot_row<D>(Wb, Xr + slot * D) - Vr[slot * D + (own ? r : 0)]);
          }
        }
      }
      const int slot = (int)(t & (kRing - 1));
      if (own && a.Y && !a.ptr) {
        const float y = dot_row<D>(Wb, Qb + j * D);
        const int64_t yo = ((int64_t)m * a.ld + t) * a.dv + r;
        if (a.out_bf16) ((uint16_t*)a.Y)[yo] = (uint16_t)bf16_bits(y);
        else ((float*)a.Y)[yo] = y;
      }
      const float e = 2.0f * (dot_row<D>(Wb, Xr + slot * D) - Vr[slot * D + (own ? r : 0)]);
#pragma unroll
      for (int u = 0; u < kMaxWindow - 1; ++u) E[u] = E[u + 1];
      E[kMaxWindow - 1] = e;
      if (!a.per_chunk) {
        float coef[kMaxWindow];
        int sl[kMaxWindow];
#pragma unroll
        for (int u = 0; u < kMaxWindow; ++u) {
          sl[u] = (int)((t - u) & (kRing - 1));
          coef[u] = (u < a.c) ? Gr[sl[u]] * E[kMaxWindow - 1 - u] : 0.0f;
        }
        const float th = Th[j], et = Et[j], om = 1.0f - Al[j];
#pragma unroll
        for (int l = 0; l < D; ++l) {
          float g = 0.0f;
#pragma unroll
          for (int u = 0; u < kMaxWindow; ++u)
            if (u < a.c) g = fmaf(coef[u], Xr[sl[u] * D + l], g);
          S[l] = et * S[l] - th * g;
          W[l] = om * W[l] + S[l];
        }
        if (own && a.Y && a.ptr) {  // the state right after this token's update
          const float y = dot_row<D>(W, Qb + j * D);
          const int64_t yo = ((int64_t)m * a.ld + t) * a.dv + r;
          if (a.out_bf16) ((uint16_t*)a.Y)[yo] = (uint16_t)bf16_bits(y);
          else ((float*)a.Y)[yo] = y;
        }
      } else {
#pragma unroll
        for (int l = 0; l < D; ++l) G[l] = fmaf(e, Xr[slot * D + l], G[l]);
        if ((t + 1) % a.C == 0) {
          const int64_t k = t / a.C;
          const int64_t go = (int64_t)m * a.ldg + k;
          const float th = a.theta[go], et = a.eta[go], om = 1.0f - a.alpha[go];
#pragma unroll
          for (int l = 0; l < D; ++l) {
            S[l] = et * S[l] - th * G[l];
            W[l] = om * W[l] + S[l];
          }
        }
      }
    }
  }
  bool bad = false;
  if (own) {
#pragma unroll
    for (int l = 0; l < D; ++l) {
      if (l < a.din) {
        a.Wout[(int64_t)m * a.P + (int64_t)r * a.din + l] = W[l];
        a.Sout[(int64_t)m * a.P + (int64_t)r * a.din + l] = S[l];
        bad |= !(isfinite(W[l]) && isfinite(S[l]));
      }
    }
  }
  if (bad) a.flag[0] = 1;
}

template <int D>
static size_t lin_smem() {
  return sizeof(float) * (2 * kRing * D + kRing + kBlockTok * D + 3 * kBlockTok);
}

template <int D>
static atlasmem_status lin_launch(const LinArgs& a, int M, hipStream_t st) {
  const size_t sm = lin_smem<D>();
  if (sm > 64 * 1024) {
    if (hipFuncSetAttribute((const void*)lin_kernel<D>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)sm) !=
        hipSuccess)
      return ATLASMEM_E_DEVICE;
  }
  hipLaunchKernelGGL(lin_kernel<D>, dim3(M), dim3(64), sm, st, a);
  AM_LAUNCH_CHECK();
  return ATLASMEM_OK;
}

atlasmem_status launch_linear_update(Handle* h, const Dims& d, const void* K, const void* Q, const void* V,
                                     const float* theta, const float* eta, const float* alpha, const float* gamma,
                                     const Span& sp, void* Y, hipStream_t st) {
  LinArgs a;
  a.K = K;
  a.Q = Q;
  a.V = V;
  a.in_bf16 = d.in_bf16;
  a.theta = theta;
  a.eta = eta;
  a.alpha = alpha;
  a.gamma = gamma;
  a.per_chunk = d.gate_mode == ATLASMEM_PER_CHUNK;
  a.T = sp.T;
  a.ld = sp.ld;
  a.ldg = sp.ldg;
  a.C = d.C;
  a.c = d.c;
  a.dk = d.dk;
  a.din = d.din;
  a.dv = d.dv;
  a.poly = d.poly;
  a.Win = h->W[h->cur];
  a.Sin = h->S[h->cur];
  a.Wout = h->W[1 - h->cur];
  a.Sout = h->S[1 - h->cur];
  a.P = d.P;
  a.hk = h->hk[h->hcur];
  a.hv = h->hv[h->hcur];
  a.hg = h->hg[h->hcur];
  a.Y = Y;
  a.out_bf16 = d.out_bf16;
  a.ptr = d.ptr;
  a.flag = h->flag;
  const int D = d.din > d.dv ? d.din : d.dv;
  atlasmem_status s;
  if (D <= 16) s = lin_launch<16>(a, d.M, st);
  else if (D <= 32) s = lin_launch<32>(a, d.M, st);
  else s = lin_launch<64>(a, d.M, st);
  if (s == ATLASMEM_OK) h->cur = 1 - h->cur;
  return s;
}

// Retrieval with the current weights: one wave per (memory, block of 64 tokens), lane r
// owns row r of W.
__global__ void __launch_bounds__(64) lin_retrieve_kernel(const float* __restrict__ W, int64_t P, const void* Q,
                                                          int in_bf16, int64_t T, int64_t ld, int dk, int din,
                                                          int dv, int poly, void* Y, int out_bf16) {
  extern __shared__ float qs[];  // [din]
  const int m = blockIdx.y;
  const int64_t t0 = (int64_t)blockIdx.x * 64;
  const int r = threadIdx.x;
  for (int64_t t = t0; t < t0 + 64 && t < T; ++t) {
    const int64_t qrow = ((int64_t)m * ld + t) * dk;
    __syncthreads();
    for (int f = r; f < din; f += 64) qs[f] = feature_of(Q, qrow, in_bf16, f, dk, poly);
    __syncthreads();
    if (r < dv) {
      const float* w = W + (int64_t)m * P + (int64_t)r * din;
      float acc = 0.0f;
      for (int l = 0; l < din; ++l) acc = fmaf(w[l], qs[l], acc);
      const int64_t yo = ((int64_t)m * ld + t) * dv + r;
      if (out_bf16) ((uint16_t*)Y)[yo] = (uint16_t)bf16_bits(acc);
      else ((float*)Y)[yo] = acc;
    }
  }
}

atlasmem_status launch_linear_retrieve(Handle* h, const void* Q, int64_t T, int64_t ld, void* Y, hipStream_t st) {
  const Dims& d = h->d;
  if (T == 0) return ATLASMEM_OK;
  dim3 grid((unsigned)((T + 63) / 64), d.M);
  hipLaunchKernelGGL(lin_retrieve_kernel, grid, dim3(64), d.din * sizeof(float), st, h->W[h->cur], d.P, Q, d.in_bf16,
                     T, ld, d.dk, d.din, d.dv, d.poly, Y, d.out_bf16);
  AM_LAUNCH_CHECK();
  return ATLASMEM_OK;
}

}  // namespace am
