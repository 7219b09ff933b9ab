// Feature map stage: every monomial of degree 0..p (p <= 3) of a row, degree-major and in
// combinations_with_replacement order inside a degree, the degree-k monomials multiplied by a
// per-degree coefficient c_k (default 1/k!, the exponential kernel's Taylor coefficients), and
// optionally projected back, phi_c(x) P^T (Atlas-Torch README, Atlas Extensions table,
// "Polynomial Features": exact monomial expansion, learnable coefficients initialised to 1/d!,
// optional project_back; ATLAS summary, sections 3.1 and 4.3 (Dot: exponential features with the
// Omega rule)).
//
// Feature index -> monomial: f = 0 is the constant, 1..d the linear terms, then the pairs
// (i <= j), then the triples (i <= j <= k).  The triples with first index below i number
// C(d+2, 3) - C(d-i+2, 3) (hockey-stick identity), so i is found by bisection and the rest is a
// pair index inside the (d - i)-wide upper triangle.  Consecutive features are reached by
// stepping the indices, so a decode is paid once per run of features.
#include "common.h"
#include "gemm.h"
#include "internal.h"

namespace am {

__device__ __forceinline__ int64_t choose3(int64_t m) { return m < 3 ? 0 : m * (m - 1) * (m - 2) / 6; }
__device__ __forceinline__ int64_t choose2(int64_t m) { return m < 2 ? 0 : m * (m - 1) / 2; }

// One monomial: degree and indices (unused ones are 0).
struct Mono {
  int deg, i, j, k;
};

__device__ __forceinline__ Mono mono_of(int64_t f, int d) {
  Mono m{0, 0, 0, 0};
  if (f == 0) return m;
  f -= 1;
  if (f < d) return Mono{1, (int)f, 0, 0};
  f -= d;
  const int64_t npair = choose2(d + 1);
  if (f < npair) {
    int i, j;
    pair_of((int)f, d, i, j);
    return Mono{2, i, j, 0};
  }
  f -= npair;
  // first index: the largest i with start3(i) <= f, start3(i) = C(d+2,3) - C(d-i+2,3)
  const int64_t total = choose3(d + 2);
  int lo = 0, hi = d - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (total - choose3(d - mid + 2) <= f) lo = mid;
    else hi = mid - 1;
  }
  const int i = lo;
  const int64_t u = f - (total - choose3(d - i + 2));
  int jj, kk;
  pair_of((int)u, d - i, jj, kk);
  return Mono{3, i, i + jj, i + kk};
}

// The monomial after m in the enumeration order.
__device__ __forceinline__ Mono mono_next(Mono m, int d) {
  switch (m.deg) {
    case 0: return Mono{1, 0, 0, 0};
    case 1: return (m.i + 1 < d) ? Mono{1, m.i + 1, 0, 0} : Mono{2, 0, 0, 0};
    case 2:
      if (m.j + 1 < d) return Mono{2, m.i, m.j + 1, 0};
      if (m.i + 1 < d) return Mono{2, m.i + 1, m.i + 1, 0};
      return Mono{3, 0, 0, 0};
    default:
      if (m.k + 1 < d) return Mono{3, m.i, m.j, m.k + 1};
      if (m.j + 1 < d) return Mono{3, m.i, m.j + 1, m.j + 1};
      return Mono{3, m.i + 1, m.i + 1, m.i + 1};  // past the last triple only beyond the row
  }
}

__device__ __forceinline__ float mono_value(const Mono& m, const float* x, const float* c) {
  switch (m.deg) {
    case 0: return c[0];
    case 1: return c[1] * x[m.i];
    case 2: return c[2] * (x[m.i] * x[m.j]);
    default: return c[3] * (x[m.i] * x[m.j] * x[m.k]);
  }
}

struct FeatureArgs {
  const void* X;
  int in_bf16;
  int64_t n;
  int d, degree;
  int64_t F;  // features per row
  float c[4];
  float* out;
};

// A monomial packed into 32 bits: degree in bits 30-31, indices in three 10-bit fields (d <= 1024).
__device__ __forceinline__ uint32_t mono_code(const Mono& m) {
  return ((uint32_t)m.deg << 30) | ((uint32_t)m.k << 20) | ((uint32_t)m.j << 10) | (uint32_t)m.i;
}
__device__ __forceinline__ float code_value(uint32_t code, const float* x, const float* c) {
  const int deg = (int)(code >> 30);
  const int i = (int)(code & 1023u), j = (int)((code >> 10) & 1023u), k = (int)((code >> 20) & 1023u);
  switch (deg) {
    case 0: return c[0];
    case 1: return c[1] * x[i];
    case 2: return c[2] * (x[i] * x[j]);
    default: return c[3] * (x[i] * x[j] * x[k]);
  }
}

// kFeatRows input rows per block in LDS, then the monomial table (TAB, when it fits) so that each
// feature costs one table read; the block streams the rows' contiguous features out as 16-byte
// stores.  Without the table a thread decodes the monomial of each run of four features.
constexpr int kFeatRows = 32;
constexpr int kFeatTabMax = 12288;  // table entries (48 KB)
template <bool TAB>
__global__ void __launch_bounds__(256) feature_kernel(FeatureArgs a) {
  extern __shared__ float xr[];  // [kFeatRows][d], then the table
  uint32_t* tab = (uint32_t*)(xr + kFeatRows * a.d);
  const int64_t r0 = (int64_t)blockIdx.x * kFeatRows;
  const int nr = (int)((a.n - r0) < kFeatRows ? (a.n - r0) : kFeatRows);
  for (int e = threadIdx.x; e < nr * a.d; e += blockDim.x) xr[e] = load_in(a.X, r0 * a.d + e, a.in_bf16);
  if (TAB) {
    const int per = (int)((a.F + blockDim.x - 1) / blockDim.x);
    const int64_t f0 = (int64_t)threadIdx.x * per;
    if (f0 < a.F) {  // each thread decodes one run and steps through it
      Mono m = mono_of(f0, a.d);
      for (int u = 0; u < per && f0 + u < a.F; ++u) {
        tab[f0 + u] = mono_code(m);
        if (f0 + u + 1 < a.F) m = mono_next(m, a.d);
      }
    }
  }
  __syncthreads();
  const int64_t total = (int64_t)nr * a.F;
  float* base = a.out + r0 * a.F;
  const bool vec = ((r0 * a.F) & 3) == 0 && (((uintptr_t)a.out) & 15) == 0;
  for (int64_t e0 = (int64_t)threadIdx.x * 4; e0 < total; e0 += (int64_t)blockDim.x * 4) {
    int64_t r = e0 / a.F;
    int64_t f = e0 - r * a.F;
    float v[4];
    if (TAB) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if (f == a.F) {
          ++r;
          f = 0;
        }
        v[u] = (e0 + u < total) ? code_value(tab[f], xr + r * a.d, a.c) : 0.0f;
        ++f;
      }
    } else {
      Mono m = mono_of(f, a.d);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if (e0 + u < total) {
          if (f == a.F) {  // the next row starts
            ++r;
            f = 0;
            m = Mono{0, 0, 0, 0};
          }
          v[u] = mono_value(m, xr + r * a.d, a.c);
          ++f;
          if (f < a.F) m = mono_next(m, a.d);
        } else {
          v[u] = 0.0f;
        }
      }
    }
    if (vec && e0 + 3 < total) {
      *(float4*)(base + e0) = float4{v[0], v[1], v[2], v[3]};
    } else {
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (e0 + u < total) base[e0 + u] = v[u];
    }
  }
}

// A operand phi_c(X) for the projection product: row = input row, k = feature.
struct FeatMapA {
  const void* X;
  int in_bf16;
  int64_t n, F;
  int d;
  float c[4];
  __device__ __forceinline__ void load8(int z, int row, int f0, float* v) const {
    (void)z;
    if (row >= n || f0 >= F) {
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = 0.0f;
      return;
    }
    // Consecutive monomials mostly advance only their last index: the coefficient times the
    // other factors is kept and refreshed when they change, so most features cost one load.
    Mono m = mono_of(f0, d);
    const int64_t rb = (int64_t)row * d;
    auto head = [&](const Mono& q) -> float {
      switch (q.deg) {
        case 0: return c[0];
        case 1: return c[1];
        case 2: return c[2] * load_in(X, rb + q.i, in_bf16);
        default: return c[3] * load_in(X, rb + q.i, in_bf16) * load_in(X, rb + q.j, in_bf16);
      }
    };
    float pre = head(m);
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      float x = 0.0f;
      if (f0 + u < F) {
        const int last = m.deg == 3 ? m.k : (m.deg == 2 ? m.j : m.i);
        x = m.deg == 0 ? pre : pre * load_in(X, rb + last, in_bf16);
        if (f0 + u + 1 < F) {
          const Mono nx = mono_next(m, d);
          const bool same_head = nx.deg == m.deg && (m.deg == 1 || (nx.i == m.i && (m.deg == 2 || nx.j == m.j)));
          m = nx;
          if (!same_head) pre = head(m);
        }
      }
      v[u] = x;
    }
  }
};

struct FeatProjStore {
  float* out;
  int ld;
  __device__ __forceinline__ void operator()(int z, int row, int col, float v) const {
    (void)z;
    out[(int64_t)row * ld + col] = v;
  }
};

int64_t feature_count_host(int d, int degree) {
  int64_t c = 1;
  for (int k = 1; k <= degree; ++k) c = c * (d + k) / k;
  return c;
}

atlasmem_status launch_feature_map(const void* X, bool in_bf16, int64_t n, int d, int degree, const float* c4,
                                   const float* P, int d_out, float* out, hipStream_t st) {
  if (n == 0) return ATLASMEM_OK;
  const int64_t F = feature_count_host(d, degree);
  if (!P) {
    FeatureArgs a;
    a.X = X;
    a.in_bf16 = in_bf16;
    a.n = n;
    a.d = d;
    a.degree = degree;
    a.F = F;
    for (int k = 0; k < 4; ++k) a.c[k] = c4[k];
    a.out = out;
    const int64_t blocks = (n + kFeatRows - 1) / kFeatRows;
    if (blocks > INT32_MAX) return ATLASMEM_E_SHAPE;
    const size_t rows_lds = (size_t)kFeatRows * d * sizeof(float);
    if (F <= kFeatTabMax) {
      const size_t lds = rows_lds + (size_t)F * sizeof(uint32_t);
      if (lds > 64 * 1024 && hipFuncSetAttribute((const void*)feature_kernel<true>,
                                                 hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess)
        return ATLASMEM_E_DEVICE;
      hipLaunchKernelGGL(feature_kernel<true>, dim3((unsigned)blocks), dim3(256), lds, st, a);
    } else {
      if (rows_lds > 64 * 1024 && hipFuncSetAttribute((const void*)feature_kernel<false>,
                                                      hipFuncAttributeMaxDynamicSharedMemorySize,
                                                      (int)rows_lds) != hipSuccess)
        return ATLASMEM_E_DEVICE;
      hipLaunchKernelGGL(feature_kernel<false>, dim3((unsigned)blocks), dim3(256), rows_lds, st, a);
    }
    AM_LAUNCH_CHECK();
    return ATLASMEM_OK;
  }
  FeatMapA la;
  la.X = X;
  la.in_bf16 = in_bf16;
  la.n = n;
  la.F = F;
  la.d = d;
  for (int k = 0; k < 4; ++k) la.c[k] = c4[k];
  StridedLoader lb;  // B(k = f, j = o) = P[o][f]
  lb.base = P;
  lb.sz = 0;
  lb.so = F;
  lb.sk = 1;
  lb.zdiv = 1;
  lb.outer_dim = d_out;
  lb.K = (int)F;
  lb.xf = XF_NONE;
  lb.coef0 = lb.coef1 = nullptr;
  lb.cz = 0;
  lb.scale = nullptr;
  lb.gofs = 0;
  lb.cld = 0;
  // rows in blocks of at most 65535 tiles along the grid's y dimension
  const int64_t rows_per_launch = (int64_t)65535 * GT;
  for (int64_t r0 = 0; r0 < n; r0 += rows_per_launch) {
    const int64_t nr = (n - r0) < rows_per_launch ? (n - r0) : rows_per_launch;
    FeatMapA lar = la;
    lar.X = (const char*)X + r0 * d * (in_bf16 ? 2 : 4);
    lar.n = nr;
    FeatProjStore ep{out + r0 * d_out, d_out};
    launch_gemm<false, false>(true, (int)nr, d_out, (int)F, 1, lar, lb, ep, st);
    AM_LAUNCH_CHECK();
  }
  return ATLASMEM_OK;
}

}  // namespace am
