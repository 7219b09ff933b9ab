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
constexpr int kFeatRows = 8;
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
  // a block's nr * F <= 32 * 2^20 elements fit 32-bit indices; the row and feature of e0 advance
  // by a fixed step each iteration, so no division runs inside the loop
  const int F = (int)a.F;
  const int total = nr * F;
  float* base = a.out + r0 * a.F;
  const bool vec = ((r0 * a.F) & 3) == 0 && (((uintptr_t)a.out) & 15) == 0;
  const int step = blockDim.x * 4;
  const int step_r = step / F, step_f = step - step_r * F;
  int row_e = (threadIdx.x * 4) / F, f_e = threadIdx.x * 4 - row_e * F;
  for (int e0 = threadIdx.x * 4; e0 < total; e0 += step) {
    int r = row_e, f = f_e;
    row_e += step_r;
    f_e += step_f;
    if (f_e >= F) {
      f_e -= F;
      ++row_e;
    }
    float v[4];
    if (TAB) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if (f == F) {
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
          if (f == F) {  // the next row starts
            ++r;
            f = 0;
            m = Mono{0, 0, 0, 0};
          }
          v[u] = mono_value(m, xr + r * a.d, a.c);
          ++f;
          if (f < F) m = mono_next(m, a.d);
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

// ---------------------------------------------------------------------------- projection
//
// phi_c(X) P^T on the matrix cores, the features formed where they are used: a workgroup takes
// 128 input rows (staged in LDS as fp32, with the monomial table of every feature) and walks the
// features in blocks of 64; each block's P columns are split into bf16 hi / lo in LDS once for the
// workgroup (the next block's values loaded while the current one is used), and each wave forms
// its 32 rows' features of a k-step from the staged rows (one table read and at most three row
// reads per feature) and multiplies them on the matrix cores (v_mfma_f32_32x32x16_bf16, hi*hi +
// hi*lo + lo*hi, fp32 accumulation) into its 32 x d_out outputs.
namespace fpj {
constexpr int NT = 256;     // four waves
constexpr int RT = 1;       // row tiles per wave: wave w takes rows 32w + 128t .. +31 (t < RT);
                            // two tiles per wave measured slower (more registers, fewer workgroups)
constexpr int ROWS = 128 * RT;  // input rows per workgroup
constexpr int KB = 64;      // features per block
constexpr int LP = KB + 8;  // P block row stride (uint16): 16-byte reads along k land on distinct banks
constexpr int kMaxD = 64, kMaxOut = 128, kMaxF = 8192;

struct Args {
  const void* X;
  int in_bf16;
  int64_t n;
  int d, F, d_out;
  float c[4];
  const float* P;  // [d_out][F]
  float* out;      // [n][d_out]
};

__host__ __device__ constexpr int fpad(int F) { return (F + KB - 1) / KB * KB; }
inline size_t lds_bytes(int d, int F, int nc) {
  return (size_t)ROWS * (d + 1) * 4 + (size_t)fpad(F) * 4 + (size_t)nc * 32 * LP * 2 * 2;
}

template <int NC>
__global__ void __launch_bounds__(NT) feat_proj_kernel(Args a) {
  extern __shared__ __attribute__((aligned(16))) float fsm[];
  const int xs = a.d + 1;  // row stride: lanes of consecutive rows on distinct banks
  float* xr = fsm;
  uint32_t* tab = (uint32_t*)(xr + ROWS * xs);
  const int FP = fpad(a.F);
  uint16_t* pbh = (uint16_t*)(tab + FP);
  uint16_t* pbl = pbh + NC * 32 * LP;
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, l32 = lane & 31, hf = lane >> 5;
  const int64_t r0 = (int64_t)blockIdx.x * ROWS;
  const int nr = (int)((a.n - r0) < ROWS ? (a.n - r0) : ROWS);
  for (int e = tid; e < ROWS * a.d; e += NT) {
    const int r = e / a.d, i = e - r * a.d;
    xr[r * xs + i] = r < nr ? load_in(a.X, (r0 + r) * a.d + i, a.in_bf16) : 0.0f;
  }
  {  // the monomial table: each thread decodes one run of features and steps through it
    const int per = (FP + NT - 1) / NT;
    const int f0 = tid * per;
    if (f0 < a.F) {
      Mono m = mono_of(f0, a.d);
      for (int u = 0; u < per && f0 + u < a.F; ++u) {
        tab[f0 + u] = mono_code(m);
        if (f0 + u + 1 < a.F) m = mono_next(m, a.d);
      }
    }
  }
  f32x16 acc[RT][NC];
#pragma unroll
  for (int t = 0; t < RT; ++t)
#pragma unroll
    for (int ct = 0; ct < NC; ++ct)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[t][ct][r] = 0.0f;
  // P block: rows o < 32 NC, features fb .. fb + 63; thread element i is e = tid + 256 i.  The next
  // block's values are loaded while the current block's products run.
  constexpr int PE = NC * 32 * KB / NT;
  float pv[PE];
  auto load_p = [&](int fb) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < PE; ++i) {
      const int e = tid + NT * i, o = e / KB, f = fb + (e - o * KB);
      pv[i] = (o < a.d_out && f < a.F) ? a.P[(int64_t)o * a.F + f] : 0.0f;
    }
  };
  load_p(0);
  for (int fb = 0; fb < FP; fb += KB) {
    __syncthreads();  // the staging above, or the previous block's reads of the P block
    // the block split into bf16 hi / lo ([o][k])
#pragma unroll
    for (int i = 0; i < PE; ++i) {
      const int e = tid + NT * i, o = e / KB, k = e - o * KB;
      uint32_t h, l;
      split_bf16(pv[i], h, l);
      pbh[o * LP + k] = (uint16_t)h;
      pbl[o * LP + k] = (uint16_t)l;
    }
    if (fb + KB < FP) load_p(fb + KB);
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < KB / 16; ++ks) {
      const int kk = 16 * ks + 8 * hf;  // this lane's 8 features of the k-step (both operands)
      u32x4 ah[RT], al[RT];
#pragma unroll
      for (int t = 0; t < RT; ++t) {
        const float* x = xr + (32 * w + 128 * t + l32) * xs;  // this lane's row of tile t
        float v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int f = fb + kk + u;
          v[u] = f < a.F ? code_value(tab[f], x, a.c) : 0.0f;
        }
        pack8(v, ah[t], al[t]);
      }
#pragma unroll
      for (int ct = 0; ct < NC; ++ct) {
        const int ob = (32 * ct + l32) * LP + kk;
        const u32x4 bh = *(const u32x4*)(pbh + ob), bl = *(const u32x4*)(pbl + ob);
#pragma unroll
        for (int t = 0; t < RT; ++t) {
          acc[t][ct] = mfma32(ah[t], bh, acc[t][ct]);
          acc[t][ct] = mfma32(ah[t], bl, acc[t][ct]);
          acc[t][ct] = mfma32(al[t], bh, acc[t][ct]);
        }
      }
    }
  }
  // register r of tile t: row 32w + 128t + 8(r/4) + 4hf + r%4, column 32ct + l32
#pragma unroll
  for (int t = 0; t < RT; ++t)
#pragma unroll
    for (int ct = 0; ct < NC; ++ct) {
      const int col = 32 * ct + l32;
      if (col >= a.d_out) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = 32 * w + 128 * t + 8 * (r >> 2) + 4 * hf + (r & 3);
        if (row < nr) a.out[(r0 + row) * a.d_out + col] = acc[t][ct][r];
      }
    }
}
}  // namespace fpj

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
  if (d <= fpj::kMaxD && F <= fpj::kMaxF && d_out <= fpj::kMaxOut) {
    fpj::Args a;
    a.X = X;
    a.in_bf16 = in_bf16;
    a.n = n;
    a.d = d;
    a.F = (int)F;
    a.d_out = d_out;
    for (int k = 0; k < 4; ++k) a.c[k] = c4[k];
    a.P = P;
    a.out = out;
    const int nc = (d_out + 31) / 32;
    const size_t lds = fpj::lds_bytes(d, (int)F, nc);
    const int64_t blocks = (n + fpj::ROWS - 1) / fpj::ROWS;
    if (blocks > INT32_MAX) return ATLASMEM_E_SHAPE;
    void (*kern)(fpj::Args) = nc == 1 ? fpj::feat_proj_kernel<1>
                              : nc == 2 ? fpj::feat_proj_kernel<2>
                              : nc == 3 ? fpj::feat_proj_kernel<3>
                                        : fpj::feat_proj_kernel<4>;
    if (hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess)
      return ATLASMEM_E_DEVICE;
    hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(fpj::NT), lds, st, a);
    AM_LAUNCH_CHECK();
    return ATLASMEM_OK;
  }
  // wider rows, more features or outputs: the GEMM engine with the features formed in its loader
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
