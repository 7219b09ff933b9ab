// Input prologue of the memory update: the causal short convolution of keys, queries and values,
// and the data-dependent gates.
//
// Short convolution: a depthwise 1-D convolution of kernel 4 along the token axis, one filter per
// (head, channel), on keys, queries and values (Atlas-Torch README, Atlas Extensions table,
// "Short Convolution"; titans-pytorch-mlx README, Configuration table, use_conv and
// conv_kernel_size 4).  Tap j multiplies token t - 3 + j; tokens before the start are zero or the
// rows carried from the previous call; the keys and queries may be L2-normalised afterwards.
//
// Gates: each gate is a maximum times a sigmoid of a per-head linear map of the token's input
// vector (titans-pytorch-mlx README, Key Innovations item 4 and the Configuration table's
// memory_lr / memory_momentum / memory_decay "scaled by gate"; titans-torch 0.1.2, "Inner-loop
// update rule"), per token or, for the per-chunk path, of the chunk's mean-pooled input
// (Atlas-Torch README, Bug Fixes table, "no-omega ablation" row: pooled gates).
#include "common.h"
#include "internal.h"

namespace am {

// ------------------------------------------------------------------------ short convolution

constexpr int kConvCh = 8;    // channels per lane (16 bytes of bf16)
constexpr int kConvSeg = 64;  // consecutive tokens per lane

struct ConvArgs {
  const void* X;      // [M, T, d]
  int64_t M, T;
  int d, heads;
  int log_lpr;        // lanes per row = 2^log_lpr >= ceil(d / 8), at most 64
  int64_t nseg;       // token segments per memory
  const float* taps;  // [heads, d, 4]
  const float* bias;  // [heads, d] or null
  const void* hist;   // [M, 3, d] or null
  int l2norm;
  void* out;          // [M, T, d]
};

// One row's 8 channels as loaded: packed bf16 pairs (4 words) or fp32 (8 words).  Loads are
// issued into these raw words and converted only where they are used, so that a whole batch of
// rows is in flight at once.
template <bool IN_BF16>
struct RawRow {
  static constexpr int N = IN_BF16 ? 4 : 8;
  uint32_t w[N];
};

template <bool IN_BF16, bool VEC>
__device__ __forceinline__ void conv_load(const void* base, int64_t off, int c0, int d, RawRow<IN_BF16>& r) {
  if (VEC) {  // d % 8 == 0 and aligned bases: one 16-byte (bf16) or two 16-byte (fp32) loads
    if (IN_BF16) {
      const u32x4 v = *(const u32x4*)((const uint16_t*)base + off + c0);
#pragma unroll
      for (int p = 0; p < 4; ++p) r.w[p] = v[p];
    } else {
      const u32x4 a = *(const u32x4*)((const float*)base + off + c0);
      const u32x4 b = *(const u32x4*)((const float*)base + off + c0 + 4);
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        r.w[p] = a[p];
        r.w[4 + p] = b[p];
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < kConvCh; ++i) {
      const int c = c0 + i < d ? c0 + i : d - 1;  // in-bounds address; the value is masked below
      const uint32_t v = IN_BF16 ? (uint32_t)((const uint16_t*)base)[off + c] : ((const uint32_t*)base)[off + c];
      const uint32_t m = c0 + i < d ? v : 0u;
      if (IN_BF16) r.w[i >> 1] = (i & 1) ? (r.w[i >> 1] | (m << 16)) : m;
      else r.w[i] = m;
    }
  }
}

template <bool IN_BF16>
__device__ __forceinline__ void conv_unpack(const RawRow<IN_BF16>& r, float (&v)[kConvCh]) {
#pragma unroll
  for (int i = 0; i < kConvCh; ++i)
    v[i] = IN_BF16 ? __uint_as_float((i & 1) ? (r.w[i >> 1] & 0xFFFF0000u) : (r.w[i >> 1] << 16))
                   : __uint_as_float(r.w[i]);
}

constexpr int kConvBatch = 8;  // rows loaded together

template <bool IN_BF16, bool OUT_BF16, bool VEC>
__global__ void __launch_bounds__(256) conv_kernel(ConvArgs a) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int lpr = 1 << a.log_lpr;
  const int g = (int)(gid & (lpr - 1));
  const int64_t row_group = gid >> a.log_lpr;  // (memory, segment)
  // Lanes past the last segment still take part in the row reductions (whole groups are either
  // valid or not, and a group never straddles a wave), but write nothing.  Every lane loads from
  // a clamped, in-bounds address, so the loads need no branches.
  const bool valid = row_group < a.M * a.nseg;
  const int64_t m = valid ? row_group / a.nseg : 0;
  const int64_t seg = valid ? row_group % a.nseg : 0;
  const int h = (int)(m % a.heads);
  const int c0 = g * kConvCh;
  const bool lane_on = valid && c0 < a.d;
  const int cl = lane_on ? c0 : 0;

  float w[4][kConvCh], bs[kConvCh];
  if (VEC) {  // the lane's 8 channels' taps are 32 consecutive floats, its biases 8
    const float4* tp = (const float4*)(a.taps + ((int64_t)h * a.d + cl) * 4);
#pragma unroll
    for (int i = 0; i < kConvCh; ++i) {
      const float4 v = tp[i];
      w[0][i] = lane_on ? v.x : 0.0f;
      w[1][i] = lane_on ? v.y : 0.0f;
      w[2][i] = lane_on ? v.z : 0.0f;
      w[3][i] = lane_on ? v.w : 0.0f;
    }
    if (a.bias) {
      const float4* bp = (const float4*)(a.bias + (int64_t)h * a.d + cl);
      const float4 b0 = bp[0], b1 = bp[1];
      const float bv[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
#pragma unroll
      for (int i = 0; i < kConvCh; ++i) bs[i] = lane_on ? bv[i] : 0.0f;
    } else {
#pragma unroll
      for (int i = 0; i < kConvCh; ++i) bs[i] = 0.0f;
    }
  } else {
#pragma unroll
    for (int i = 0; i < kConvCh; ++i) {
      const bool in = lane_on && c0 + i < a.d;
      const float* tp = a.taps + ((int64_t)h * a.d + (in ? c0 + i : 0)) * 4;
#pragma unroll
      for (int j = 0; j < 4; ++j) w[j][i] = in ? tp[j] : 0.0f;
      bs[i] = (in && a.bias) ? a.bias[(int64_t)h * a.d + c0 + i] : 0.0f;
    }
  }

  const int64_t t0 = seg * kConvSeg;
  const int64_t t1 = t0 + kConvSeg < a.T ? t0 + kConvSeg : a.T;
  const int64_t rowbase = m * a.T;  // row index of token 0 of this memory
  // the three rows before the segment: x_{t0-3}, x_{t0-2}, x_{t0-1}
  float p3[kConvCh], p2[kConvCh], p1[kConvCh];
  auto prev_row = [&](int64_t t, float (&v)[kConvCh]) __attribute__((always_inline)) {
    if (!lane_on || (t < 0 && !a.hist)) {
#pragma unroll
      for (int i = 0; i < kConvCh; ++i) v[i] = 0.0f;
    } else {
      RawRow<IN_BF16> r;
      if (t >= 0) conv_load<IN_BF16, VEC>(a.X, (rowbase + t) * a.d, c0, a.d, r);
      else conv_load<IN_BF16, VEC>(a.hist, (m * 3 + 3 + t) * a.d, c0, a.d, r);
      conv_unpack<IN_BF16>(r, v);
    }
  };
  prev_row(t0 - 3, p3);
  prev_row(t0 - 2, p2);
  prev_row(t0 - 1, p1);

#pragma unroll
  for (int bt = 0; bt < kConvSeg / kConvBatch; ++bt) {
    RawRow<IN_BF16> raw[kConvBatch];
#pragma unroll
    for (int i = 0; i < kConvBatch; ++i) {
      const int64_t t = t0 + bt * kConvBatch + i;
      const int64_t tc = t < t1 ? t : t1 - 1;
      conv_load<IN_BF16, VEC>(a.X, (rowbase + tc) * a.d, cl, a.d, raw[i]);
    }
#pragma unroll
    for (int i = 0; i < kConvBatch; ++i) {
      const int64_t t = t0 + bt * kConvBatch + i;
      const bool tok = lane_on && t < t1;
      float x[kConvCh];
      conv_unpack<IN_BF16>(raw[i], x);
      float y[kConvCh];
      float ss = 0.0f;
#pragma unroll
      for (int k = 0; k < kConvCh; ++k) {
        const float xv = tok ? x[k] : 0.0f;
        float acc = bs[k];
        acc = fmaf(w[0][k], p3[k], acc);
        acc = fmaf(w[1][k], p2[k], acc);
        acc = fmaf(w[2][k], p1[k], acc);
        acc = fmaf(w[3][k], xv, acc);
        y[k] = acc;
        ss = fmaf(acc, acc, ss);
        p3[k] = p2[k];
        p2[k] = p1[k];
        p1[k] = xv;
      }
      if (a.l2norm) {  // uniform branch: every lane of the wave takes it
        for (int off = 1; off < lpr; off <<= 1) ss += __shfl_xor(ss, off, 64);
        const float inv = 1.0f / fmaxf(sqrtf(ss), 1e-12f);
#pragma unroll
        for (int k = 0; k < kConvCh; ++k) y[k] *= inv;
      }
      if (!tok) continue;
      const int64_t o = (rowbase + t) * a.d + c0;
      if (OUT_BF16) {
        uint16_t* dst = (uint16_t*)a.out + o;
        if (VEC) {
          *(u32x4*)dst = u32x4{cvt_pk_bf16(y[0], y[1]), cvt_pk_bf16(y[2], y[3]), cvt_pk_bf16(y[4], y[5]),
                               cvt_pk_bf16(y[6], y[7])};
        } else {
#pragma unroll
          for (int k = 0; k < kConvCh; ++k)
            if (c0 + k < a.d) dst[k] = (uint16_t)bf16_bits(y[k]);
        }
      } else {
        float* dst = (float*)a.out + o;
        if (VEC) {
          *(float4*)dst = float4{y[0], y[1], y[2], y[3]};
          *(float4*)(dst + 4) = float4{y[4], y[5], y[6], y[7]};
        } else {
#pragma unroll
          for (int k = 0; k < kConvCh; ++k)
            if (c0 + k < a.d) dst[k] = y[k];
        }
      }
    }
  }
}

// The three rows before the next call's first token: the last three of (hist ++ X).
__global__ void conv_hist_kernel(const void* X, const void* hist, int esz, int64_t M, int64_t T, int d,
                                 void* hist_out) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= M * 3 * d) return;
  const int c = (int)(idx % d);
  const int r = (int)((idx / d) % 3);
  const int64_t m = idx / (3 * (int64_t)d);
  const int64_t t = T - 3 + r;
  const char* src = nullptr;
  if (t >= 0) src = (const char*)X + ((m * T + t) * d + c) * esz;
  else if (hist) src = (const char*)hist + ((m * 3 + 3 + t) * d + c) * esz;
  char* dst = (char*)hist_out + idx * esz;
  if (esz == 2) *(uint16_t*)dst = src ? *(const uint16_t*)src : (uint16_t)0;
  else *(float*)dst = src ? *(const float*)src : 0.0f;
}

atlasmem_status launch_short_conv(const void* X, bool in_bf16, int64_t M, int64_t T, int d, int heads,
                                  const float* taps, const float* bias, const void* hist, bool l2norm, void* out,
                                  bool out_bf16, void* hist_out, hipStream_t st) {
  if (T > 0) {
    ConvArgs a;
    a.X = X;
    a.M = M;
    a.T = T;
    a.d = d;
    a.heads = heads;
    int lpr = 1, log_lpr = 0;
    while (lpr * kConvCh < d) {
      lpr <<= 1;
      ++log_lpr;
    }
    a.log_lpr = log_lpr;
    a.nseg = (T + kConvSeg - 1) / kConvSeg;
    a.taps = taps;
    a.bias = bias;
    a.hist = hist;
    a.l2norm = l2norm;
    a.out = out;
    const int64_t lanes = M * a.nseg * lpr;
    const int64_t blocks = (lanes + 255) / 256;
    if (blocks > INT32_MAX) return ATLASMEM_E_SHAPE;
    // 16-byte row, tap and bias accesses need whole 8-channel runs and aligned bases
    const bool vec = d % kConvCh == 0 &&
                     (((uintptr_t)X | (uintptr_t)out | (uintptr_t)hist | (uintptr_t)taps | (uintptr_t)bias) & 15) == 0;
#define AM_CONV(IB, OB, V) hipLaunchKernelGGL((conv_kernel<IB, OB, V>), dim3((unsigned)blocks), dim3(256), 0, st, a)
    if (in_bf16 && out_bf16) { if (vec) AM_CONV(true, true, true); else AM_CONV(true, true, false); }
    else if (in_bf16) { if (vec) AM_CONV(true, false, true); else AM_CONV(true, false, false); }
    else if (out_bf16) { if (vec) AM_CONV(false, true, true); else AM_CONV(false, true, false); }
    else { if (vec) AM_CONV(false, false, true); else AM_CONV(false, false, false); }
#undef AM_CONV
    AM_LAUNCH_CHECK();
  }
  if (hist_out) {
    const int64_t n = M * 3 * d;
    if (n > 0) {
      hipLaunchKernelGGL(conv_hist_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, X, hist,
                         in_bf16 ? 2 : 4, M, T, d, hist_out);
      AM_LAUNCH_CHECK();
    }
  }
  return ATLASMEM_OK;
}

// ------------------------------------------------------------------------ convolution folded into the update
//
// The inverse L2 norm of each convolved row, for the update's loaders, which convolve the raw rows
// as they read them (the convolved rows are never written: only this 4-byte factor per row).  The
// lanes, channels and order of the multiply-adds and of the norm's reduction are those of
// conv_kernel, so the loaders' rows equal the stand-alone convolution's bit for bit.
__global__ void __launch_bounds__(256) conv_inv_norm_kernel(const void* __restrict__ X, const void* __restrict__ hist,
                                                            int in_bf16, int64_t M, int64_t ld, int64_t t0, int64_t n,
                                                            int d, int heads, int log_lpr, const float* __restrict__ taps,
                                                            const float* __restrict__ bias, float* __restrict__ inv,
                                                            int64_t ld_inv) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int lpr = 1 << log_lpr;
  const int g = (int)(gid & (lpr - 1));
  const int64_t row = gid >> log_lpr;  // (memory, token)
  const bool valid = row < M * n;
  const int64_t m = valid ? row / n : 0;
  const int64_t t = t0 + (valid ? row % n : 0);
  const int h = (int)(m % heads);
  const int c0 = g * kConvCh;
  float ss = 0.0f;
#pragma unroll
  for (int k = 0; k < kConvCh; ++k) {
    const int c = c0 + k;
    const bool on = valid && c < d;
    const int cc = on ? c : 0;
    const float* tp = taps + ((int64_t)h * d + cc) * 4;
    float x[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t t2 = t - 3 + j;
      x[j] = !on ? 0.0f
                 : (t2 >= 0 ? load_in(X, (m * ld + t2) * d + cc, in_bf16)
                            : load_in(hist, (m * 3 + 3 + t2) * d + cc, in_bf16));
    }
    float acc = (on && bias) ? bias[(int64_t)h * d + cc] : 0.0f;
    acc = fmaf(on ? tp[0] : 0.0f, x[0], acc);
    acc = fmaf(on ? tp[1] : 0.0f, x[1], acc);
    acc = fmaf(on ? tp[2] : 0.0f, x[2], acc);
    acc = fmaf(on ? tp[3] : 0.0f, x[3], acc);
    ss = fmaf(acc, acc, ss);
  }
  for (int off = 1; off < lpr; off <<= 1) ss += __shfl_xor(ss, off, 64);
  if (valid && g == 0) inv[m * ld_inv + (t - t0)] = 1.0f / fmaxf(sqrtf(ss), 1e-12f);
}

// The three rows before the next call's first token: the last three of hist ++ X[0, T).
__global__ void conv_carry_kernel(const void* __restrict__ X, const void* __restrict__ hist, int esz, int64_t M,
                                  int64_t ld, int64_t T, int d, void* __restrict__ out) {
  const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= M * 3 * d) return;
  const int i = (int)(e % d);
  const int r = (int)((e / d) % 3);
  const int64_t m = e / (3 * (int64_t)d);
  const int64_t tau = T - 3 + r;
  if (esz == 2) {
    const uint16_t v = tau >= 0 ? ((const uint16_t*)X)[(m * ld + tau) * d + i]
                                : ((const uint16_t*)hist)[(m * 3 + 3 + tau) * d + i];
    ((uint16_t*)out)[e] = v;
  } else {
    const float v = tau >= 0 ? ((const float*)X)[(m * ld + tau) * d + i] : ((const float*)hist)[(m * 3 + 3 + tau) * d + i];
    ((float*)out)[e] = v;
  }
}

atlasmem_status launch_conv_inv_norm(const void* X, const void* hist, bool in_bf16, int M, int64_t ld, int64_t t0,
                                     int64_t n, int d, int heads, const float* taps, const float* bias, float* inv,
                                     int64_t ld_inv, hipStream_t st) {
  if (n <= 0 || M <= 0) return ATLASMEM_OK;
  if (d < 1 || d > 512) return ATLASMEM_E_SHAPE;
  int log_lpr = 0;
  while ((1 << log_lpr) * kConvCh < d) ++log_lpr;
  const int64_t threads = (int64_t)M * n << log_lpr;
  hipLaunchKernelGGL(conv_inv_norm_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, st, X, hist,
                     (int)in_bf16, (int64_t)M, ld, t0, n, d, heads, log_lpr, taps, bias, inv, ld_inv);
  AM_LAUNCH_CHECK();
  return ATLASMEM_OK;
}

atlasmem_status launch_conv_carry(const void* X, const void* hist, bool in_bf16, int M, int64_t ld, int64_t T, int d,
                                  void* hist_out, hipStream_t st) {
  const int64_t n = (int64_t)M * 3 * d;
  if (n == 0) return ATLASMEM_OK;
  hipLaunchKernelGGL(conv_carry_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, X, hist, in_bf16 ? 2 : 4,
                     (int64_t)M, ld, T, d, hist_out);
  AM_LAUNCH_CHECK();
  return ATLASMEM_OK;
}

// ------------------------------------------------------------------------ gates

constexpr int kGateCols = 64;    // output columns (gate, head) per pass
constexpr int kGateRows = 32;    // tokens per MFMA block
constexpr int kGateWaves = 16;  // at most: one workgroup per CU (LDS), four waves per SIMD
constexpr int kGateMaxDm = 512;

struct GateArgs {
  const uint16_t* U;  // [B, T, dm] bf16
  int64_t B, T;
  int dm, H, ncol;    // ncol = n_gates * H
  int n0;             // first column of this pass
  const float* Wg;    // [ncol, dm]
  const float* bg;    // [ncol]
  const float* scale; // [n_gates]
  int chunk;          // 1: per token; else a multiple of 32: mean-pooled per chunk
  int64_t nout;       // outputs per sequence: T or ceil(T / chunk)
  int64_t units;      // B * (blocks or chunks per sequence)
  float* out;         // [n_gates, B, H, nout]
};

// LDS: the pass's 64 weight rows split into bf16 hi / lo, [col][k] with a row stride of dm + 8
// (16-byte reads of 16 consecutive rows then fall on distinct banks).
template <bool POOL>
__global__ void __launch_bounds__(kGateWaves * 64) gates_kernel(GateArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint16_t gl[];
  const int ldw = a.dm + 8;
  uint16_t* wh = gl;
  uint16_t* wl = gl + kGateCols * ldw;
  for (int e = threadIdx.x; e < kGateCols * a.dm; e += blockDim.x) {
    const int n = e / a.dm, k = e - n * a.dm;
    const float v = (a.n0 + n < a.ncol) ? a.Wg[(int64_t)(a.n0 + n) * a.dm + k] : 0.0f;
    uint32_t hi, lo;
    split_bf16(v, hi, lo);
    wh[n * ldw + k] = (uint16_t)hi;
    wl[n * ldw + k] = (uint16_t)lo;
  }
  __syncthreads();

  const int lane = threadIdx.x & 63, hf = lane >> 5, l32 = lane & 31;
  const int wave = threadIdx.x >> 6, nwaves = blockDim.x >> 6;
  const int ksteps = a.dm / 16;
  // this lane's two output columns and their constants
  float bias[2], sc[2];
  int gi[2], hi_[2];
  bool col_ok[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int n = a.n0 + 32 * j + l32;
    col_ok[j] = n < a.ncol;
    const int nn = col_ok[j] ? n : 0;
    gi[j] = nn / a.H;
    hi_[j] = nn - gi[j] * a.H;
    bias[j] = a.bg[nn];
    sc[j] = a.scale[gi[j]];
  }
  const int64_t per_seq = a.units / a.B;
  const int blocks_per_unit = POOL ? a.chunk / kGateRows : 1;

  for (int64_t u = (int64_t)blockIdx.x * nwaves + wave; u < a.units; u += (int64_t)gridDim.x * nwaves) {
    const int64_t b = u / per_seq, c = u - b * per_seq;
    const rsrc_t rU = make_rsrc(a.U + b * a.T * a.dm, (uint32_t)(a.T * a.dm * 2));
    float colsum[2] = {0.0f, 0.0f};
    for (int blk = 0; blk < blocks_per_unit; ++blk) {
      const int64_t t0 = (POOL ? c * a.chunk : 0) + (int64_t)(POOL ? blk : c) * kGateRows;
      f32x16 acc[2] = {f32x16{}, f32x16{}};
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[j][r] = 0.0f;
      if (t0 < a.T) {
        // rows past T read as zero (range-checked buffer loads), so they add nothing
        const int voff = (int)(((t0 + l32) * a.dm + 8 * hf) * 2);
        // k-steps in runs of four, double-buffered: the next run's loads are issued before the
        // current run's products, so a wave keeps eight 16-byte loads per lane in flight throughout
        constexpr int KR = 4;
        auto load_run = [&](int k0, u32x4 (&x)[KR]) __attribute__((always_inline)) {
#pragma unroll
          for (int i = 0; i < KR; ++i) x[i] = buf_ld16(rU, voff + (k0 + i) * 32, 0);
        };
        auto mul_run = [&](int k0, const u32x4 (&x)[KR]) __attribute__((always_inline)) {
#pragma unroll
          for (int i = 0; i < KR; ++i) {
            if (k0 + i < ksteps) {
              const int ko = 16 * (k0 + i) + 8 * hf;
#pragma unroll
              for (int j = 0; j < 2; ++j) {
                const int o = (32 * j + l32) * ldw + ko;
                acc[j] = mfma32(x[i], *(const u32x4*)(wh + o), acc[j]);
                acc[j] = mfma32(x[i], *(const u32x4*)(wl + o), acc[j]);
              }
            }
          }
        };
        u32x4 xa[KR], xb[KR];
        load_run(0, xa);
        for (int k0 = 0; k0 < ksteps; k0 += 2 * KR) {
          if (k0 + KR < ksteps) load_run(k0 + KR, xb);
          mul_run(k0, xa);
          if (k0 + 2 * KR < ksteps) load_run(k0 + 2 * KR, xa);
          if (k0 + KR < ksteps) mul_run(k0 + KR, xb);
        }
      }
      if (POOL) {
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) colsum[j] += acc[j][r];
      } else {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          if (!col_ok[j]) continue;
          float* row = a.out + (((int64_t)gi[j] * a.B + b) * a.H + hi_[j]) * a.nout;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            // four consecutive tokens per register quad: one 16-byte store when whole and aligned
            const int64_t t = t0 + 8 * q + 4 * hf;
            float v[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) v[u] = sc[j] * sigmoidf_(acc[j][4 * q + u] + bias[j]);
            if (a.nout % 4 == 0 && t + 3 < a.T) {
              *(float4*)(row + t) = float4{v[0], v[1], v[2], v[3]};
            } else {
#pragma unroll
              for (int u = 0; u < 4; ++u)
                if (t + u < a.T) row[t + u] = v[u];
            }
          }
        }
      }
    }
    if (POOL) {
      const int64_t s0 = c * a.chunk;
      const int64_t cnt = (a.T - s0) < a.chunk ? (a.T - s0) : a.chunk;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const float tot = colsum[j] + __shfl_xor(colsum[j], 32, 64);
        if (hf == 0 && col_ok[j]) {
          const float z = tot / (float)cnt + bias[j];
          a.out[(((int64_t)gi[j] * a.B + b) * a.H + hi_[j]) * a.nout + c] = sc[j] * sigmoidf_(z);
        }
      }
    }
  }
}

size_t gates_lds_bytes(int dm) { return (size_t)2 * kGateCols * (dm + 8) * sizeof(uint16_t); }

atlasmem_status launch_gates(const void* U, int64_t B, int64_t T, int dm, int H, int n_gates, const float* Wg,
                             const float* bg, const float* scale, int chunk, float* out, hipStream_t st) {
  if (B == 0 || T == 0) return ATLASMEM_OK;
  GateArgs a;
  a.U = (const uint16_t*)U;
  a.B = B;
  a.T = T;
  a.dm = dm;
  a.H = H;
  a.ncol = n_gates * H;
  a.Wg = Wg;
  a.bg = bg;
  a.scale = scale;
  a.chunk = chunk;
  const bool pool = chunk > 1;
  a.nout = pool ? (T + chunk - 1) / chunk : T;
  a.units = B * (pool ? a.nout : (T + kGateRows - 1) / kGateRows);
  a.out = out;
  const size_t lds = gates_lds_bytes(dm);
  int dev = 0, ncu = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) !=
                                              hipSuccess)
    return ATLASMEM_E_DEVICE;
  // one workgroup per CU (the weights fill most of the LDS); as many waves as the units keep busy
  const int64_t per_cu = (a.units + ncu - 1) / ncu;
  const int nw = per_cu < 4 ? 4 : (per_cu > kGateWaves ? kGateWaves : (int)per_cu);
  const int64_t want = (a.units + nw - 1) / nw;
  const unsigned grid = (unsigned)(want < ncu ? want : ncu);
  for (int n0 = 0; n0 < a.ncol; n0 += kGateCols) {
    a.n0 = n0;
    if (pool) {
      if (hipFuncSetAttribute((const void*)gates_kernel<true>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) !=
          hipSuccess)
        return ATLASMEM_E_DEVICE;
      hipLaunchKernelGGL(gates_kernel<true>, dim3(grid), dim3(nw * 64), lds, st, a);
    } else {
      if (hipFuncSetAttribute((const void*)gates_kernel<false>, hipFuncAttributeMaxDynamicSharedMemorySize,
                              (int)lds) != hipSuccess)
        return ATLASMEM_E_DEVICE;
      hipLaunchKernelGGL(gates_kernel<false>, dim3(grid), dim3(nw * 64), lds, st, a);
    }
    AM_LAUNCH_CHECK();
  }
  return ATLASMEM_OK;
}

bool gates_supported(int dm, int chunk) {
  return dm >= 16 && dm <= kGateMaxDm && dm % 16 == 0 && (chunk == 1 || chunk % kGateRows == 0);
}

}  // namespace am
