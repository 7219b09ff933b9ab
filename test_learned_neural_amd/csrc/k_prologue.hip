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
constexpr int kConvSeg = 32;  // consecutive tokens per lane

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

template <bool IN_BF16, bool OUT_BF16, bool VEC>
__device__ __forceinline__ void conv_load(const void* base, int64_t off, int c0, int d, float (&v)[kConvCh]) {
  if (VEC) {  // d % 8 == 0: the lane's 8 channels are one aligned 16-byte (bf16) or 32-byte (fp32) run
    if (IN_BF16) {
      const u32x4 w = *(const u32x4*)((const uint16_t*)base + off + c0);
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        v[2 * p] = __uint_as_float(w[p] << 16);
        v[2 * p + 1] = __uint_as_float(w[p] & 0xFFFF0000u);
      }
    } else {
      const float4 a = *(const float4*)((const float*)base + off + c0);
      const float4 b = *(const float4*)((const float*)base + off + c0 + 4);
      v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
      v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < kConvCh; ++i) v[i] = (c0 + i < d) ? load_in(base, off + c0 + i, IN_BF16) : 0.0f;
  }
}

template <bool IN_BF16, bool OUT_BF16, bool VEC>
__global__ void __launch_bounds__(256) conv_kernel(ConvArgs a) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int lpr = 1 << a.log_lpr;
  const int g = (int)(gid & (lpr - 1));
  const int64_t row_group = gid >> a.log_lpr;  // (memory, segment)
  // Lanes past the last segment still take part in the row reductions (whole groups are either
  // valid or not, and a group never straddles a wave), but read and write nothing.
  const bool valid = row_group < a.M * a.nseg;
  const int64_t m = valid ? row_group / a.nseg : 0;
  const int64_t seg = valid ? row_group % a.nseg : 0;
  const int h = (int)(m % a.heads);
  const int c0 = g * kConvCh;
  const bool lane_on = valid && c0 < a.d;

  float w[4][kConvCh], bs[kConvCh];
#pragma unroll
  for (int i = 0; i < kConvCh; ++i) {
    const bool in = lane_on && c0 + i < a.d;
    const float* tp = a.taps + ((int64_t)h * a.d + c0 + i) * 4;
#pragma unroll
    for (int j = 0; j < 4; ++j) w[j][i] = in ? tp[j] : 0.0f;
    bs[i] = (in && a.bias) ? a.bias[(int64_t)h * a.d + c0 + i] : 0.0f;
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
    } else if (t >= 0) {
      conv_load<IN_BF16, OUT_BF16, VEC>(a.X, (rowbase + t) * a.d, c0, a.d, v);
    } else {
      conv_load<IN_BF16, OUT_BF16, VEC>(a.hist, (m * 3 + 3 + t) * a.d, c0, a.d, v);
    }
  };
  prev_row(t0 - 3, p3);
  prev_row(t0 - 2, p2);
  prev_row(t0 - 1, p1);

  for (int64_t t = t0; t < t0 + kConvSeg; ++t) {
    const bool tok = lane_on && t < t1;
    float x[kConvCh];
    if (tok) {
      conv_load<IN_BF16, OUT_BF16, VEC>(a.X, (rowbase + t) * a.d, c0, a.d, x);
    } else {
#pragma unroll
      for (int i = 0; i < kConvCh; ++i) x[i] = 0.0f;
    }
    float y[kConvCh];
    float ss = 0.0f;
#pragma unroll
    for (int i = 0; i < kConvCh; ++i) {
      float acc = bs[i];
      acc = fmaf(w[0][i], p3[i], acc);
      acc = fmaf(w[1][i], p2[i], acc);
      acc = fmaf(w[2][i], p1[i], acc);
      acc = fmaf(w[3][i], x[i], acc);
      y[i] = acc;
      ss = fmaf(acc, acc, ss);
      p3[i] = p2[i];
      p2[i] = p1[i];
      p1[i] = x[i];
    }
    if (a.l2norm) {  // uniform branch: every lane of the wave takes it
      for (int off = 1; off < lpr; off <<= 1) ss += __shfl_xor(ss, off, 64);
      const float inv = 1.0f / fmaxf(sqrtf(ss), 1e-12f);
#pragma unroll
      for (int i = 0; i < kConvCh; ++i) y[i] *= inv;
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
        for (int i = 0; i < kConvCh; ++i)
          if (c0 + i < a.d) dst[i] = (uint16_t)bf16_bits(y[i]);
      }
    } else {
      float* dst = (float*)a.out + o;
      if (VEC) {
        *(float4*)dst = float4{y[0], y[1], y[2], y[3]};
        *(float4*)(dst + 4) = float4{y[4], y[5], y[6], y[7]};
      } else {
#pragma unroll
        for (int i = 0; i < kConvCh; ++i)
          if (c0 + i < a.d) dst[i] = y[i];
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
    // 16-byte row accesses need whole 8-channel runs and aligned bases
    const bool vec = d % kConvCh == 0 && (((uintptr_t)X | (uintptr_t)out | (uintptr_t)hist) & 15) == 0;
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

// ------------------------------------------------------------------------ gates

constexpr int kGateCols = 64;    // output columns (gate, head) per pass
constexpr int kGateRows = 32;    // tokens per MFMA block
constexpr int kGateWaves = 8;
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
  const int wave = threadIdx.x >> 6;
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

  for (int64_t u = (int64_t)blockIdx.x * kGateWaves + wave; u < a.units; u += (int64_t)gridDim.x * kGateWaves) {
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
        for (int k0 = 0; k0 < ksteps; k0 += 8) {
          u32x4 xa[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) xa[i] = buf_ld16(rU, voff + (k0 + i) * 32, 0);
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            if (k0 + i < ksteps) {
              const int ko = 16 * (k0 + i) + 8 * hf;
#pragma unroll
              for (int j = 0; j < 2; ++j) {
                const int o = (32 * j + l32) * ldw + ko;
                acc[j] = mfma32(xa[i], *(const u32x4*)(wh + o), acc[j]);
                acc[j] = mfma32(xa[i], *(const u32x4*)(wl + o), acc[j]);
              }
            }
          }
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
          for (int r = 0; r < 16; ++r) {
            const int64_t t = t0 + 8 * (r >> 2) + 4 * hf + (r & 3);
            if (t < a.T) row[t] = sc[j] * sigmoidf_(acc[j][r] + bias[j]);
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
  const int64_t want = (a.units + kGateWaves - 1) / kGateWaves;
  const unsigned grid = (unsigned)(want < ncu ? want : ncu);
  for (int n0 = 0; n0 < a.ncol; n0 += kGateCols) {
    a.n0 = n0;
    if (pool) {
      if (hipFuncSetAttribute((const void*)gates_kernel<true>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) !=
          hipSuccess)
        return ATLASMEM_E_DEVICE;
      hipLaunchKernelGGL(gates_kernel<true>, dim3(grid), dim3(kGateWaves * 64), lds, st, a);
    } else {
      if (hipFuncSetAttribute((const void*)gates_kernel<false>, hipFuncAttributeMaxDynamicSharedMemorySize,
                              (int)lds) != hipSuccess)
        return ATLASMEM_E_DEVICE;
      hipLaunchKernelGGL(gates_kernel<false>, dim3(grid), dim3(kGateWaves * 64), lds, st, a);
    }
    AM_LAUNCH_CHECK();
  }
  return ATLASMEM_OK;
}

bool gates_supported(int dm, int chunk) {
  return dm >= 16 && dm <= kGateMaxDm && dm % 16 == 0 && (chunk == 1 || chunk % kGateRows == 0);
}

}  // namespace am
