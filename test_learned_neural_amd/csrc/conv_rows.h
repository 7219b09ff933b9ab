// The causal short convolution evaluated where a row element is read (the update's loaders), so
// that the convolved rows are never written: element i of token tau of a tensor X (keys, queries
// or values of memory m, head h = m % heads) is
//     round(inv[tau] * (bias[h][i] + sum_{j=0..3} taps[h][i][j] * X[tau - 3 + j][i]))
// with X[tau'] for tau' < 0 from the three rows carried from the previous call, inv the row's
// inverse L2 norm (keys and queries; 1 without normalisation) and one rounding to the input dtype
// (Atlas-Torch README, Atlas Extensions table, "Short Convolution": kernel 4 on keys, values and
// queries; titans-pytorch-mlx README, Configuration table, use_conv / conv_kernel_size 4).  The
// multiply-adds run in the stand-alone convolution kernel's order, so both give the same rows.
#pragma once

#include "common.h"

namespace am {

struct ConvTensor {
  const void* X;       // raw rows of the call, memory m, token tau at (m * ld + tau) * d
  const void* hist;    // [M][3][d] the three raw rows before the call (oldest first), input dtype
  const float* taps;   // [heads][d][4]
  const float* bias;   // [heads][d] or null
  const float* inv;    // inverse row norms [M][ninv] of tokens [t0, t0 + ninv), or null
  int64_t t0;
  int ninv, heads, d, in_bf16;

  __device__ __forceinline__ float at(int m, int64_t ld, int64_t tau, int i) const {
    const int h = m % heads;
    const float* tp = taps + ((int64_t)h * d + i) * 4;
    float x[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t t2 = tau - 3 + j;
      x[j] = t2 >= 0 ? load_in(X, ((int64_t)m * ld + t2) * d + i, in_bf16)
                     : load_in(hist, ((int64_t)m * 3 + 3 + t2) * d + i, in_bf16);
    }
    float acc = bias ? bias[(int64_t)h * d + i] : 0.0f;
    acc = fmaf(tp[0], x[0], acc);
    acc = fmaf(tp[1], x[1], acc);
    acc = fmaf(tp[2], x[2], acc);
    acc = fmaf(tp[3], x[3], acc);
    if (inv) acc *= inv[(int64_t)m * ninv + (tau - t0)];
    return in_bf16 ? bf16_value(bf16_bits(acc)) : acc;
  }
};

}  // namespace am
