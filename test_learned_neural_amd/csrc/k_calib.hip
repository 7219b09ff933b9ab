// Calibration kernels: the matrix-core rate and a plain copy, the measured ceilings next to which
// the update's kernels are reported.
#include "common.h"
#include "internal.h"
#include "../../include/atlasmem_calibration.h"

namespace am {

// Eight independent accumulation chains per wave: each v_mfma_f32_32x32x16_bf16 depends only on
// the previous instruction of its own chain, eight instructions back, so the matrix core issues
// back to back.  The operands come from the thread index (no memory traffic).
__global__ void __launch_bounds__(512) mfma_peak_kernel(int64_t iters, float* sink) {
  const int t = threadIdx.x;
  const uint32_t x = 0x3F803F80u ^ (uint32_t)(t & 7);  // bf16 pairs near 1.0
  const u32x4 a = u32x4{x, x ^ 1u, x ^ 2u, x ^ 3u};
  const u32x4 b = u32x4{x ^ 4u, x ^ 5u, x ^ 6u, x ^ 7u};
  f32x16 acc[8];
#pragma unroll
  for (int c = 0; c < 8; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[c][r] = 0.0f;
  for (int64_t i = 0; i < iters; ++i) {
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[c] = mfma32(a, b, acc[c]);
  }
  float s = 0.0f;
#pragma unroll
  for (int c = 0; c < 8; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[c][r];
  if (t == 0) sink[blockIdx.x] = s;
}

// Eight 16-byte loads in flight per thread before their stores; a block covers 8 x 256 consecutive
// 16-byte words per round.
constexpr int kCopyUnroll = 8;
__global__ void __launch_bounds__(256) copy16_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst, int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * (256 * kCopyUnroll);
  for (int64_t b = (int64_t)blockIdx.x * (256 * kCopyUnroll); b < n; b += stride) {
    u32x4 v[kCopyUnroll];
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) {
      const int64_t i = b + u * 256 + threadIdx.x;
      if (i < n) v[u] = __builtin_nontemporal_load(src + i);
    }
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) {
      const int64_t i = b + u * 256 + threadIdx.x;
      if (i < n) __builtin_nontemporal_store(v[u], dst + i);
    }
  }
}

}  // namespace am

extern "C" {

int atlasmem_calibrate_mfma(int64_t iters, int32_t n_workgroups, float* sink, void* stream) {
  if (iters < 1 || n_workgroups < 1 || !sink) return ATLASMEM_E_INVALID;
  hipLaunchKernelGGL(am::mfma_peak_kernel, dim3(n_workgroups), dim3(512), 0, (hipStream_t)stream, iters, sink);
  AM_LAUNCH_CHECK();
  return ATLASMEM_OK;
}

int atlasmem_calibrate_copy(const void* src, void* dst, int64_t bytes, void* stream) {
  if (!src || !dst || bytes < 0 || bytes % 16 != 0) return ATLASMEM_E_INVALID;
  const char* s = (const char*)src;
  char* d = (char*)dst;
  if (s < d + bytes && d < s + bytes && bytes > 0) return ATLASMEM_E_INVALID;
  if (bytes == 0) return ATLASMEM_OK;
  const int64_t n = bytes / 16;
  const int64_t per_block = 256 * am::kCopyUnroll;
  const int64_t blocks = (n + per_block - 1) / per_block < 8192 ? (n + per_block - 1) / per_block : 8192;
  hipLaunchKernelGGL(am::copy16_kernel, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream, (const u32x4*)src,
                     (u32x4*)dst, n);
  AM_LAUNCH_CHECK();
  return ATLASMEM_OK;
}

}  // extern "C"
