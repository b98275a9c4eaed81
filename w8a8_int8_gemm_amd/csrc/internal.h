// internal.h -- shared declarations of the HIP kernels' launchers and the
// small device helpers they use.  Not part of the public ABI (include/w8a8.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace w8a8 {

// ---------------------------------------------------------------------------
// device helpers
// ---------------------------------------------------------------------------

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// binary32 -> BF16 bits, nearest with ties to even (carry into the exponent
// gives the next binade or Inf, both correct); NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  uint32_t r = (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
  return (f != f) ? ((u >> 16) | 0x40u) : r;
}

// binary64 -> BF16 bits with a single rounding: first to binary32 with
// round-to-odd (truncate toward zero, set the last bit when inexact), then
// to BF16 with ties to even.  Round-to-odd into a format with at least two
// more significand bits than the target makes the second rounding correct.
__device__ __forceinline__ uint32_t f64_to_bf16_rne(double d) {
  const float f = (float)d;
  uint32_t u = __float_as_uint(f);
  const double back = (double)f;
  if (back != d) {
    if (fabs(back) > fabs(d)) u -= 1u;  // rounded away from zero: step back
    u |= 1u;
  }
  return f32_to_bf16_rne(__uint_as_float(u));
}

// SiLU(x) = x / (1 + exp(-x)) correctly rounded to BF16.  The binary32
// evaluation is within a few ulps of the exact value for |x| < 64, so its
// BF16 rounding is already correct unless it lies within 64 binary32 ulps
// of a BF16 rounding midpoint (low 16 bits near 0x8000); those rare
// elements, and |x| >= 64, are evaluated in binary64 and rounded once.
// Shared by the stand-alone SiLU kernel and the fused SiLU + quantize
// kernel, so both produce the same bits.
__device__ __forceinline__ uint32_t silu_bf16_bits(uint32_t xbits16) {
  const float x = bf16_to_f32(xbits16);
  const float y = x / (1.0f + expf(-x));
  const int d = (int)(__float_as_uint(y) & 0xFFFFu) - 0x8000;
  if (fabsf(x) < 64.0f && (d > 64 || d < -64)) return f32_to_bf16_rne(y);
  const double xd = (double)x;
  return f64_to_bf16_rne(xd / (1.0 + exp(-xd)));
}

// ---------------------------------------------------------------------------
// launchers (arguments already validated by the API layer)
// ---------------------------------------------------------------------------

hipError_t launch_quantize_act(const uint16_t *x, int8_t *q, float *sa,
                               int64_t M, int64_t K, bool fuse_silu,
                               hipStream_t stream);
hipError_t launch_silu(const uint16_t *x, uint16_t *y, int64_t n,
                       hipStream_t stream);
hipError_t launch_pow2_renorm(const uint16_t *x, uint16_t *y, int64_t M,
                              int64_t K, hipStream_t stream);

enum EpiKind : int { EPI_BF16 = 0, EPI_FP32 = 1, EPI_I32 = 2 };

struct GemmArgs {
  const int8_t *a;     // [M,K]
  const float *sa;     // [M]
  const int8_t *w;     // [N,K]
  const float *sw;     // [N]
  const uint16_t *bias;  // [N] or nullptr
  void *out;           // [M,N]
  int epi;             // EpiKind
  int64_t M, N, K;
  void *workspace;
  size_t workspace_bytes;
};

// Plan of one GEMM launch: which tile configuration, how many K splits.
struct GemmPlan {
  int config;      // index into the kernel table
  int splits;      // 1 = no split-K
  size_t workspace;  // bytes of INT32 partials (0 when splits == 1)
};

GemmPlan plan_gemm(int64_t M, int64_t N, int64_t K);
hipError_t launch_gemm(const GemmArgs &args, const GemmPlan &plan,
                       hipStream_t stream);

}  // namespace w8a8
