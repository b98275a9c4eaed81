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

typedef float f2v __attribute__((ext_vector_type(2)));
typedef __bf16 bf2v __attribute__((ext_vector_type(2)));

// Two binary32 values -> two BF16 (round to nearest, ties to even) packed in
// one dword, low half first: gfx950's v_cvt_pk_bf16_f32.  Callers pass
// finite values or +-Inf, never NaN.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf2v b = __builtin_convertvector(f2v{lo, hi}, bf2v);
  return __builtin_bit_cast(uint32_t, b);
}

// SiLU(x) = x / (1 + exp(-x)) evaluated in binary64 and rounded once to
// BF16 (the slow, always-correct path).
__device__ __noinline__ uint32_t silu_bf16_slow(float x) {
  const double xd = (double)x;
  return f64_to_bf16_rne(xd / (1.0 + exp(-xd)));
}

// SiLU of one BF16 input in binary32 with hardware exp2 / reciprocal.
// exp(-x) = 2^(-x*log2 e): log2 e is split into a 16-bit head (x has 8
// significant bits, so x*head is exact) and a tail whose 2^t factor is its
// second-order Taylor polynomial.  Over every BF16 input with |x| < 64 the
// result is within 2.5 binary32 ulps of SiLU(x) (measured on gfx950 against
// a binary64 evaluation); `ok` is false when the value lies within 6
// binary32 ulps of a BF16 rounding midpoint (low 16 bits near 0x8000),
// where that error could flip the rounding, or when |x| >= 64.
__device__ __forceinline__ float silu_f32(float x, bool &ok) {
  constexpr float kLog2eHi = 0x1.7154p+0f;       // 47274 / 2^15
  constexpr float kLog2eLo = 0x1.d94aep-18f;     // log2 e - kLog2eHi
  constexpr float kLn2 = 0x1.62e43p-1f;
  const float p1 = -x * kLog2eHi;
  const float t = (-x * kLog2eLo) * kLn2;
  const float e = __builtin_amdgcn_exp2f(p1) * fmaf(t, fmaf(t, 0.5f, 1.0f), 1.0f);
  const float y = x * __builtin_amdgcn_rcpf(1.0f + e);
  const int d = (int)(__float_as_uint(y) & 0xFFFFu) - 0x8000;
  ok = fabsf(x) < 64.0f && (d > 6 || d < -6);
  return y;
}

// SiLU of two packed BF16 values, each correctly rounded to BF16.  Shared by
// the stand-alone SiLU kernel and the fused SiLU + quantize kernel, so both
// produce the same bits.
__device__ __forceinline__ uint32_t silu_bf16x2(uint32_t packed) {
  const float x0 = bf16_to_f32(packed & 0xFFFFu);
  const float x1 = bf16_to_f32(packed >> 16);
  bool ok0, ok1;
  const float y0 = silu_f32(x0, ok0);
  const float y1 = silu_f32(x1, ok1);
  uint32_t r = pack_bf16x2(ok0 ? y0 : 0.0f, ok1 ? y1 : 0.0f);
  if (!ok0) r = (r & 0xFFFF0000u) | silu_bf16_slow(x0);
  if (!ok1) r = (r & 0x0000FFFFu) | (silu_bf16_slow(x1) << 16);
  return r;
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
  int config;        // index into the kernel table
  int splits;        // split-K over the whole output (1 = none)
  int group_m;       // token tiles per group in the tile order
  int main_tiles;    // tiles of the main launch (all tiles unless a tail)
  int tail_tiles;    // trailing tiles run split-K in a second launch
  int tail_splits;   // K slices per tail tile (0 = no tail launch)
  size_t workspace;  // bytes of INT32 partials needed (0 if none)
  int skinny_tm;     // single-launch skinny kernel: token fragments (1, 2)
};

GemmPlan plan_gemm(int64_t M, int64_t N, int64_t K);

// Device scratch of the allocation-free GEMM entry point: a file-scope
// device array in gemm.hip, one copy per GPU.  resolve_scratch() looks up
// this device's copy once (with the device current) and caches it;
// scratch_on_device() then returns it (nullptr if never resolved).
constexpr size_t kScratchBytes = size_t(64) << 20;
hipError_t resolve_scratch(int device);
void *scratch_on_device(int device);
// Whether every launch of the plan fits the hardware grid limits.
bool plan_launchable(const GemmPlan &plan);
hipError_t launch_gemm(const GemmArgs &args, const GemmPlan &plan,
                       hipStream_t stream);

}  // namespace w8a8
