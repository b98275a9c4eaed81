// rowwise.hip -- per-token kernels for gfx950: activation quantization
// (optionally fused with SiLU), the power-of-two row renormalization, and
// element-wise SiLU.
//
// Per-token symmetric quantization ("feat(mps): support MiniMax-H3 INT8
// inference on Apple M5", LightX2V pull request #1672, commit notes):
// scale = max|x| / 127 in binary32, code = round-half-even(x / scale)
// clamped to [-127, 127]; rows are split into 16-byte chunks of 8 BF16 and
// the partial chunk at the end of a row is masked.
//
// Layout: one row is owned by WPR wavefronts (WPR = 1 for rows up to 5632
// elements, 4 above); each lane keeps CH chunks of its row in registers, so
// HBM is read once and written once.  Chunk j of a row is held by lane
// (j mod 64) of wave part ((j / 64) mod WPR), which keeps every load and
// store instruction of a wave on 1 KiB (loads) or 512 B (INT8 stores) of
// consecutive bytes.  The row maximum is a wave64 butterfly reduction
// (and, for WPR = 4, one LDS exchange between the row's waves).
#include "internal.h"

namespace w8a8 {
namespace {

typedef unsigned v4u __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;  // 4 waves of 64
constexpr int kWaves = kThreads / 64;

enum RowOp : int { OP_QUANT = 0, OP_QUANT_SILU = 1, OP_RENORM = 2 };

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

// Per-row constants of the quantizer.  For rows whose scale is a normal
// number the codes come from u = fma(x, 1/s, 128): the reciprocal (one
// IEEE division per row), the product and the sum together stay within
// 2.3e-5 of 128 + RN(x/s) (|x/s| <= 127 + 2^-17), so when u is farther
// than 2^-14 from a half-integer, rounding u to the nearest integer gives
// exactly 128 + round_half_even(RN(x/s)).  The remaining elements (about
// one in 8000) and rows with a subnormal scale use the division itself.
struct QuantRow {
  float s, r;
  bool fast;
};

__device__ __forceinline__ QuantRow quant_row(float amax) {
  QuantRow q;
  q.s = amax / 127.0f;
  q.fast = q.s >= 0x1p-126f;
  q.r = q.fast ? 1.0f / q.s : 0.0f;
  return q;
}

// Code of one value as the byte (q + 128), q = clamp(rint(x / s)).
__device__ __noinline__ float quant_biased_exact(float x, float s) {
  const float q = fminf(fmaxf(rintf(x / s), -127.0f), 127.0f);
  return q + 128.0f;  // exact small integer
}

// Four BF16 values (two packed pairs) -> four INT8 codes in one dword.
__device__ __forceinline__ uint32_t quant4(uint32_t p01, uint32_t p23,
                                           const QuantRow &R) {
  const float f[4] = {bf16_to_f32(p01 & 0xFFFFu), bf16_to_f32(p01 >> 16),
                      bf16_to_f32(p23 & 0xFFFFu), bf16_to_f32(p23 >> 16)};
  uint32_t out = 0;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    float u = R.fast ? fmaf(f[e], R.r, 128.0f) : 0.5f;
    const float fr = __builtin_amdgcn_fractf(u);
    if (!(fabsf(fr - 0.5f) > 0x1p-14f)) u = quant_biased_exact(f[e], R.s);
    // round to the nearest integer in [0, 255] and insert as byte e
    out = __builtin_amdgcn_cvt_pk_u8_f32(u, e, out);
  }
  return out ^ 0x80808080u;  // biased byte -> two's complement code
}

__device__ __forceinline__ uint32_t silu_pair(uint32_t packed) {
  return silu_bf16x2(packed);
}

__device__ __forceinline__ float absmax_pair(uint32_t packed) {
  return fmaxf(fabsf(bf16_to_f32(packed & 0xFFFFu)),
               fabsf(bf16_to_f32(packed >> 16)));
}

__device__ __forceinline__ uint32_t renorm_pair(uint32_t packed, int e) {
  float f0 = ldexpf(bf16_to_f32(packed & 0xFFFFu), -e);
  float f1 = ldexpf(bf16_to_f32(packed >> 16), -e);
  return f32_to_bf16_rne(f0) | (f32_to_bf16_rne(f1) << 16);
}

template <int CH, int WPR, int OP>
__global__ __launch_bounds__(kThreads) void row_kernel(
    const uint16_t *x, void *out, float *__restrict__ scale, int64_t M,
    int K) {
  constexpr int RPB = kWaves / WPR;  // rows per block
  __shared__ float part_max[kWaves];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int part = wave % WPR;
  const int64_t row = (int64_t)blockIdx.x * RPB + wave / WPR;
  const bool row_ok = row < M;
  const int chunks = K >> 3;
  const v4u *xr = reinterpret_cast<const v4u *>(x + row * (int64_t)K);

  v4u v[CH];
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    const int j = (i * WPR + part) * 64 + lane;
    v[i] = v4u{0, 0, 0, 0};
    if (row_ok && j < chunks) {
      v4u c = __builtin_nontemporal_load(xr + j);
      if (OP == OP_QUANT_SILU) {
        c.x = silu_pair(c.x);
        c.y = silu_pair(c.y);
        c.z = silu_pair(c.z);
        c.w = silu_pair(c.w);
      }
      v[i] = c;
      amax = fmaxf(amax, fmaxf(fmaxf(absmax_pair(c.x), absmax_pair(c.y)),
                               fmaxf(absmax_pair(c.z), absmax_pair(c.w))));
    }
  }
  amax = wave_max(amax);
  if (WPR > 1) {
    if (lane == 0) part_max[wave] = amax;
    __syncthreads();
    const int base = (wave / WPR) * WPR;
    amax = part_max[base];
#pragma unroll
    for (int p = 1; p < WPR; ++p) amax = fmaxf(amax, part_max[base + p]);
  }
  if (!row_ok) return;

  if (OP == OP_RENORM) {
    v4u *yr = reinterpret_cast<v4u *>(static_cast<uint16_t *>(out) +
                                        row * (int64_t)K);
    int ex = 0;
    frexpf(amax, &ex);  // amax = f * 2^ex, f in [0.5, 1); ex = 0 for 0
    const int e = (amax == 0.0f) ? 0 : ex - 1;  // floor(log2(amax))
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int j = (i * WPR + part) * 64 + lane;
      if (j < chunks) {
        const v4u c = v[i];
        v4u o;
        o.x = renorm_pair(c.x, e);
        o.y = renorm_pair(c.y, e);
        o.z = renorm_pair(c.z, e);
        o.w = renorm_pair(c.w, e);
        __builtin_nontemporal_store(o, yr + j);
      }
    }
    return;
  }

  // Quantize: scale = amax / 127 (IEEE division), zero row -> scale 0.
  const QuantRow R = quant_row(amax);
  const float s = R.s;
  if (lane == 0 && part == 0) scale[row] = s;
  uint2 *qr = reinterpret_cast<uint2 *>(static_cast<int8_t *>(out) +
                                        row * (int64_t)K);
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    const int j = (i * WPR + part) * 64 + lane;
    if (j < chunks) {
      uint2 o = make_uint2(0, 0);
      if (s != 0.0f) {
        const v4u c = v[i];
        o.x = quant4(c.x, c.y, R);
        o.y = quant4(c.z, c.w, R);
      }
      qr[j] = o;
    }
  }
}

__global__ __launch_bounds__(kThreads) void silu_kernel(
    const uint16_t *x, uint16_t *y, int64_t chunks) {
  const v4u *xs = reinterpret_cast<const v4u *>(x);
  v4u *ys = reinterpret_cast<v4u *>(y);
  for (int64_t j = (int64_t)blockIdx.x * kThreads + threadIdx.x; j < chunks;
       j += (int64_t)gridDim.x * kThreads) {
    v4u c = __builtin_nontemporal_load(xs + j);
    c.x = silu_pair(c.x);
    c.y = silu_pair(c.y);
    c.z = silu_pair(c.z);
    c.w = silu_pair(c.w);
    __builtin_nontemporal_store(c, ys + j);
  }
}

// Chunk-per-lane counts that are instantiated, per waves-per-row.
template <int WPR, int OP>
hipError_t launch_rows(const uint16_t *x, void *out, float *scale, int64_t M,
                       int K, int ch, hipStream_t stream) {
  constexpr int RPB = kWaves / WPR;
  const dim3 grid((unsigned)((M + RPB - 1) / RPB));
#define W8A8_ROW_CASE(C)                                                  \
  if (ch <= C) {                                                          \
    hipLaunchKernelGGL((row_kernel<C, WPR, OP>), grid, dim3(kThreads), 0, \
                       stream, x, out, scale, M, K);                      \
    return hipGetLastError();                                             \
  }
  W8A8_ROW_CASE(1)
  W8A8_ROW_CASE(2)
  W8A8_ROW_CASE(3)
  W8A8_ROW_CASE(4)
  W8A8_ROW_CASE(6)
  W8A8_ROW_CASE(8)
  W8A8_ROW_CASE(11)
  if constexpr (WPR > 1) {
    W8A8_ROW_CASE(16)
    W8A8_ROW_CASE(22)
    W8A8_ROW_CASE(33)
    W8A8_ROW_CASE(44)
  }
#undef W8A8_ROW_CASE
  return hipErrorInvalidValue;
}

template <int OP>
hipError_t launch_row_op(const uint16_t *x, void *out, float *scale,
                         int64_t M, int64_t K, hipStream_t stream) {
  const int chunks = (int)(K / 8);
  if (chunks <= 11 * 64) {
    const int ch = (chunks + 63) / 64;
    return launch_rows<1, OP>(x, out, scale, M, (int)K, ch, stream);
  }
  const int ch = (chunks + 4 * 64 - 1) / (4 * 64);
  return launch_rows<4, OP>(x, out, scale, M, (int)K, ch, stream);
}

}  // namespace

hipError_t launch_quantize_act(const uint16_t *x, int8_t *q, float *sa,
                               int64_t M, int64_t K, bool fuse_silu,
                               hipStream_t stream) {
  if (fuse_silu)
    return launch_row_op<OP_QUANT_SILU>(x, q, sa, M, K, stream);
  return launch_row_op<OP_QUANT>(x, q, sa, M, K, stream);
}

hipError_t launch_pow2_renorm(const uint16_t *x, uint16_t *y, int64_t M,
                              int64_t K, hipStream_t stream) {
  return launch_row_op<OP_RENORM>(x, y, nullptr, M, K, stream);
}

hipError_t launch_silu(const uint16_t *x, uint16_t *y, int64_t n,
                       hipStream_t stream) {
  const int64_t chunks = n / 8;
  if (chunks == 0) return hipSuccess;
  int64_t blocks = (chunks + kThreads - 1) / kThreads;
  if (blocks > 256 * 16) blocks = 256 * 16;  // grid-stride beyond 16 per CU
  hipLaunchKernelGGL(silu_kernel, dim3((unsigned)blocks), dim3(kThreads), 0,
                     stream, x, y, chunks);
  return hipGetLastError();
}

}  // namespace w8a8
