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
//
// SiLU kernels: a BF16 input has only 65536 bit patterns, so SiLU is a table
// lookup.  The table (128 KiB) is built in device memory by a small kernel
// that evaluates the correctly rounded SiLU of every pattern, enqueued on
// the caller's stream ahead of each SiLU kernel (so it is always complete
// when read; a concurrent rebuild on another stream writes the same bits).
// The SiLU kernels keep one work group per CU, copy the table into LDS once
// and then stream rows (or chunks) through it: two LDS reads and a few
// integer operations per pair of values replace the exp / reciprocal
// evaluation.
#include "internal.h"
#include "rowwise.h"

#include <mutex>
#include <unordered_map>

namespace w8a8 {
namespace {

typedef unsigned v4u __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;  // 4 waves of 64
constexpr int kWaves = kThreads / 64;

// OP_QUANT_W: per-output-channel weight rows; an all-zero row takes scale 1.
// OP_RENORM_QUANT: the power-of-two renormalization written to `aux`, and
// the per-token quantization of that renormalized row, in one pass.
enum RowOp : int {
  OP_QUANT = 0,
  OP_RENORM = 2,
  OP_QUANT_W = 3,
  OP_RENORM_QUANT = 4
};

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
// The closeness test runs on the four values together; in the rare group
// where one is close to a half-integer (or the row needs the exact path),
// every code of the group comes from the division.
__device__ __forceinline__ uint32_t quant4(uint32_t p01, uint32_t p23,
                                           const QuantRow &R) {
  const float f[4] = {bf16_to_f32(p01 & 0xFFFFu), bf16_to_f32(p01 >> 16),
                      bf16_to_f32(p23 & 0xFFFFu), bf16_to_f32(p23 >> 16)};
  float u[4], d[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    u[e] = fmaf(f[e], R.r, 128.0f);
    d[e] = fabsf(__builtin_amdgcn_fractf(u[e]) - 0.5f);
  }
  const float dmin = fminf(fminf(d[0], d[1]), fminf(d[2], d[3]));
  if (!R.fast || !(dmin > 0x1p-14f)) {
#pragma unroll
    for (int e = 0; e < 4; ++e) u[e] = quant_biased_exact(f[e], R.s);
  }
  uint32_t out = 0;
#pragma unroll
  for (int e = 0; e < 4; ++e)  // nearest integer in [0, 255] as byte e
    out = __builtin_amdgcn_cvt_pk_u8_f32(u[e], e, out);
  return out ^ 0x80808080u;  // biased byte -> two's complement code
}

// Row maximum of |x| on the BF16 bit patterns: for finite values the
// magnitude bits (sign cleared) order like the magnitudes, so a packed
// 16-bit unsigned max over two values per dword finds the largest |x|
// exactly; the two halves are merged once per row.
typedef unsigned short us2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ us2 mag_max4(us2 m, v4u c) {
  const uint32_t k = 0x7FFF7FFFu;
  const us2 a = __builtin_bit_cast(us2, c.x & k);
  const us2 b = __builtin_bit_cast(us2, c.y & k);
  const us2 d = __builtin_bit_cast(us2, c.z & k);
  const us2 e = __builtin_bit_cast(us2, c.w & k);
  return __builtin_elementwise_max(
      __builtin_elementwise_max(m, a),
      __builtin_elementwise_max(__builtin_elementwise_max(b, d), e));
}

__device__ __forceinline__ float mag_to_f32(us2 m) {
  const uint32_t hi = m.x > m.y ? m.x : m.y;
  return __uint_as_float(hi << 16);
}

__device__ __forceinline__ uint32_t renorm_pair(uint32_t packed, int e) {
  float f0 = ldexpf(bf16_to_f32(packed & 0xFFFFu), -e);
  float f1 = ldexpf(bf16_to_f32(packed >> 16), -e);
  return f32_to_bf16_rne(f0) | (f32_to_bf16_rne(f1) << 16);
}

template <int CH, int WPR, int OP>
__global__ __launch_bounds__(kThreads) void row_kernel(
    const uint16_t *x, void *out, float *__restrict__ scale, int64_t M,
    int K, uint16_t *aux) {
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
  us2 mag = us2{0, 0};
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    const int j = (i * WPR + part) * 64 + lane;
    v[i] = v4u{0, 0, 0, 0};
    if (row_ok && j < chunks) v[i] = __builtin_nontemporal_load(xr + j);
    mag = mag_max4(mag, v[i]);  // masked chunks are zero
  }
  float amax = wave_max(mag_to_f32(mag));
  if (WPR > 1) {
    if (lane == 0) part_max[wave] = amax;
    __syncthreads();
    const int base = (wave / WPR) * WPR;
    amax = part_max[base];
#pragma unroll
    for (int p = 1; p < WPR; ++p) amax = fmaxf(amax, part_max[base + p]);
  }
  if (OP == OP_RENORM_QUANT) {
    // Renormalize in registers, then take the row maximum again from the
    // renormalized BF16 values, so the codes and scale are exactly those a
    // separate quantization of the written row computes.
    int ex = 0;
    frexpf(amax, &ex);
    const int e = (amax == 0.0f) ? 0 : ex - 1;
    us2 mag2 = us2{0, 0};
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      v4u c = v[i];  // masked chunks are zero and stay zero
      c.x = renorm_pair(c.x, e);
      c.y = renorm_pair(c.y, e);
      c.z = renorm_pair(c.z, e);
      c.w = renorm_pair(c.w, e);
      v[i] = c;
      mag2 = mag_max4(mag2, c);
    }
    amax = wave_max(mag_to_f32(mag2));
    if (WPR > 1) {
      __syncthreads();  // every wave has read the first exchange
      if (lane == 0) part_max[wave] = amax;
      __syncthreads();
      const int base = (wave / WPR) * WPR;
      amax = part_max[base];
#pragma unroll
      for (int p = 1; p < WPR; ++p) amax = fmaxf(amax, part_max[base + p]);
    }
    if (!row_ok) return;
    v4u *yr = reinterpret_cast<v4u *>(aux + row * (int64_t)K);
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int j = (i * WPR + part) * 64 + lane;
      if (j < chunks) __builtin_nontemporal_store(v[i], yr + j);
    }
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

  // Quantize: scale = amax / 127 (IEEE division), zero row -> scale 0
  // (activations) or 1 (weights, whose scales must be positive).
  const QuantRow R = quant_row(amax);
  const float s = R.s;
  if (lane == 0 && part == 0)
    scale[row] = (OP == OP_QUANT_W && s == 0.0f) ? 1.0f : s;
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

// Quantization of rows longer than the register-resident kernel holds
// (K > 90112, up to the GEMM's INT32 bound): one work group per row reads
// the row twice, first for its maximum and then for the codes, with the
// same arithmetic as row_kernel.
template <int OP>
__global__ __launch_bounds__(kThreads) void long_row_quant_kernel(
    const uint16_t *x, int8_t *q, float *__restrict__ scale, int K) {
  __shared__ float part_max[kWaves];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t row = blockIdx.x;
  const int chunks = K >> 3;
  const v4u *xr = reinterpret_cast<const v4u *>(x + row * (int64_t)K);
  us2 mag = us2{0, 0};
  for (int j = threadIdx.x; j < chunks; j += kThreads)
    mag = mag_max4(mag, xr[j]);
  float amax = wave_max(mag_to_f32(mag));
  if (lane == 0) part_max[wave] = amax;
  __syncthreads();
  amax = part_max[0];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) amax = fmaxf(amax, part_max[w]);
  const QuantRow R = quant_row(amax);
  if (threadIdx.x == 0)
    scale[row] = (OP == OP_QUANT_W && R.s == 0.0f) ? 1.0f : R.s;
  uint2 *qr = reinterpret_cast<uint2 *>(q + row * (int64_t)K);
  for (int j = threadIdx.x; j < chunks; j += kThreads) {
    uint2 o = make_uint2(0, 0);
    if (R.s != 0.0f) {
      const v4u c = xr[j];  // the second read of the row, likely cached
      o.x = quant4(c.x, c.y, R);
      o.y = quant4(c.z, c.w, R);
    }
    qr[j] = o;
  }
}

// ---------------------------------------------------------------------------
// SiLU through a lookup table
// ---------------------------------------------------------------------------

constexpr int kLutEntries = 65536;
constexpr int kLutThreads = 1024;  // 16 waves, one work group per CU
constexpr int kLutWaves = kLutThreads / 64;

// SiLU of BF16 bit pattern i in the low (i even) or high (i odd) half of
// dword i / 2.
__device__ uint32_t g_silu_lut[kLutEntries / 2];

__global__ __launch_bounds__(256) void silu_lut_build_kernel() {
  const uint32_t i = blockIdx.x * 256 + threadIdx.x;  // pair index
  g_silu_lut[i] = silu_bf16x2((2 * i) | ((2 * i + 1) << 16));
}

// Copy the table into this work group's LDS.
__device__ __forceinline__ void lut_to_lds(uint32_t *lut) {
  const v4u *src = reinterpret_cast<const v4u *>(g_silu_lut);
  v4u *dst = reinterpret_cast<v4u *>(lut);
  for (int i = threadIdx.x; i < kLutEntries / 8; i += blockDim.x)
    dst[i] = src[i];
  __syncthreads();
}

__device__ __forceinline__ uint32_t silu_lut_pair(const uint16_t *lut,
                                                  uint32_t p) {
  return (uint32_t)lut[p & 0xFFFFu] | ((uint32_t)lut[p >> 16] << 16);
}

__device__ __forceinline__ v4u silu_lut_chunk(const uint16_t *lut, v4u c) {
  return v4u{silu_lut_pair(lut, c.x), silu_lut_pair(lut, c.y),
             silu_lut_pair(lut, c.z), silu_lut_pair(lut, c.w)};
}

// Gated form (SwiGLU): BF16(silu(g)) from the table times the up value u;
// both are BF16, so the binary32 product is exact and v_cvt_pk_bf16_f32
// rounds it once (a product too small for binary32's normal range lies
// below half the smallest BF16 subnormal unless it is exact, so it still
// rounds as the exact value would).
__device__ __forceinline__ uint32_t swiglu_pair(const uint16_t *lut,
                                                uint32_t g, uint32_t u) {
  const uint32_t s = silu_lut_pair(lut, g);
  return pack_bf16x2(bf16_to_f32(s & 0xFFFFu) * bf16_to_f32(u & 0xFFFFu),
                     bf16_to_f32(s >> 16) * bf16_to_f32(u >> 16));
}

__device__ __forceinline__ v4u swiglu_chunk(const uint16_t *lut, v4u g,
                                            v4u u) {
  return v4u{swiglu_pair(lut, g.x, u.x), swiglu_pair(lut, g.y, u.y),
             swiglu_pair(lut, g.z, u.z), swiglu_pair(lut, g.w, u.w)};
}

// SiLU (or, GATED, SwiGLU over rows of gate | up, 2K wide) + per-token
// quantization of the K results.  The whole work group owns one row at a
// time (chunk j of the row is held by thread j mod 1024, CH chunks per
// thread) and loads the following rows while it quantizes the current one.
template <int CH, bool GATED>
__global__ __launch_bounds__(kLutThreads, 1) void silu_quant_lut_kernel(
    const uint16_t *x, int8_t *q, float *__restrict__ scale, int64_t M,
    int K) {
  __shared__ uint32_t lut32[kLutEntries / 2];
  __shared__ float part_max[2][kLutWaves];
  lut_to_lds(lut32);
  const uint16_t *lut = reinterpret_cast<const uint16_t *>(lut32);
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int chunks = K >> 3;

  // Buffer b holds the row's chunks; with GATED, b[CH + i] is the up half
  // of chunk i.
  constexpr int NB = GATED ? 2 * CH : CH;
  const int64_t stride = GATED ? 2 * (int64_t)K : K;
  auto load_row = [&](int64_t row, v4u *v) {
    const v4u *xr = reinterpret_cast<const v4u *>(x + row * stride);
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int j = i * kLutThreads + threadIdx.x;
      v[i] = v4u{0, 0, 0, 0};
      if (GATED) v[CH + i] = v4u{0, 0, 0, 0};
      if (row < M && j < chunks) {
        v[i] = __builtin_nontemporal_load(xr + j);
        if (GATED) v[CH + i] = __builtin_nontemporal_load(xr + chunks + j);
      }
    }
  };

  // Rows loaded ahead of the one being quantized: two while three row
  // buffers fit in registers, else one, else none.  With one work group per
  // CU, the loads in flight per CU are what keeps HBM busy.
  constexpr int kDepth = NB <= 4 ? 2 : (NB <= 6 ? 1 : 0);
  v4u cur[NB], nxt[kDepth >= 1 ? NB : 1], nxt2[kDepth >= 2 ? NB : 1];
  int64_t row = blockIdx.x;
  const int64_t g = gridDim.x;
  if (kDepth >= 1) load_row(row, cur);
  if (kDepth >= 2) load_row(row + g, nxt);  // rows past M load nothing
  for (int it = 0; row < M; ++it, row += g) {
    if (kDepth == 2)
      load_row(row + 2 * g, nxt2);
    else if (kDepth == 1)
      load_row(row + g, nxt);
    else
      load_row(row, cur);
    us2 mag = us2{0, 0};
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      // zero chunks map to zero
      const v4u c = GATED ? swiglu_chunk(lut, cur[i], cur[CH + i])
                          : silu_lut_chunk(lut, cur[i]);
      cur[i] = c;
      mag = mag_max4(mag, c);
    }
    float amax = wave_max(mag_to_f32(mag));
    if (lane == 0) part_max[it & 1][wave] = amax;
    __syncthreads();
    amax = part_max[it & 1][0];
#pragma unroll
    for (int w = 1; w < kLutWaves; ++w) amax = fmaxf(amax, part_max[it & 1][w]);

    const QuantRow R = quant_row(amax);
    if (threadIdx.x == 0) scale[row] = R.s;
    uint2 *qr = reinterpret_cast<uint2 *>(q + row * (int64_t)K);
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int j = i * kLutThreads + threadIdx.x;
      if (j < chunks) {
        uint2 o = make_uint2(0, 0);
        if (R.s != 0.0f) {
          o.x = quant4(cur[i].x, cur[i].y, R);
          o.y = quant4(cur[i].z, cur[i].w, R);
        }
        qr[j] = o;
      }
    }
    if (kDepth >= 1) {
#pragma unroll
      for (int i = 0; i < NB; ++i) cur[i] = nxt[kDepth >= 1 ? i : 0];
    }
    if (kDepth >= 2) {
#pragma unroll
      for (int i = 0; i < NB; ++i) nxt[i] = nxt2[kDepth >= 2 ? i : 0];
    }
  }
}

// SwiGLU alone: chunk c of the output (row c / (F/8)) from the gate and up
// chunks of its row.
__global__ __launch_bounds__(kLutThreads, 1) void swiglu_lut_kernel(
    const uint16_t *h, uint16_t *y, int64_t M, int64_t F) {
  __shared__ uint32_t lut32[kLutEntries / 2];
  lut_to_lds(lut32);
  const uint16_t *lut = reinterpret_cast<const uint16_t *>(lut32);
  const int64_t cpr = F / 8;  // output chunks per row
  const v4u *hs = reinterpret_cast<const v4u *>(h);
  v4u *ys = reinterpret_cast<v4u *>(y);
  for (int64_t c = (int64_t)blockIdx.x * kLutThreads + threadIdx.x;
       c < M * cpr; c += (int64_t)gridDim.x * kLutThreads) {
    const int64_t row = c / cpr, j = c - row * cpr;
    const v4u g = __builtin_nontemporal_load(hs + row * 2 * cpr + j);
    const v4u u = __builtin_nontemporal_load(hs + row * 2 * cpr + cpr + j);
    __builtin_nontemporal_store(swiglu_chunk(lut, g, u), ys + c);
  }
}

// Number of scales that are not finite and > 0 (one work group).
__global__ __launch_bounds__(1024) void check_scales_kernel(
    const float *sw, int64_t N, int *bad) {
  __shared__ int part[16];
  int count = 0;
  for (int64_t n = threadIdx.x; n < N; n += 1024) {
    const float v = sw[n];
    count += (v > 0.0f && v <= 0x1.fffffep127f) ? 0 : 1;  // NaN fails both
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) count += __shfl_xor(count, off, 64);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = count;
  __syncthreads();
  if (threadIdx.x == 0) {
    int total = 0;
#pragma unroll
    for (int w = 0; w < 16; ++w) total += part[w];
    *bad = total;
  }
}

__global__ __launch_bounds__(kLutThreads, 1) void silu_lut_kernel(
    const uint16_t *x, uint16_t *y, int64_t chunks) {
  __shared__ uint32_t lut32[kLutEntries / 2];
  lut_to_lds(lut32);
  const uint16_t *lut = reinterpret_cast<const uint16_t *>(lut32);
  const v4u *xs = reinterpret_cast<const v4u *>(x);
  v4u *ys = reinterpret_cast<v4u *>(y);
  for (int64_t j = (int64_t)blockIdx.x * kLutThreads + threadIdx.x;
       j < chunks; j += (int64_t)gridDim.x * kLutThreads)
    __builtin_nontemporal_store(
        silu_lut_chunk(lut, __builtin_nontemporal_load(xs + j)), ys + j);
}

// Compute units of the current device (cached per device).
int cu_count() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  static std::mutex mu;
  static std::unordered_map<int, int> cache;
  std::lock_guard<std::mutex> lock(mu);
  auto it = cache.find(dev);
  if (it != cache.end()) return it->second;
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) !=
          hipSuccess || n <= 0)
    n = 256;
  cache[dev] = n;
  return n;
}

hipError_t build_silu_lut(hipStream_t stream) {
  hipLaunchKernelGGL(silu_lut_build_kernel, dim3(kLutEntries / 2 / 256),
                     dim3(256), 0, stream);
  return hipGetLastError();
}

// SwiGLU + quantization: h [M, 2F] -> codes [M, F].
hipError_t launch_swiglu_quant_impl(const uint16_t *h, int8_t *q,
                                    float *scale, int64_t M, int64_t F,
                                    hipStream_t stream) {
  hipError_t e = build_silu_lut(stream);
  if (e != hipSuccess) return e;
  const int chunks = (int)(F / 8);
  const int ch = (chunks + kLutThreads - 1) / kLutThreads;
  const dim3 grid((unsigned)(M < cu_count() ? M : cu_count()));
#define W8A8_GLU_CASE(C)                                                     \
  if (ch <= C) {                                                             \
    hipLaunchKernelGGL((silu_quant_lut_kernel<C, true>), grid,              \
                       dim3(kLutThreads), 0, stream, h, q, scale, M, (int)F); \
    return hipGetLastError();                                                \
  }
  W8A8_GLU_CASE(1)
  W8A8_GLU_CASE(2)
  W8A8_GLU_CASE(3)
  W8A8_GLU_CASE(4)
  W8A8_GLU_CASE(6)
  W8A8_GLU_CASE(8)
  W8A8_GLU_CASE(11)
#undef W8A8_GLU_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_silu_quant(const uint16_t *x, int8_t *q, float *scale,
                             int64_t M, int64_t K, hipStream_t stream) {
  hipError_t e = build_silu_lut(stream);
  if (e != hipSuccess) return e;
  const int chunks = (int)(K / 8);
  const int ch = (chunks + kLutThreads - 1) / kLutThreads;
  const dim3 grid((unsigned)(M < cu_count() ? M : cu_count()));
#define W8A8_LUT_CASE(C)                                                     \
  if (ch <= C) {                                                             \
    hipLaunchKernelGGL((silu_quant_lut_kernel<C, false>), grid,             \
                       dim3(kLutThreads), 0, stream, x, q, scale, M, (int)K); \
    return hipGetLastError();                                                \
  }
  W8A8_LUT_CASE(1)
  W8A8_LUT_CASE(2)
  W8A8_LUT_CASE(3)
  W8A8_LUT_CASE(4)
  W8A8_LUT_CASE(6)
  W8A8_LUT_CASE(8)
  W8A8_LUT_CASE(11)
#undef W8A8_LUT_CASE
  return hipErrorInvalidValue;
}

// Chunk-per-lane counts that are instantiated, per waves-per-row.
template <int WPR, int OP>
hipError_t launch_rows(const uint16_t *x, void *out, float *scale, int64_t M,
                       int K, int ch, hipStream_t stream, uint16_t *aux) {
  constexpr int RPB = kWaves / WPR;
  const dim3 grid((unsigned)((M + RPB - 1) / RPB));
#define W8A8_ROW_CASE(C)                                                  \
  if (ch <= C) {                                                          \
    hipLaunchKernelGGL((row_kernel<C, WPR, OP>), grid, dim3(kThreads), 0, \
                       stream, x, out, scale, M, K, aux);                 \
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
                         int64_t M, int64_t K, hipStream_t stream,
                         uint16_t *aux = nullptr) {
  const int chunks = (int)(K / 8);
  if constexpr (OP == OP_QUANT || OP == OP_QUANT_W) {
    if (chunks > 44 * 4 * 64) {
      hipLaunchKernelGGL((long_row_quant_kernel<OP>), dim3((unsigned)M),
                         dim3(kThreads), 0, stream, x,
                         static_cast<int8_t *>(out), scale, (int)K);
      return hipGetLastError();
    }
  }
  // One wave per row, or a row split over 2 or 4 waves of a work group
  // (their maxima meet in LDS).  Plain quantization splits rows of more
  // than 2 chunks per lane: more waves share a row's loads, which pays at
  // every token count (K = 5376: M = 64 4.2 against 10.0 us, M = 4096 15.4
  // against 19.1 us, M = 19077 52.7 against 56.3 us).  The renormalizing
  // kernels, which also write the BF16 row, measured no faster split and
  // keep one wave per row up to 11 chunks per lane.
  const bool split = (OP == OP_QUANT || OP == OP_QUANT_W) ? chunks > 2 * 64
                                                          : chunks > 11 * 64;
  if (!split) {
    const int ch = (chunks + 63) / 64;
    return launch_rows<1, OP>(x, out, scale, M, (int)K, ch, stream, aux);
  }
  // Many rows: two waves per row, two rows per work group, while a row
  // fits 44 chunks per lane (K = 5376: M = 19077 51.1 against 52.9 us,
  // M = 37503 93.5 against 99.2 us; at M = 4096 and below four waves per
  // row stay faster).
  if constexpr (OP == OP_QUANT || OP == OP_QUANT_W) {
    const int ch2 = (chunks + 2 * 64 - 1) / (2 * 64);
    if (M >= 8192 && ch2 <= 44)
      return launch_rows<2, OP>(x, out, scale, M, (int)K, ch2, stream, aux);
  }
  const int ch = (chunks + 4 * 64 - 1) / (4 * 64);
  return launch_rows<4, OP>(x, out, scale, M, (int)K, ch, stream, aux);
}

}  // namespace

hipError_t launch_quantize_act(const uint16_t *x, int8_t *q, float *sa,
                               int64_t M, int64_t K, bool fuse_silu,
                               hipStream_t stream) {
  if (fuse_silu) return launch_silu_quant(x, q, sa, M, K, stream);
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
  hipError_t e = build_silu_lut(stream);
  if (e != hipSuccess) return e;
  int64_t blocks = (chunks + kLutThreads - 1) / kLutThreads;
  if (blocks > cu_count()) blocks = cu_count();
  hipLaunchKernelGGL(silu_lut_kernel, dim3((unsigned)blocks),
                     dim3(kLutThreads), 0, stream, x, y, chunks);
  return hipGetLastError();
}

hipError_t launch_quantize_weight(const uint16_t *w, int8_t *q, float *sw,
                                  int64_t N, int64_t K, hipStream_t stream) {
  return launch_row_op<OP_QUANT_W>(w, q, sw, N, K, stream);
}

hipError_t launch_pow2_renorm_quant(const uint16_t *x, uint16_t *y, int8_t *q,
                                    float *sa, int64_t M, int64_t K,
                                    hipStream_t stream) {
  return launch_row_op<OP_RENORM_QUANT>(x, q, sa, M, K, stream, y);
}

hipError_t launch_check_scales(const float *sw, int64_t N, int *bad,
                               hipStream_t stream) {
  hipLaunchKernelGGL(check_scales_kernel, dim3(1), dim3(1024), 0, stream, sw,
                     N, bad);
  return hipGetLastError();
}

hipError_t launch_swiglu(const uint16_t *h, uint16_t *y, int64_t M, int64_t F,
                         hipStream_t stream) {
  hipError_t e = build_silu_lut(stream);
  if (e != hipSuccess) return e;
  const int64_t chunks = M * (F / 8);
  int64_t blocks = (chunks + kLutThreads - 1) / kLutThreads;
  if (blocks > cu_count()) blocks = cu_count();
  hipLaunchKernelGGL(swiglu_lut_kernel, dim3((unsigned)blocks),
                     dim3(kLutThreads), 0, stream, h, y, M, F);
  return hipGetLastError();
}

hipError_t launch_swiglu_quant(const uint16_t *h, int8_t *q, float *scale,
                               int64_t M, int64_t F, hipStream_t stream) {
  return launch_swiglu_quant_impl(h, q, scale, M, F, stream);
}

}  // namespace w8a8
