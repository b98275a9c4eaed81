// mfma_ceiling.hip -- measurement support, not part of the W8A8 library:
// the sustained rate of v_mfma_i32_32x32x32_i8 with register operands only
// (no memory traffic inside the timed loop), fed the workload's own INT8
// codes and weights.
//
// The matrix cores' energy per instruction grows with how many operand bits
// switch, and the board caps its power, so the rate an MFMA-bound kernel can
// reach depends on the data it multiplies.  This kernel gives that ceiling
// for a given pair of code matrices: every wave of 8 per CU (two per SIMD,
// as in the GEMM) holds 4 k-steps of 2 token fragments and 4 weight
// fragments, taken from the matrices in the GEMM's fragment layout, and
// issues the GEMM's MFMA sequence over them for `iters` rounds.
//
// Built as its own shared object (libw8a8_ceiling.so); only bench.py loads it.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int kThreads = 512;  // 8 waves
constexpr int kTM = 2, kTN = 4, kKS = 4;

// Lane l of a fragment holds 16 bytes of row (l mod 32) of a 32-row block:
// bytes [32 ks + 16 (l / 32), +16) of that row.
__device__ __forceinline__ v4i frag(const int8_t *m, int64_t ld, int row0,
                                    int ks, int lane) {
  return *reinterpret_cast<const v4i *>(m + (int64_t)(row0 + (lane & 31)) * ld +
                                        ks * 32 + (lane >> 5) * 16);
}

__global__ __launch_bounds__(kThreads, 1) void mfma_ceiling_kernel(
    const int8_t *x, int x_blocks, const int8_t *w, int w_blocks, int K,
    int iters, int *out) {
  const int lane = threadIdx.x & 63;
  const int gw = blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  v4i xa[kKS][kTM], wb[kKS][kTN];
#pragma unroll
  for (int ks = 0; ks < kKS; ++ks) {
#pragma unroll
    for (int j = 0; j < kTM; ++j)
      xa[ks][j] = frag(x, K, ((gw * kTM + j) % x_blocks) * 32, ks, lane);
#pragma unroll
    for (int i = 0; i < kTN; ++i)
      wb[ks][i] = frag(w, K, ((gw * kTN + i) % w_blocks) * 32, ks, lane);
  }
  v16i acc[kTN][kTM];
#pragma unroll
  for (int i = 0; i < kTN; ++i)
#pragma unroll
    for (int j = 0; j < kTM; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int ks = 0; ks < kKS; ++ks)
#pragma unroll
      for (int i = 0; i < kTN; ++i)
#pragma unroll
        for (int j = 0; j < kTM; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(
              wb[ks][i], xa[ks][j], acc[i][j], 0, 0, 0);
  }
  // Keep every accumulator live: one sum per lane (wrapping is harmless).
  int s = 0;
#pragma unroll
  for (int i = 0; i < kTN; ++i)
#pragma unroll
    for (int j = 0; j < kTM; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) s += acc[i][j][e];
  out[(int64_t)blockIdx.x * kThreads + threadIdx.x] = s;
}

}  // namespace

extern "C" {

// Integer operations one launch performs: blocks x 8 waves x iters x 32
// MFMAs x 65536.
double w8a8_ceiling_ops(int blocks, int iters) {
  return (double)blocks * (kThreads / 64) * iters * (kKS * kTN * kTM) *
         (2.0 * 32 * 32 * 32);
}

// Ints `out` must hold.
int64_t w8a8_ceiling_out_len(int blocks) { return (int64_t)blocks * kThreads; }

// x: token codes [x_rows, K], w: weights [w_rows, K], both row-major INT8 on
// the device, 16-byte aligned; out: int32 [w8a8_ceiling_out_len(blocks)].
// Returns 0, or 1 for an argument the kernel cannot take (rows < 32, K < 128
// or not a multiple of 16, non-positive counts, null pointers), or 2 when
// the launch fails.  Asynchronous on `stream`.
int w8a8_ceiling_run(const int8_t *x, int64_t x_rows, const int8_t *w,
                     int64_t w_rows, int64_t K, int blocks, int iters,
                     int *out, void *stream) {
  if (!x || !w || !out || x_rows < 32 || w_rows < 32 || K < 128 ||
      K % 16 != 0 || K > 0x7fffffff || blocks <= 0 || iters <= 0)
    return 1;
  const int xb = (int)(x_rows / 32 > 0x7fffffff ? 0x7fffffff : x_rows / 32);
  const int wb = (int)(w_rows / 32 > 0x7fffffff ? 0x7fffffff : w_rows / 32);
  hipLaunchKernelGGL(mfma_ceiling_kernel, dim3((unsigned)blocks),
                     dim3(kThreads), 0, (hipStream_t)stream, x, xb, w, wb,
                     (int)K, iters, out);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

}  // extern "C"
