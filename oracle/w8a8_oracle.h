/*
 * w8a8_oracle.h -- plain CPU reference of the W8A8 INT8 projection.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library includes,
 * links or calls this file; only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark load the shared object built from
 * w8a8_oracle.c.  It shares no code, header, table or constant with the
 * HIP path.
 *
 * What is computed, and where the pages state it:
 *   - "feat(mps): support MiniMax-H3 INT8 inference on Apple M5"
 *     (LightX2V pull request #1672), description and commit notes: W8A8
 *     projections run at the native hidden width with no K padding and no
 *     weight dequantization; activations are quantized per token and the
 *     quantizer masks partial chunks when K is not a multiple of its chunk
 *     width; weights are INT8 with one finite positive FP32 scale per
 *     output row ("Validation", "Changes" table).
 *   - "MLX implementation and experiment report" (MiniMax-H3-Image-mlx),
 *     section "What the default preserves": a biased BF16 linear adds the
 *     bias inside the epilogue, before the single rounding to BF16.
 *
 * Every function is row-parallel (OpenMP over rows) and otherwise a
 * literal evaluation of its definition.  All floating point is IEEE
 * binary32 where the method fixes FP32 (scales, epilogue), binary64 for
 * the harness glue whose precision the pages leave open.
 *
 * Return codes (the oracle's own; unrelated to the library's codes):
 *   0  success
 *   1  a required pointer is NULL
 *   2  a size is out of range (M, N, K < 1, or n < 0)
 *   3  a non-finite activation (NaN or Inf) was found
 *   4  a weight scale is not finite or not > 0
 *   5  an accumulator left the INT32 range
 */
#ifndef W8A8_ORACLE_H
#define W8A8_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* BF16 bits -> binary32 (exact). */
float orc_bf16_to_f32(uint16_t b);
/* binary32 -> BF16 bits, round to nearest, ties to even; NaN -> quiet NaN. */
uint16_t orc_f32_to_bf16(float f);
/* binary64 -> BF16 bits with a single round-to-nearest-even. */
uint16_t orc_f64_to_bf16(double d);

/* Per-token symmetric quantization.  x: BF16 [M,K] row-major.
 * q: INT8 [M,K]; sa: FP32 [M].  sa = amax/127 (binary32 division);
 * q = clamp(round_half_even(x / sa), -127, 127); an all-zero row gives
 * sa = 0 and q = 0. */
int orc_quantize_act(const uint16_t *x, int64_t M, int64_t K,
                     int8_t *q, float *sa);

/* Per-output-channel weight quantization: each row of w (BF16 [N,K], one
 * row per output channel) is quantized like an activation row; an all-zero
 * row gets codes 0 and scale 1 (scales must be finite and positive). */
int orc_quantize_weight(const uint16_t *w, int64_t N, int64_t K,
                        int8_t *q, float *sw);

/* *bad = number of scales that are not finite and > 0. */
int orc_check_scales(const float *sw, int64_t N, int64_t *bad);

/* acc[m,n] = sum_k a[m,k] * w[n,k], exact, stored as INT32.
 * a: INT8 [M,K]; w: INT8 [N,K] (a Linear's stored layout). */
int orc_gemm_i32(const int8_t *a, const int8_t *w, int64_t M, int64_t N,
                 int64_t K, int32_t *acc);

/* t = ((float)acc[m,n] * sa[m]) * sw[n] (+ bf16->f32(bias[n])), each
 * operation rounded in binary32, no fused multiply-add.  y_f32 receives t
 * and y_bf16 receives its one BF16 rounding; either may be NULL, bias may
 * be NULL (no add). */
int orc_epilogue(const int32_t *acc, const float *sa, const float *sw,
                 const uint16_t *bias, int64_t M, int64_t N,
                 float *y_f32, uint16_t *y_bf16);

/* quantize -> gemm -> epilogue, BF16 output. */
int orc_linear(const uint16_t *x, const int8_t *w, const float *sw,
               const uint16_t *bias, int64_t M, int64_t N, int64_t K,
               uint16_t *y);

/* Harness glue between FC1 and FC2: y = x / (1 + exp(-x)) evaluated in
 * binary64 and rounded once to BF16.  n elements. */
int orc_silu_bf16(const uint16_t *x, int64_t n, uint16_t *y);

/* Gated MLP glue (fused gate/up projection, width 2F per token): the
 * first F values of a row are the gate g, the next F the up value u;
 * y = BF16(BF16(silu(g)) * u): SiLU rounded once to BF16 as above, then
 * the product rounded once to BF16.  h: BF16 [M, 2F]; y: BF16 [M, F]. */
int orc_swiglu_bf16(const uint16_t *h, int64_t M, int64_t F, uint16_t *y);

/* Harness glue between blocks: each row is scaled by 2^-e with
 * e = floor(log2(max_k |x[m,k]|)) so that its largest magnitude lies in
 * [1, 2); the product is rounded once to BF16.  All-zero rows are copied. */
int orc_pow2_renorm(const uint16_t *x, int64_t M, int64_t K, uint16_t *y);

/* Number of OpenMP threads a parallel region of the oracle uses. */
int orc_num_threads(void);

#ifdef __cplusplus
}
#endif

#endif /* W8A8_ORACLE_H */
