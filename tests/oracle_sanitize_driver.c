/*
 * oracle_sanitize_driver.c -- runs every entry point of the CPU oracle on
 * exactly sized heap buffers, so that a build with AddressSanitizer and
 * UndefinedBehaviorSanitizer reports any out-of-bounds access, overflow or
 * other undefined behaviour (test infrastructure; built and run by
 * tests/test_oracle_sanitized.py).  Shapes include single rows, ragged
 * widths, zero rows, subnormal and signed-zero inputs and every error
 * path.  A few results are also checked against brute force.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "w8a8_oracle.h"

static int failures = 0;

#define EXPECT(cond)                                                  \
  do {                                                                \
    if (!(cond)) {                                                    \
      fprintf(stderr, "%s:%d: expectation failed: %s\n", __FILE__,    \
              __LINE__, #cond);                                       \
      ++failures;                                                     \
    }                                                                 \
  } while (0)

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static uint32_t next_u32(void) {  /* xorshift64* */
  rng_state ^= rng_state >> 12;
  rng_state ^= rng_state << 25;
  rng_state ^= rng_state >> 27;
  return (uint32_t)((rng_state * 0x2545F4914F6CDD1Dull) >> 32);
}

static uint16_t bf16_of(float f) { return orc_f32_to_bf16(f); }

/* Finite BF16 values of a few magnitudes, with subnormals and -0. */
static uint16_t random_bf16(void) {
  uint32_t r = next_u32();
  switch (r & 7u) {
    case 0: return (uint16_t)(r >> 16) & 0x007Fu;           /* subnormal */
    case 1: return 0x8000u;                                  /* -0 */
    default: {
      float v = ((float)(int)(r >> 8 & 0xFFFF) - 32768.0f) / 1024.0f;
      return bf16_of(v);
    }
  }
}

static void *xmalloc(size_t n) {
  void *p = malloc(n ? n : 1);
  if (!p) {
    fprintf(stderr, "out of memory\n");
    exit(2);
  }
  return p;
}

static void check_quant_and_linear(int64_t M, int64_t N, int64_t K) {
  uint16_t *x = xmalloc((size_t)(M * K) * sizeof *x);
  int8_t *q = xmalloc((size_t)(M * K));
  float *sa = xmalloc((size_t)M * sizeof *sa);
  int8_t *w = xmalloc((size_t)(N * K));
  float *sw = xmalloc((size_t)N * sizeof *sw);
  uint16_t *bias = xmalloc((size_t)N * sizeof *bias);
  int32_t *acc = xmalloc((size_t)(M * N) * sizeof *acc);
  float *yf = xmalloc((size_t)(M * N) * sizeof *yf);
  uint16_t *yb = xmalloc((size_t)(M * N) * sizeof *yb);
  uint16_t *y = xmalloc((size_t)(M * N) * sizeof *y);
  for (int64_t i = 0; i < M * K; ++i) x[i] = random_bf16();
  if (M > 1)
    for (int64_t k = 0; k < K; ++k) x[K + k] = 0; /* an all-zero row */
  for (int64_t i = 0; i < N * K; ++i) w[i] = (int8_t)(next_u32() & 0xFF);
  for (int64_t n = 0; n < N; ++n) {
    sw[n] = ldexpf(1.0f + (float)(next_u32() & 0xFF) / 256.0f, -8);
    bias[n] = random_bf16();
  }
  EXPECT(orc_quantize_act(x, M, K, q, sa) == 0);
  EXPECT(orc_gemm_i32(q, w, M, N, K, acc) == 0);
  for (int64_t m = 0; m < M; ++m)
    for (int64_t n = 0; n < N; ++n) {
      int64_t s = 0;
      for (int64_t k = 0; k < K; ++k) s += (int64_t)q[m * K + k] * w[n * K + k];
      EXPECT(acc[m * N + n] == (int32_t)s);
    }
  EXPECT(orc_epilogue(acc, sa, sw, bias, M, N, yf, yb) == 0);
  EXPECT(orc_epilogue(acc, sa, sw, NULL, M, N, NULL, yb) == 0);
  EXPECT(orc_epilogue(acc, sa, sw, bias, M, N, yf, NULL) == 0);
  EXPECT(orc_linear(x, w, sw, bias, M, N, K, y) == 0);
  EXPECT(orc_linear(x, w, sw, NULL, M, N, K, y) == 0);
  EXPECT(orc_quantize_weight(x, M, K, q, sa) == 0);
  if (M > 1) EXPECT(sa[1] == 1.0f); /* all-zero weight row: scale 1 */
  uint16_t *r = xmalloc((size_t)(M * K) * sizeof *r);
  EXPECT(orc_pow2_renorm(x, M, K, r) == 0);
  if (K % 2 == 0) {
    uint16_t *g = xmalloc((size_t)(M * K / 2) * sizeof *g);
    EXPECT(orc_swiglu_bf16(x, M, K / 2, g) == 0);
    free(g);
  }
  free(r);
  free(x); free(q); free(sa); free(w); free(sw); free(bias);
  free(acc); free(yf); free(yb); free(y);
}

static void check_glue_and_conversions(void) {
  /* SiLU over every finite BF16 input */
  uint16_t *in = xmalloc(65536 * sizeof *in), *out = xmalloc(65536 * sizeof *out);
  int64_t n = 0;
  for (uint32_t b = 0; b < 65536; ++b)
    if (((b >> 7) & 0xFFu) != 0xFFu) in[n++] = (uint16_t)b;
  EXPECT(orc_silu_bf16(in, n, out) == 0);
  EXPECT(orc_silu_bf16(in, 0, out) == 0);
  free(in);
  free(out);
  const float f32s[] = {0.0f, -0.0f, 1.0f, 0x1p-149f, 0x1.fffffep127f,
                        -0x1p-126f, 257.0f, INFINITY, NAN};
  for (size_t i = 0; i < sizeof f32s / sizeof *f32s; ++i) {
    (void)orc_f32_to_bf16(f32s[i]);
    (void)orc_f64_to_bf16((double)f32s[i]);
  }
  EXPECT(orc_f64_to_bf16(0x1p-133) == 0x0001u); /* smallest subnormal */
  EXPECT(orc_bf16_to_f32(0x3F80u) == 1.0f);
  float sc[5] = {1.0f, 0.0f, -1.0f, NAN, INFINITY};
  int64_t bad = -1;
  EXPECT(orc_check_scales(sc, 5, &bad) == 0 && bad == 4);
  EXPECT(orc_check_scales(sc, 0, &bad) == 0 && bad == 0);
}

static void check_error_paths(void) {
  uint16_t x[16] = {0};
  int8_t q[16];
  float sa[2] = {1.0f, 1.0f};
  int8_t w[16] = {0};
  float sw[2] = {1.0f, 0.0f};
  int32_t acc[4] = {0};
  uint16_t y[4];
  EXPECT(orc_quantize_act(NULL, 2, 8, q, sa) == 1);
  EXPECT(orc_quantize_act(x, 0, 8, q, sa) == 2);
  x[3] = 0x7F80u; /* +Inf */
  EXPECT(orc_quantize_act(x, 2, 8, q, sa) == 3);
  x[3] = 0;
  EXPECT(orc_gemm_i32(q, w, 2, 2, 0, acc) == 2);
  EXPECT(orc_epilogue(acc, sa, sw, NULL, 2, 2, NULL, y) == 4); /* sw = 0 */
  EXPECT(orc_linear(x, w, sw, NULL, 2, 2, 8, y) == 4);
  EXPECT(orc_silu_bf16(x, -1, y) == 2);
  EXPECT(orc_pow2_renorm(NULL, 1, 8, y) == 1);
  int64_t bad;
  EXPECT(orc_check_scales(NULL, 2, &bad) == 1);
}

int main(void) {
  const int64_t shapes[][3] = {{1, 1, 1},   {1, 128, 8},  {3, 5, 37},
                               {5, 7, 128}, {2, 3, 5376}, {4, 2, 130}};
  for (size_t i = 0; i < sizeof shapes / sizeof *shapes; ++i)
    check_quant_and_linear(shapes[i][0], shapes[i][1], shapes[i][2]);
  check_glue_and_conversions();
  check_error_paths();
  if (failures) {
    fprintf(stderr, "%d expectation(s) failed\n", failures);
    return 1;
  }
  printf("oracle sanitizer driver: ok (threads %d)\n", orc_num_threads());
  return 0;
}
