/*
 * w8a8_oracle.c -- plain CPU reference of the W8A8 INT8 projection.
 *
 * TEST INFRASTRUCTURE ONLY (see w8a8_oracle.h).  Slow on purpose: every
 * result is the literal definition, evaluated element by element in the
 * order the definition states, with OpenMP spreading independent rows
 * over host threads.  Build with -ffp-contract=off and without fast-math
 * so that each binary32 operation is a single IEEE round-to-nearest-even.
 */
#include "w8a8_oracle.h"

#include <float.h>
#include <math.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

#if !defined(FLT_EVAL_METHOD) || FLT_EVAL_METHOD != 0
#error "the oracle needs binary32 expressions evaluated in binary32"
#endif

/* ------------------------------------------------------------------ */
/* BF16 <-> binary32 / binary64                                        */
/* ------------------------------------------------------------------ */

float orc_bf16_to_f32(uint16_t b) {
  /* A BF16 value is the upper half of the binary32 with the same bits. */
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return f;
}

uint16_t orc_f32_to_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  if (isnan(f)) return (uint16_t)((u >> 16) | 0x0040u); /* quiet NaN */
  /* Keep the upper 16 bits after adding half an ulp of the result, plus
   * one more when the kept part is odd: round to nearest, ties to even.
   * A carry out of the mantissa moves to the next binade or to Inf,
   * which is the correct rounding in both cases. */
  uint32_t lsb = (u >> 16) & 1u;
  u += 0x7FFFu + lsb;
  return (uint16_t)(u >> 16);
}

uint16_t orc_f64_to_bf16(double d) {
  if (isnan(d)) return 0x7FC0u;
  uint16_t sign = signbit(d) ? 0x8000u : 0u;
  double a = fabs(d);
  if (a == 0.0) return sign;
  if (isinf(a)) return (uint16_t)(sign | 0x7F80u);
  /* BF16 keeps 8 significant bits: inside [2^e, 2^(e+1)) its spacing is
   * 2^(e-7); below the smallest normal (2^-126) the spacing stays 2^-133. */
  int e = ilogb(a);
  if (e < -126) e = -126;
  int qexp = e - 7;
  double r = nearbyint(ldexp(a, -qexp)); /* exact scaling, one rounding */
  double v = ldexp(r, qexp);             /* exact                     */
  float f = (float)v; /* v is a BF16 value (or 2^128 -> Inf): exact */
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  return (uint16_t)(sign | (u >> 16));
}

/* ------------------------------------------------------------------ */
/* Per-token activation quantization                                   */
/* ------------------------------------------------------------------ */

/* One row: returns 0 or 3 (non-finite input). */
static int quant_row(const uint16_t *x, int64_t K, int8_t *q, float *sa) {
  float amax = 0.0f;
  for (int64_t k = 0; k < K; ++k) {
    float v = orc_bf16_to_f32(x[k]);
    if (!isfinite(v)) return 3;
    float a = fabsf(v);
    if (a > amax) amax = a;
  }
  if (amax == 0.0f) {
    /* Nothing to scale: a zero scale and zero codes reproduce the row. */
    *sa = 0.0f;
    memset(q, 0, (size_t)K);
    return 0;
  }
  /* Symmetric INT8: the largest magnitude maps to 127. */
  float s = amax / 127.0f;
  *sa = s;
  for (int64_t k = 0; k < K; ++k) {
    float v = orc_bf16_to_f32(x[k]) / s;
    float r = nearbyintf(v); /* default mode: nearest, ties to even */
    if (r > 127.0f) r = 127.0f;
    if (r < -127.0f) r = -127.0f;
    q[k] = (int8_t)r;
  }
  return 0;
}

int orc_quantize_act(const uint16_t *x, int64_t M, int64_t K,
                     int8_t *q, float *sa) {
  if (!x || !q || !sa) return 1;
  if (M < 1 || K < 1) return 2;
  int status = 0;
#pragma omp parallel for schedule(static)
  for (int64_t m = 0; m < M; ++m) {
    int rc = quant_row(x + m * K, K, q + m * K, sa + m);
    if (rc) {
#pragma omp atomic write
      status = rc;
    }
  }
  return status;
}

/* ------------------------------------------------------------------ */
/* Per-output-channel weight quantization (the converter side)         */
/* ------------------------------------------------------------------ */

/* "feat(mps): support MiniMax-H3 INT8 inference on Apple M5" (LightX2V pull
 * request #1672), "Validation" and "Changes": weights become INT8 row by
 * row (one row per output channel) with a finite, positive FP32 scale per
 * channel.  Each row is quantized exactly like an activation row; an
 * all-zero row, whose amax/127 would be 0, keeps zero codes and takes the
 * scale 1 so that every scale is positive. */
int orc_quantize_weight(const uint16_t *w, int64_t N, int64_t K,
                        int8_t *q, float *sw) {
  if (!w || !q || !sw) return 1;
  if (N < 1 || K < 1) return 2;
  int status = 0;
#pragma omp parallel for schedule(static)
  for (int64_t n = 0; n < N; ++n) {
    int rc = quant_row(w + n * K, K, q + n * K, sw + n);
    if (rc) {
#pragma omp atomic write
      status = rc;
    } else if (sw[n] == 0.0f) {
      sw[n] = 1.0f;
    }
  }
  return status;
}

int orc_check_scales(const float *sw, int64_t N, int64_t *bad) {
  if (!sw || !bad) return 1;
  if (N < 0) return 2;
  int64_t count = 0;
  for (int64_t n = 0; n < N; ++n)
    if (!(isfinite(sw[n]) && sw[n] > 0.0f)) ++count;
  *bad = count;
  return 0;
}

/* ------------------------------------------------------------------ */
/* INT8 x INT8 -> INT32 matrix product                                 */
/* ------------------------------------------------------------------ */

/* Exact dot product of two INT8 rows of length K; 5 if it leaves INT32. */
static int dot_row(const int8_t *a, const int8_t *w, int64_t K,
                   int32_t *out) {
  int64_t s = 0;
  for (int64_t k = 0; k < K; ++k) s += (int64_t)a[k] * (int64_t)w[k];
  if (s > INT32_MAX || s < INT32_MIN) return 5;
  *out = (int32_t)s;
  return 0;
}

int orc_gemm_i32(const int8_t *a, const int8_t *w, int64_t M, int64_t N,
                 int64_t K, int32_t *acc) {
  if (!a || !w || !acc) return 1;
  if (M < 1 || N < 1 || K < 1) return 2;
  int status = 0;
#pragma omp parallel for schedule(static)
  for (int64_t m = 0; m < M; ++m) {
    for (int64_t n = 0; n < N; ++n) {
      int rc = dot_row(a + m * K, w + n * K, K, acc + m * N + n);
      if (rc) {
#pragma omp atomic write
        status = rc;
      }
    }
  }
  return status;
}

/* ------------------------------------------------------------------ */
/* Epilogue: dequantize, add bias, round once                          */
/* ------------------------------------------------------------------ */

static float epi_one(int32_t acc, float sa, float sw, const uint16_t *bias,
                     int64_t n) {
  float t = (float)acc; /* int -> binary32, nearest-even */
  t = t * sa;
  t = t * sw;
  if (bias) t = t + orc_bf16_to_f32(bias[n]);
  return t;
}

static int check_scales(const float *sw, int64_t N) {
  for (int64_t n = 0; n < N; ++n)
    if (!isfinite(sw[n]) || !(sw[n] > 0.0f)) return 4;
  return 0;
}

int orc_epilogue(const int32_t *acc, const float *sa, const float *sw,
                 const uint16_t *bias, int64_t M, int64_t N,
                 float *y_f32, uint16_t *y_bf16) {
  if (!acc || !sa || !sw) return 1;
  if (M < 1 || N < 1) return 2;
  int rc = check_scales(sw, N);
  if (rc) return rc;
#pragma omp parallel for schedule(static)
  for (int64_t m = 0; m < M; ++m) {
    for (int64_t n = 0; n < N; ++n) {
      float t = epi_one(acc[m * N + n], sa[m], sw[n], bias, n);
      if (y_f32) y_f32[m * N + n] = t;
      if (y_bf16) y_bf16[m * N + n] = orc_f32_to_bf16(t);
    }
  }
  return 0;
}

/* ------------------------------------------------------------------ */
/* Whole linear: quantize, then per output element dot + epilogue      */
/* ------------------------------------------------------------------ */

int orc_linear(const uint16_t *x, const int8_t *w, const float *sw,
               const uint16_t *bias, int64_t M, int64_t N, int64_t K,
               uint16_t *y) {
  if (!x || !w || !sw || !y) return 1;
  if (M < 1 || N < 1 || K < 1) return 2;
  int rc = check_scales(sw, N);
  if (rc) return rc;
  int status = 0;
#pragma omp parallel
  {
    int8_t *q = (int8_t *)malloc((size_t)K);
    if (!q) {
#pragma omp atomic write
      status = 1;
    }
#pragma omp for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
      if (!q) continue;
      float sa;
      int r = quant_row(x + m * K, K, q, &sa);
      for (int64_t n = 0; !r && n < N; ++n) {
        int32_t acc;
        r = dot_row(q, w + n * K, K, &acc);
        if (!r) y[m * N + n] = orc_f32_to_bf16(epi_one(acc, sa, sw[n], bias, n));
      }
      if (r) {
#pragma omp atomic write
        status = r;
      }
    }
    free(q);
  }
  return status;
}

/* ------------------------------------------------------------------ */
/* Harness glue                                                        */
/* ------------------------------------------------------------------ */

int orc_silu_bf16(const uint16_t *x, int64_t n, uint16_t *y) {
  if (!x || !y) return 1;
  if (n < 0) return 2;
  int status = 0;
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    double v = (double)orc_bf16_to_f32(x[i]);
    if (!isfinite(v)) {
#pragma omp atomic write
      status = 3;
      continue;
    }
    y[i] = orc_f64_to_bf16(v / (1.0 + exp(-v)));
  }
  return status;
}

int orc_swiglu_bf16(const uint16_t *h, int64_t M, int64_t F, uint16_t *y) {
  if (!h || !y) return 1;
  if (M < 1 || F < 1) return 2;
  int status = 0;
#pragma omp parallel for schedule(static)
  for (int64_t m = 0; m < M; ++m) {
    const uint16_t *gate = h + m * 2 * F;
    const uint16_t *up = gate + F;
    for (int64_t f = 0; f < F; ++f) {
      double g = (double)orc_bf16_to_f32(gate[f]);
      double u = (double)orc_bf16_to_f32(up[f]);
      if (!isfinite(g) || !isfinite(u)) {
#pragma omp atomic write
        status = 3;
        continue;
      }
      /* SiLU of the gate, rounded once to BF16 (as orc_silu_bf16) ... */
      double s = (double)orc_bf16_to_f32(orc_f64_to_bf16(g / (1.0 + exp(-g))));
      /* ... times the up value: two BF16 values multiply exactly in
       * binary64, and the product is rounded once to BF16. */
      y[m * F + f] = orc_f64_to_bf16(s * u);
    }
  }
  return status;
}

int orc_pow2_renorm(const uint16_t *x, int64_t M, int64_t K, uint16_t *y) {
  if (!x || !y) return 1;
  if (M < 1 || K < 1) return 2;
  int status = 0;
#pragma omp parallel for schedule(static)
  for (int64_t m = 0; m < M; ++m) {
    const uint16_t *xr = x + m * K;
    uint16_t *yr = y + m * K;
    float amax = 0.0f;
    int bad = 0;
    for (int64_t k = 0; k < K; ++k) {
      float v = orc_bf16_to_f32(xr[k]);
      if (!isfinite(v)) bad = 1;
      if (fabsf(v) > amax) amax = fabsf(v);
    }
    if (bad) {
#pragma omp atomic write
      status = 3;
      continue;
    }
    if (amax == 0.0f) {
      memcpy(yr, xr, (size_t)K * sizeof *yr);
      continue;
    }
    int ex;
    frexpf(amax, &ex); /* amax = f * 2^ex, f in [0.5, 1) */
    int e = ex - 1;    /* floor(log2(amax)), subnormals included */
    for (int64_t k = 0; k < K; ++k)
      yr[k] = orc_f64_to_bf16(ldexp((double)orc_bf16_to_f32(xr[k]), -e));
  }
  return status;
}

int orc_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
