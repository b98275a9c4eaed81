/*
 * quant_fastpath_model.c -- a CPU model of the device quantizer's
 * arithmetic (test infrastructure; built by tests/test_quant_fastpath.py).
 *
 * The device quantizer (quant_row / quant4 in rowwise.hip) does not divide
 * every element by the row scale.  For a row with scale s = amax / 127
 * (binary32) it forms r = 1 / s once (binary32 division) and, per element,
 * u = fma(x, r, 128) (one rounding); when u lies farther than 2^-14 from
 * a half-integer, the code is round(u) - 128 (the conversion to an
 * unsigned byte rounds to nearest).  Elements whose u lies within 2^-14
 * of a half-integer, and every element of a row whose scale is below the
 * smallest normal binary32 (2^-126), take the division instead:
 * clamp(rint(x / s), -127, 127).  The device applies the closeness test
 * to groups of four elements (a close element sends its whole group to
 * the division); modelled per element, the fast path is taken for a
 * superset of the elements the device takes it for, so agreement here
 * covers the device's choice too.
 *
 * model_codes() evaluates that arithmetic in C (binary32 with a correctly
 * rounded fmaf, no contraction, round-to-nearest), so a test can compare
 * it with the oracle's x / s over every BF16 input.  `closeness` is the
 * half-integer margin (2^-14 on the device; 0 disables the test, for the
 * negative control).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

static float bf16_to_f32(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return f;
}

/* Codes of x[0..n) in a row whose largest magnitude is amax (BF16 bits);
 * *fast_count receives how many took the reciprocal path.  Returns 0. */
int model_codes(const uint16_t *x, int64_t n, uint16_t amax_bits,
                float closeness, int8_t *codes, int64_t *fast_count) {
  const float amax = bf16_to_f32(amax_bits);
  const float s = amax / 127.0f;
  const int fast_row = s >= 0x1p-126f;
  const float r = fast_row ? 1.0f / s : 0.0f;
  int64_t fast = 0;
  for (int64_t i = 0; i < n; ++i) {
    const float f = bf16_to_f32(x[i]);
    if (s == 0.0f) {
      codes[i] = 0;
      continue;
    }
    const float u = fmaf(f, r, 128.0f);
    const float d = fabsf((u - floorf(u)) - 0.5f);
    if (fast_row && d > closeness) {
      codes[i] = (int8_t)((int)rintf(u) - 128);
      ++fast;
    } else {
      float q = rintf(f / s);
      if (q > 127.0f) q = 127.0f;
      if (q < -127.0f) q = -127.0f;
      codes[i] = (int8_t)q;
    }
  }
  *fast_count = fast;
  return 0;
}
