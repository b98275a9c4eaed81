/*
 * w8a8.h -- C ABI of the MI355X (gfx950) W8A8 INT8 projection library.
 *
 * The operation is the INT8 projection GEMM inside each block of a
 * MiniMax-H3-style audio/video diffusion transformer: Q, K, V, attention
 * output, FC1 and FC2 run with INT8 weights and per-token INT8 activations
 * at the model's native hidden width (5376), without padding K and without
 * dequantizing the weights ("feat(mps): support MiniMax-H3 INT8 inference
 * on Apple M5", LightX2V pull request #1672: description, commit notes and
 * "Changes" table).
 *
 * Conventions shared by every entry point:
 *   - All tensors are dense and row-major, with no leading-dimension
 *     arguments.  BF16 values are passed as their 16-bit patterns.
 *   - Device pointers only (memory the caller allocated on the current HIP
 *     device); the caller owns every buffer, including any workspace.  The
 *     library never allocates, frees or synchronizes.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Calls enqueue
 *     kernels on it and return without waiting.
 *   - Arguments are validated on the host before anything is enqueued; on
 *     error nothing is launched and no output is touched.  A launch failure
 *     returns W8A8_ERR_HIP; a device fault surfaces at the caller's next
 *     synchronization.
 *   - The current device must be a gfx950 GPU; otherwise W8A8_ERR_DEVICE
 *     (there is no other code path).
 *   - Calls on one stream are ordered; concurrent calls on different
 *     streams are safe as long as their output buffers do not overlap.
 *   - Not checked on the device (documented preconditions): activations are
 *     finite; weight scales are finite and > 0 (the converter on the
 *     LightX2V page validates exactly this, "Validation").
 */
#ifndef W8A8_H
#define W8A8_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  W8A8_OUT_BF16 = 0, /* y: uint16 BF16 bits [M,N]                        */
  W8A8_OUT_FP32 = 1, /* y: float [M,N], the epilogue before BF16 rounding */
  W8A8_OUT_I32 = 2   /* y: int32 [M,N], the raw INT32 accumulators        */
} w8a8_out_t;

typedef enum {
  W8A8_OK = 0,
  W8A8_ERR_NULL = 1,      /* a required pointer is NULL                  */
  W8A8_ERR_SHAPE = 2,     /* a size violates the shape contract          */
  W8A8_ERR_ALIGN = 3,     /* a pointer is not aligned as required        */
  W8A8_ERR_WORKSPACE = 4, /* workspace missing or smaller than required  */
  W8A8_ERR_OUT_DTYPE = 5, /* unknown output type                         */
  W8A8_ERR_ALIAS = 6,     /* an output overlaps an input or other output */
  W8A8_ERR_DEVICE = 7,    /* no HIP device, or it is not gfx950          */
  W8A8_ERR_HIP = 8        /* a HIP call or kernel launch failed          */
} w8a8_status_t;

/* Largest K accepted by w8a8_gemm / w8a8_linear: with INT8 operands every
 * product is at most 128*128 = 2^14 in magnitude, so the INT32 accumulator
 * cannot overflow while K*2^14 <= 2^31 - 1; 130944 is the largest multiple
 * of 128 below that bound. */
#define W8A8_MAX_K 130944

/*
 * Per-token activation quantization.
 *   x        BF16 [M,K], 16-byte aligned.
 *   a_q      INT8 [M,K] out, 8-byte aligned.
 *   a_scale  FP32 [M] out, 4-byte aligned.
 * For each row m: amax = max_k |x[m,k]|; a_scale[m] = amax / 127 (binary32
 * division, round to nearest even); a_q[m,k] = x[m,k] / a_scale[m] divided
 * in binary32 and rounded to the nearest integer, ties to even, clamped to
 * [-127, 127].  A row of zeros gives a_scale = 0 and zero codes.  FP32
 * subnormals are kept.
 * Shape: 1 <= M <= 2^24 - 1 (a launch holds fewer than 2^32 work-items,
 * up to 256 per row), 8 <= K <= W8A8_MAX_K and K % 8 == 0 (16-byte rows
 * of BF16; up to K = 90112 a row stays in registers and is read once,
 * longer rows are read twice); rows whose length is not a multiple of the
 * kernel's chunk width are handled by masking the partial chunk, as the
 * LightX2V page's quantizer does (commit notes, "Changes" table).
 * Errors: NULL, SHAPE, ALIGN, ALIAS (a_q or a_scale overlapping x or each
 * other), DEVICE, HIP.
 */
int w8a8_quantize_act(const uint16_t *x, int64_t M, int64_t K, int8_t *a_q,
                      float *a_scale, void *stream);

/*
 * INT8 GEMM with fused dequantization epilogue.
 *   a_q       INT8 [M,K] activation codes, 16-byte aligned.
 *   a_scale   FP32 [M] per-token scales, 4-byte aligned.
 *   w_q       INT8 [N,K] weights in a Linear's stored layout (one row per
 *             output channel), 16-byte aligned, consumed as stored.
 *   w_scale   FP32 [N] per-output-channel scales (finite, > 0), 4-byte
 *             aligned (16-byte alignment lets the epilogue use vector
 *             loads; a channel slice of a larger array is accepted).
 *   bias      BF16 [N] or NULL (no bias), 2-byte aligned (8-byte: vector
 *             loads).
 *   out       [M,N] of the type selected by out_dtype, 16-byte aligned.
 *   out_dtype W8A8_OUT_BF16, W8A8_OUT_FP32 or W8A8_OUT_I32.
 *   workspace device scratch of at least w8a8_gemm_workspace_bytes(M, N,
 *             K) bytes (w8a8_workspace_bytes is always enough; may be NULL
 *             when the former is 0), 16-byte aligned.  It holds INT32
 *             partial sums of split-K launches; its contents before and
 *             after the call do not matter.
 * acc[m,n] = sum_k a_q[m,k] * w_q[n,k] exactly in INT32;
 * t = ((float)acc * a_scale[m]) * w_scale[n] + bf16->f32(bias[n]), each
 * operation rounded in binary32 with no fused multiply-add; BF16 output is
 * t rounded once to nearest even.  Adding the bias before the one rounding
 * follows "MLX implementation and experiment report" (MiniMax-H3-Image-mlx),
 * "What the default preserves".
 * Shape: 1 <= M < 2^31; N and K positive multiples of 128 (the LightX2V
 * page's shape contract, commit notes); N < 2^31; K <= W8A8_MAX_K; and the
 * tile grid (256 x 256 tiles of 512 work-items, or 64 x 128 tiles of 256)
 * below 2^32 work-items: M * N up to about 2^39 (M <= 25.6 million at
 * N = 21504).
 * Errors: NULL, SHAPE, ALIGN, WORKSPACE, OUT_DTYPE, ALIAS, DEVICE, HIP.
 */
int w8a8_gemm(const int8_t *a_q, const float *a_scale, const int8_t *w_q,
              const float *w_scale, const uint16_t *bias, void *out,
              int out_dtype, int64_t M, int64_t N, int64_t K,
              void *workspace, size_t workspace_bytes, void *stream);

/*
 * w8a8_gemm without a workspace, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation).  Arguments, results and errors as w8a8_gemm;
 * the split-K partial sums go to a device array the library holds, one
 * copy of W8A8_NOALLOC_SCRATCH_BYTES per GPU for the life of the process
 * (no call allocates or frees anything).  Every shape w8a8_gemm accepts
 * fits: its partial sums never exceed that size (W8A8_ERR_WORKSPACE
 * otherwise).  Calls of this entry point that overlap in time on one GPU
 * (on different streams, or from different threads) share that array and
 * race: order them on one stream.  The array's contents between calls do
 * not matter (nothing in it needs clearing).  The array's address is
 * looked up once per GPU at the first call of any entry point there.
 */
#define W8A8_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int w8a8_gemm_noalloc(const int8_t *a_q, const float *a_scale,
                      const int8_t *w_q, const float *w_scale,
                      const uint16_t *bias, void *out, int out_dtype,
                      int64_t M, int64_t N, int64_t K, void *stream);

/*
 * Whole projection, the quantized Linear that replaces a BF16 Linear on
 * each of the six block projections ("feat(mps): support MiniMax-H3 INT8
 * inference on Apple M5", LightX2V pull request #1672, description: W8A8
 * on Q, K, V, attention output, FC1 and FC2; commit notes: per-token
 * activation quantization feeding the INT8 GEMM at native K): per-token
 * quantization of x (as w8a8_quantize_act) into the workspace, then the
 * INT8 GEMM with BF16 output (as w8a8_gemm), y = bf16(((float)acc*sa[m]) *
 * sw[n] + bias[n]) with the bias added before the one rounding ("MLX
 * implementation and experiment report", "What the default preserves").
 *   x   BF16 [M,K] (16-byte aligned); y BF16 [M,N] (16-byte aligned);
 *   the other arguments as for w8a8_gemm.
 * Workspace: at least w8a8_workspace_bytes(M, N, K) bytes, 16-byte
 * aligned, not overlapping any argument (the INT8 codes, their scales and
 * the GEMM's partial sums).  M <= 2^24 - 1 (the quantizer's bound).
 * Errors: as w8a8_gemm.
 */
int w8a8_linear(const uint16_t *x, const int8_t *w_q, const float *w_scale,
                const uint16_t *bias, uint16_t *y, int64_t M, int64_t N,
                int64_t K, void *workspace, size_t workspace_bytes,
                void *stream);

/*
 * Per-output-channel weight quantization (the converter side of the
 * GEMM: "feat(mps): support MiniMax-H3 INT8 inference on Apple M5",
 * LightX2V pull request #1672, "Validation" and "Changes": weights become
 * INT8 one row per output channel with a finite, positive FP32 scale).
 *   w        BF16 [N,K] in a Linear's layout, 16-byte aligned.
 *   w_q      INT8 [N,K] out, 8-byte aligned.
 *   w_scale  FP32 [N] out, 4-byte aligned.
 * Each row is quantized exactly as w8a8_quantize_act quantizes a token
 * row, except that an all-zero row takes the scale 1 (its codes are 0), so
 * every scale is finite and positive.  Shape, alignment and errors as
 * w8a8_quantize_act with M = N.
 */
int w8a8_quantize_weight(const uint16_t *w, int64_t N, int64_t K,
                         int8_t *w_q, float *w_scale, void *stream);

/*
 * Scale contract check: *bad_count (a device int32, 4-byte aligned)
 * receives the number of entries of w_scale [N] that are not finite and
 * > 0 (NaN, +-Inf, zero or negative), for weights produced elsewhere.
 * 0 <= N < 2^31.  Errors: NULL, SHAPE, ALIGN, DEVICE, HIP.
 */
int w8a8_check_scales(const float *w_scale, int64_t N, int32_t *bad_count,
                      void *stream);

/* Workspace bytes that serve both w8a8_linear and w8a8_gemm for this
 * shape: the INT8 activation codes [M,K] and their scales [M] that
 * w8a8_linear stages, plus the INT32 split-K partial sums of the GEMM, each
 * part starting at a 256-byte offset.  0 for shapes the contract rejects. */
size_t w8a8_workspace_bytes(int64_t M, int64_t N, int64_t K);

/* The smaller workspace w8a8_gemm alone needs (only its split-K partial
 * sums; 0 when the plan for this shape splits nothing, and for shapes the
 * contract rejects). */
size_t w8a8_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K);

/* Static description of a status code (never NULL). */
const char *w8a8_status_string(int status);

/* hipError_t code of the last W8A8_ERR_HIP returned on this thread (0 if
 * none yet), for diagnostics. */
int w8a8_last_hip_error(void);

/* SHA-256 (64 hex digits) of the sources this library was compiled from
 * (its kernels, API layer and this header), so a caller can refuse a build
 * that no longer matches the sources beside it. */
const char *w8a8_build_id(void);

/*
 * Glue between projections (not part of the W8A8 method; it produces the
 * inputs a DiT block feeds to FC2 and to the next block).
 *
 * w8a8_silu_bf16: y[i] = x / (1 + exp(-x)) correctly rounded to BF16, for
 *   n elements, read from a table of all 65536 BF16 inputs that a small
 *   kernel fills on the device (FP32 evaluation, FP64 for the rare inputs
 *   whose FP32 value lies too close to a BF16 rounding midpoint) on the
 *   caller's stream ahead of every call; x and y 16-byte aligned, n >= 0
 *   and n % 8 == 0; x and y may be the same buffer (in place) but must not
 *   partially overlap.
 *   Between FC1 and FC2 the block applies SiLU to the BF16 output of FC1
 *   ("MLX implementation and experiment report", "What the default
 *   preserves": SiLU rounding follows the original recipe).
 *
 * w8a8_pow2_renorm: each row of x [M,K] is multiplied by 2^-e, where
 *   e = floor(log2(max_k |x[m,k]|)), and rounded to BF16 (all-zero rows
 *   are copied).  Per-token symmetric quantization is exactly invariant to
 *   such a scaling, so chaining blocks through it changes no INT8 code
 *   while keeping BF16 activations finite.  K % 8 == 0, 16-byte aligned;
 *   in place allowed.
 *
 * w8a8_pow2_renorm_quantize: w8a8_pow2_renorm of x into y followed by
 *   w8a8_quantize_act of y, in one pass over x: y BF16 [M,K] is written
 *   and a_q INT8 [M,K], a_scale FP32 [M] are exactly what
 *   w8a8_quantize_act(y) produces.  x, y 16-byte aligned, a_q 8-byte,
 *   a_scale 4-byte; 8 <= K <= 90112, K % 8 == 0; y may be x (in place) but
 *   must not partially overlap it; a_q and a_scale overlap nothing.
 *   Errors as w8a8_quantize_act.
 *
 * w8a8_quantize_act_silu: w8a8_silu_bf16 followed by w8a8_quantize_act in
 *   one pass over x (the SiLU values are rounded to BF16 before they are
 *   quantized, exactly as the two separate calls do); the BF16 SiLU output
 *   is not written.  Arguments and errors as w8a8_quantize_act, with
 *   8 <= K <= 90112.
 */
int w8a8_silu_bf16(const uint16_t *x, uint16_t *y, int64_t n, void *stream);

/*
 * Gated-MLP glue for the fused gate/up projection of the pages' H3 shapes
 * ("MLX implementation and experiment report", "Operator tuning": a fused
 * gate/up GEMM 5376 -> 28672 feeding a down GEMM 14336 -> 5376; "What the
 * default preserves": BF16 products and SiLU rounding as in the original).
 *
 * w8a8_swiglu_bf16: h BF16 [M, 2F] holds the gate g in its first F columns
 *   and the up value u in the next F; y BF16 [M, F] = BF16(BF16(silu(g)) *
 *   u), the SiLU as w8a8_silu_bf16 and the product (exact in FP32) rounded
 *   once to nearest even.  h and y 16-byte aligned, F % 8 == 0, M >= 1; y
 *   must not overlap h.
 *
 * w8a8_quantize_act_swiglu: w8a8_swiglu_bf16 followed by
 *   w8a8_quantize_act of the [M, F] result in one pass over h (the SwiGLU
 *   output is not written).  a_q INT8 [M, F] (8-byte aligned), a_scale
 *   FP32 [M] (4-byte aligned); 8 <= F <= 90112.  Errors as
 *   w8a8_quantize_act.
 */
int w8a8_swiglu_bf16(const uint16_t *h, uint16_t *y, int64_t M, int64_t F,
                     void *stream);
int w8a8_quantize_act_swiglu(const uint16_t *h, int64_t M, int64_t F,
                             int8_t *a_q, float *a_scale, void *stream);
int w8a8_pow2_renorm(const uint16_t *x, uint16_t *y, int64_t M, int64_t K,
                     void *stream);
int w8a8_pow2_renorm_quantize(const uint16_t *x, int64_t M, int64_t K,
                              uint16_t *y, int8_t *a_q, float *a_scale,
                              void *stream);
int w8a8_quantize_act_silu(const uint16_t *x, int64_t M, int64_t K,
                           int8_t *a_q, float *a_scale, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* W8A8_H */
