// w8a8_api.cpp -- the C ABI declared in include/w8a8.h.
//
// Every entry point validates its arguments on the host first (pointers,
// shape contract, alignment, overlap, workspace size, device) and launches
// nothing when a check fails; only then does it enqueue kernels on the
// caller's stream.  The library allocates nothing and never synchronizes.
#include <hip/hip_runtime.h>

#include <cstring>
#include <mutex>
#include <unordered_map>

#include "internal.h"
#include "rowwise.h"
#include "w8a8.h"

namespace {

using w8a8::GemmArgs;
using w8a8::GemmPlan;

// Largest K the register-resident row kernels cover (44 chunks of 8 BF16
// per lane x 4 waves x 64 lanes): the glue kernels (SiLU, renormalization)
// and the fused quantizers.  The plain quantizers (activations, weights)
// take longer rows, up to W8A8_MAX_K, through a kernel that reads each row
// twice.
constexpr int64_t kGlueMaxK = 44 * 8 * 4 * 64;
constexpr int64_t kQuantMaxK = W8A8_MAX_K;
constexpr int64_t kMaxRows = 0x7FFFFFFF;
// Rows of the per-token kernels: their launches hold up to 256 work-items
// per row, and a launch holds fewer than 2^32 work-items.
constexpr int64_t kMaxTokenRows = (int64_t(1) << 24) - 1;

thread_local int g_last_hip_error = 0;

inline bool aligned(const void *p, uintptr_t a) {
  return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0;
}

struct Range {
  uintptr_t lo, hi;  // [lo, hi)
};

inline Range range_of(const void *p, int64_t bytes) {
  const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
  return Range{lo, lo + (uintptr_t)(bytes > 0 ? bytes : 0)};
}

inline bool overlap(Range a, Range b) {
  return a.lo < b.hi && b.lo < a.hi && a.hi > a.lo && b.hi > b.lo;
}

inline size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// The current device must be gfx950; checked once per device and cached.
int check_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return W8A8_ERR_DEVICE;
  static std::mutex mu;
  static std::unordered_map<int, int> checked;
  std::lock_guard<std::mutex> lock(mu);
  auto it = checked.find(dev);
  if (it != checked.end()) return it->second;
  hipDeviceProp_t prop;
  int status = W8A8_ERR_DEVICE;
  if (hipGetDeviceProperties(&prop, dev) == hipSuccess &&
      std::strncmp(prop.gcnArchName, "gfx950", 6) == 0)
    status = W8A8_OK;
  // Set-up on the first call on a gfx950 device, with it current: the
  // address of this device's copy of the allocation-free entry point's
  // scratch (a failure is reported by that entry point, which retries).
  if (status == W8A8_OK) (void)w8a8::resolve_scratch(dev);
  checked[dev] = status;
  return status;
}

inline int hip_status(hipError_t e) {
  if (e == hipSuccess) return W8A8_OK;
  g_last_hip_error = (int)e;
  return W8A8_ERR_HIP;
}

bool gemm_shape_ok(int64_t M, int64_t N, int64_t K) {
  return M >= 1 && M <= kMaxRows && N >= 128 && N % 128 == 0 &&
         N <= kMaxRows && K >= 128 && K % 128 == 0 && K <= W8A8_MAX_K;
}

int validate_quant(const uint16_t *x, int64_t M, int64_t K, const int8_t *q,
                   const float *sa, int64_t max_k = kQuantMaxK) {
  if (!x || !q || !sa) return W8A8_ERR_NULL;
  if (M < 1 || M > kMaxTokenRows || K < 8 || K % 8 != 0 || K > max_k)
    return W8A8_ERR_SHAPE;
  if (!aligned(x, 16) || !aligned(q, 8) || !aligned(sa, 4))
    return W8A8_ERR_ALIGN;
  const Range rx = range_of(x, M * K * 2), rq = range_of(q, M * K),
              rs = range_of(sa, M * 4);
  if (overlap(rx, rq) || overlap(rx, rs) || overlap(rq, rs))
    return W8A8_ERR_ALIAS;
  return W8A8_OK;
}

int out_elem_bytes(int out_dtype) {
  switch (out_dtype) {
    case W8A8_OUT_BF16: return 2;
    case W8A8_OUT_FP32: return 4;
    case W8A8_OUT_I32: return 4;
    default: return 0;
  }
}

// Everything w8a8_gemm checks except its workspace: pointers, shape,
// output type, alignment, a launchable plan and overlaps between the
// output and the inputs.
int validate_gemm_args(const int8_t *a_q, const float *a_scale,
                       const int8_t *w_q, const float *w_scale,
                       const uint16_t *bias, const void *out, int out_dtype,
                       int64_t M, int64_t N, int64_t K, GemmPlan *plan) {
  if (!a_q || !a_scale || !w_q || !w_scale || !out) return W8A8_ERR_NULL;
  if (!gemm_shape_ok(M, N, K)) return W8A8_ERR_SHAPE;
  const int eb = out_elem_bytes(out_dtype);
  if (eb == 0) return W8A8_ERR_OUT_DTYPE;
  if (!aligned(a_q, 16) || !aligned(w_q, 16) || !aligned(out, 16) ||
      !aligned(w_scale, 4) || !aligned(a_scale, 4) ||
      (bias && !aligned(bias, 2)))
    return W8A8_ERR_ALIGN;
  *plan = w8a8::plan_gemm(M, N, K);
  if (!w8a8::plan_launchable(*plan)) return W8A8_ERR_SHAPE;
  const Range ro = range_of(out, M * N * eb);
  const Range ins[] = {range_of(a_q, M * K), range_of(a_scale, M * 4),
                       range_of(w_q, N * K), range_of(w_scale, N * 4),
                       range_of(bias, bias ? N * 2 : 0)};
  for (const Range &r : ins)
    if (overlap(ro, r)) return W8A8_ERR_ALIAS;
  return W8A8_OK;
}

// The partial-sum buffer of a plan against the call's other buffers.
int scratch_alias(const void *buf, const GemmPlan &plan, const int8_t *a_q,
                  const float *a_scale, const int8_t *w_q,
                  const float *w_scale, const uint16_t *bias,
                  const void *out, int out_dtype, int64_t M, int64_t N,
                  int64_t K) {
  if (plan.workspace == 0) return W8A8_OK;
  const Range rw = range_of(buf, (int64_t)plan.workspace);
  const Range all[] = {range_of(out, M * N * out_elem_bytes(out_dtype)),
                       range_of(a_q, M * K), range_of(a_scale, M * 4),
                       range_of(w_q, N * K), range_of(w_scale, N * 4),
                       range_of(bias, bias ? N * 2 : 0)};
  for (const Range &r : all)
    if (overlap(rw, r)) return W8A8_ERR_ALIAS;
  return W8A8_OK;
}

int validate_gemm(const int8_t *a_q, const float *a_scale, const int8_t *w_q,
                  const float *w_scale, const uint16_t *bias, const void *out,
                  int out_dtype, int64_t M, int64_t N, int64_t K,
                  const void *workspace, size_t workspace_bytes,
                  GemmPlan *plan) {
  int st = validate_gemm_args(a_q, a_scale, w_q, w_scale, bias, out,
                              out_dtype, M, N, K, plan);
  if (st != W8A8_OK) return st;
  if (plan->workspace > 0) {
    if (!workspace || workspace_bytes < plan->workspace)
      return W8A8_ERR_WORKSPACE;
    if (!aligned(workspace, 16)) return W8A8_ERR_ALIGN;
  }
  return scratch_alias(workspace, *plan, a_q, a_scale, w_q, w_scale, bias,
                       out, out_dtype, M, N, K);
}

}  // namespace

extern "C" {

const char *w8a8_status_string(int status) {
  switch (status) {
    case W8A8_OK: return "ok";
    case W8A8_ERR_NULL: return "a required pointer is NULL";
    case W8A8_ERR_SHAPE: return "a size violates the shape contract";
    case W8A8_ERR_ALIGN: return "a pointer is not aligned as required";
    case W8A8_ERR_WORKSPACE: return "workspace missing or too small";
    case W8A8_ERR_OUT_DTYPE: return "unknown output type";
    case W8A8_ERR_ALIAS: return "an output overlaps another buffer";
    case W8A8_ERR_DEVICE: return "no HIP device, or it is not gfx950";
    case W8A8_ERR_HIP: return "a HIP call or kernel launch failed";
    default: return "unknown status";
  }
}

int w8a8_last_hip_error(void) { return g_last_hip_error; }

#ifndef W8A8_SOURCE_SHA256
#define W8A8_SOURCE_SHA256 "unknown"
#endif
const char *w8a8_build_id(void) { return W8A8_SOURCE_SHA256; }

size_t w8a8_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  if (!gemm_shape_ok(M, N, K)) return 0;
  return w8a8::plan_gemm(M, N, K).workspace;
}

size_t w8a8_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  if (!gemm_shape_ok(M, N, K) || M > kMaxTokenRows) return 0;
  return round_up((size_t)(M * K), 256) + round_up((size_t)M * 4, 256) +
         w8a8::plan_gemm(M, N, K).workspace;
}

int w8a8_quantize_act(const uint16_t *x, int64_t M, int64_t K, int8_t *a_q,
                      float *a_scale, void *stream) {
  int st = validate_quant(x, M, K, a_q, a_scale);
  if (st != W8A8_OK) return st;
  if ((st = check_device()) != W8A8_OK) return st;
  return hip_status(w8a8::launch_quantize_act(
      x, a_q, a_scale, M, K, false, static_cast<hipStream_t>(stream)));
}

int w8a8_quantize_act_silu(const uint16_t *x, int64_t M, int64_t K,
                           int8_t *a_q, float *a_scale, void *stream) {
  int st = validate_quant(x, M, K, a_q, a_scale, kGlueMaxK);
  if (st != W8A8_OK) return st;
  if ((st = check_device()) != W8A8_OK) return st;
  return hip_status(w8a8::launch_quantize_act(
      x, a_q, a_scale, M, K, true, static_cast<hipStream_t>(stream)));
}

int w8a8_gemm(const int8_t *a_q, const float *a_scale, const int8_t *w_q,
              const float *w_scale, const uint16_t *bias, void *out,
              int out_dtype, int64_t M, int64_t N, int64_t K,
              void *workspace, size_t workspace_bytes, void *stream) {
  GemmPlan plan;
  int st = validate_gemm(a_q, a_scale, w_q, w_scale, bias, out, out_dtype, M,
                         N, K, workspace, workspace_bytes, &plan);
  if (st != W8A8_OK) return st;
  if ((st = check_device()) != W8A8_OK) return st;
  GemmArgs g{a_q, a_scale, w_q, w_scale, bias, out, out_dtype,
             M,   N,       K,   workspace, workspace_bytes};
  return hip_status(
      w8a8::launch_gemm(g, plan, static_cast<hipStream_t>(stream)));
}

int w8a8_gemm_noalloc(const int8_t *a_q, const float *a_scale,
                      const int8_t *w_q, const float *w_scale,
                      const uint16_t *bias, void *out, int out_dtype,
                      int64_t M, int64_t N, int64_t K, void *stream) {
  // As w8a8_gemm, with the split-K partial sums in the library's own device
  // scratch (one copy per GPU) instead of a caller's workspace: nothing is
  // allocated here.  A plan needing more than the scratch is refused (the
  // planner's bound on partial sums makes that impossible today).
  GemmPlan plan;
  int st = validate_gemm_args(a_q, a_scale, w_q, w_scale, bias, out,
                              out_dtype, M, N, K, &plan);
  if (st != W8A8_OK) return st;
  if (plan.workspace > w8a8::kScratchBytes) return W8A8_ERR_WORKSPACE;
  if ((st = check_device()) != W8A8_OK) return st;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return W8A8_ERR_DEVICE;
  void *scratch = w8a8::scratch_on_device(dev);
  if (scratch == nullptr) {  // set-up failed at the device check: retry
    st = hip_status(w8a8::resolve_scratch(dev));
    if (st != W8A8_OK) return st;
    scratch = w8a8::scratch_on_device(dev);
  }
  st = scratch_alias(scratch, plan, a_q, a_scale, w_q, w_scale, bias, out,
                     out_dtype, M, N, K);
  if (st != W8A8_OK) return st;
  GemmArgs g{a_q, a_scale, w_q, w_scale, bias, out, out_dtype,
             M,   N,       K,   scratch, w8a8::kScratchBytes};
  return hip_status(
      w8a8::launch_gemm(g, plan, static_cast<hipStream_t>(stream)));
}

int w8a8_linear(const uint16_t *x, const int8_t *w_q, const float *w_scale,
                const uint16_t *bias, uint16_t *y, int64_t M, int64_t N,
                int64_t K, void *workspace, size_t workspace_bytes,
                void *stream) {
  if (!x || !w_q || !w_scale || !y) return W8A8_ERR_NULL;
  if (!gemm_shape_ok(M, N, K) || K > kQuantMaxK || M > kMaxTokenRows)
    return W8A8_ERR_SHAPE;
  if (!aligned(x, 16)) return W8A8_ERR_ALIGN;
  const size_t need = w8a8_workspace_bytes(M, N, K);
  if (!workspace || workspace_bytes < need) return W8A8_ERR_WORKSPACE;
  if (!aligned(workspace, 16)) return W8A8_ERR_ALIGN;
  int8_t *aq = static_cast<int8_t *>(workspace);
  float *sa = reinterpret_cast<float *>(static_cast<char *>(workspace) +
                                        round_up((size_t)(M * K), 256));
  void *gws = static_cast<char *>(workspace) + round_up((size_t)(M * K), 256) +
              round_up((size_t)M * 4, 256);
  const size_t gws_bytes = workspace_bytes - (need - w8a8::plan_gemm(M, N, K).workspace);
  // The workspace and y must stay clear of the inputs.
  const Range rws = range_of(workspace, (int64_t)need);
  const Range ry = range_of(y, M * N * 2);
  const Range ins[] = {range_of(x, M * K * 2), range_of(w_q, N * K),
                       range_of(w_scale, N * 4),
                       range_of(bias, bias ? N * 2 : 0)};
  for (const Range &r : ins)
    if (overlap(rws, r) || overlap(ry, r)) return W8A8_ERR_ALIAS;
  if (overlap(rws, ry)) return W8A8_ERR_ALIAS;
  GemmPlan plan;
  int st = validate_gemm(aq, sa, w_q, w_scale, bias, y, W8A8_OUT_BF16, M, N, K,
                         gws, gws_bytes, &plan);
  if (st != W8A8_OK) return st;
  if ((st = check_device()) != W8A8_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  st = hip_status(w8a8::launch_quantize_act(x, aq, sa, M, K, false, s));
  if (st != W8A8_OK) return st;
  GemmArgs g{aq, sa, w_q, w_scale, bias, y, W8A8_OUT_BF16,
             M,  N,  K,   gws,     gws_bytes};
  return hip_status(w8a8::launch_gemm(g, plan, s));
}

int w8a8_quantize_weight(const uint16_t *w, int64_t N, int64_t K,
                         int8_t *w_q, float *w_scale, void *stream) {
  int st = validate_quant(w, N, K, w_q, w_scale);
  if (st != W8A8_OK) return st;
  if ((st = check_device()) != W8A8_OK) return st;
  return hip_status(w8a8::launch_quantize_weight(
      w, w_q, w_scale, N, K, static_cast<hipStream_t>(stream)));
}

int w8a8_check_scales(const float *w_scale, int64_t N, int32_t *bad_count,
                      void *stream) {
  if (!w_scale || !bad_count) return W8A8_ERR_NULL;
  if (N < 0 || N > kMaxRows) return W8A8_ERR_SHAPE;
  if (!aligned(w_scale, 4) || !aligned(bad_count, 4)) return W8A8_ERR_ALIGN;
  if (overlap(range_of(w_scale, N * 4), range_of(bad_count, 4)))
    return W8A8_ERR_ALIAS;
  int st = check_device();
  if (st != W8A8_OK) return st;
  return hip_status(w8a8::launch_check_scales(
      w_scale, N, bad_count, static_cast<hipStream_t>(stream)));
}

int w8a8_swiglu_bf16(const uint16_t *h, uint16_t *y, int64_t M, int64_t F,
                     void *stream) {
  if (!h || !y) return W8A8_ERR_NULL;
  if (M < 1 || M > kMaxTokenRows || F < 8 || F % 8 != 0 || F > kMaxRows / 2)
    return W8A8_ERR_SHAPE;
  if (!aligned(h, 16) || !aligned(y, 16)) return W8A8_ERR_ALIGN;
  if (overlap(range_of(h, M * F * 4), range_of(y, M * F * 2)))
    return W8A8_ERR_ALIAS;
  int st = check_device();
  if (st != W8A8_OK) return st;
  return hip_status(
      w8a8::launch_swiglu(h, y, M, F, static_cast<hipStream_t>(stream)));
}

int w8a8_quantize_act_swiglu(const uint16_t *h, int64_t M, int64_t F,
                             int8_t *a_q, float *a_scale, void *stream) {
  if (!h || !a_q || !a_scale) return W8A8_ERR_NULL;
  if (M < 1 || M > kMaxTokenRows || F < 8 || F % 8 != 0 || F > kGlueMaxK)
    return W8A8_ERR_SHAPE;
  if (!aligned(h, 16) || !aligned(a_q, 8) || !aligned(a_scale, 4))
    return W8A8_ERR_ALIGN;
  const Range rh = range_of(h, M * F * 4), rq = range_of(a_q, M * F),
              rs = range_of(a_scale, M * 4);
  if (overlap(rh, rq) || overlap(rh, rs) || overlap(rq, rs))
    return W8A8_ERR_ALIAS;
  int st = check_device();
  if (st != W8A8_OK) return st;
  return hip_status(w8a8::launch_swiglu_quant(
      h, a_q, a_scale, M, F, static_cast<hipStream_t>(stream)));
}

int w8a8_silu_bf16(const uint16_t *x, uint16_t *y, int64_t n, void *stream) {
  if (!x || !y) return W8A8_ERR_NULL;
  if (n < 0 || n % 8 != 0) return W8A8_ERR_SHAPE;
  if (!aligned(x, 16) || !aligned(y, 16)) return W8A8_ERR_ALIGN;
  if (x != y && overlap(range_of(x, n * 2), range_of(y, n * 2)))
    return W8A8_ERR_ALIAS;
  int st = check_device();
  if (st != W8A8_OK) return st;
  return hip_status(
      w8a8::launch_silu(x, y, n, static_cast<hipStream_t>(stream)));
}

int w8a8_pow2_renorm(const uint16_t *x, uint16_t *y, int64_t M, int64_t K,
                     void *stream) {
  if (!x || !y) return W8A8_ERR_NULL;
  if (M < 1 || M > kMaxTokenRows || K < 8 || K % 8 != 0 || K > kGlueMaxK)
    return W8A8_ERR_SHAPE;
  if (!aligned(x, 16) || !aligned(y, 16)) return W8A8_ERR_ALIGN;
  if (x != y && overlap(range_of(x, M * K * 2), range_of(y, M * K * 2)))
    return W8A8_ERR_ALIAS;
  int st = check_device();
  if (st != W8A8_OK) return st;
  return hip_status(w8a8::launch_pow2_renorm(x, y, M, K,
                                              static_cast<hipStream_t>(stream)));
}

int w8a8_pow2_renorm_quantize(const uint16_t *x, int64_t M, int64_t K,
                              uint16_t *y, int8_t *a_q, float *a_scale,
                              void *stream) {
  if (!x || !y || !a_q || !a_scale) return W8A8_ERR_NULL;
  if (M < 1 || M > kMaxTokenRows || K < 8 || K % 8 != 0 || K > kGlueMaxK)
    return W8A8_ERR_SHAPE;
  if (!aligned(x, 16) || !aligned(y, 16) || !aligned(a_q, 8) ||
      !aligned(a_scale, 4))
    return W8A8_ERR_ALIGN;
  const Range rx = range_of(x, M * K * 2), ry = range_of(y, M * K * 2),
              rq = range_of(a_q, M * K), rs = range_of(a_scale, M * 4);
  if ((x != y && overlap(rx, ry)) || overlap(rx, rq) || overlap(rx, rs) ||
      overlap(ry, rq) || overlap(ry, rs) || overlap(rq, rs))
    return W8A8_ERR_ALIAS;
  int st = check_device();
  if (st != W8A8_OK) return st;
  return hip_status(w8a8::launch_pow2_renorm_quant(
      x, y, a_q, a_scale, M, K, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
