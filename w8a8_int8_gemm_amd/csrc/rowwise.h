// rowwise.h -- launchers of the per-token kernels added beside the
// quantizer: weight quantization, the scale check and the SwiGLU glue.
// Not part of the public ABI (include/w8a8.h); arguments are validated by
// the API layer before these are called.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w8a8 {

hipError_t launch_quantize_weight(const uint16_t *w, int8_t *q, float *sw,
                                  int64_t N, int64_t K, hipStream_t stream);
hipError_t launch_check_scales(const float *sw, int64_t N, int *bad,
                               hipStream_t stream);
hipError_t launch_swiglu(const uint16_t *h, uint16_t *y, int64_t M, int64_t F,
                         hipStream_t stream);
hipError_t launch_swiglu_quant(const uint16_t *h, int8_t *q, float *scale,
                               int64_t M, int64_t F, hipStream_t stream);
hipError_t launch_pow2_renorm_quant(const uint16_t *x, uint16_t *y, int8_t *q,
                                    float *sa, int64_t M, int64_t K,
                                    hipStream_t stream);

}  // namespace w8a8
