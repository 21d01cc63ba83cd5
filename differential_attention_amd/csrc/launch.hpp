// launch.hpp -- internal interface between the C ABI (api.cpp) and the
// kernel translation units. Host code only; not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>

#include "diffattn.h"
#include "plan.hpp"

namespace da {

hipError_t launch_lambda(const float *lq1, const float *lk1, const float *lq2, const float *lk2,
                         int H, int d_lambda, float lambda_init, float *out, hipStream_t stream);

hipError_t launch_prefill_f32(const diffattn_prefill_args &a, float scale, float lambda_init,
                              hipStream_t stream);

hipError_t launch_prefill_bf16(const diffattn_prefill_args &a, float scale, float lambda_init,
                               hipStream_t stream);

hipError_t launch_backward_bf16(const diffattn_backward_args &a, const BackwardPlan &plan, void *workspace,
                                float scale, float lambda_init, hipStream_t stream);

hipError_t launch_lambda_backward(const float *lq1, const float *lk1, const float *lq2, const float *lk2, int H,
                                  int d_lambda, const float *dlambda, float *dlq1, float *dlk1, float *dlq2,
                                  float *dlk2, hipStream_t stream);

hipError_t launch_decode_bf16(const diffattn_decode_args &a, const DecodePlan &plan, void *workspace,
                              float scale, float lambda_init, hipStream_t stream);

// Device address of the current device's static decode scratch
// (kDecodeScratchBytes), looked up once per device.
hipError_t decode_scratch(void **ptr);

}  // namespace da
