// lambda.hip -- per-head lambda of differential attention (lesson
// "Differential Attention V2", section "Concept"):
//   lambda[h] = exp(lq1[h] . lk1[h]) - exp(lq2[h] . lk2[h]) + lambda_init
// One wave per head: each lane accumulates a strided slice of both dot
// products in fp32, a butterfly reduction finishes them, lane 0 writes.
#include "common.hpp"
#include "launch.hpp"

namespace da {

__global__ __launch_bounds__(64) void lambda_kernel(const float *__restrict__ lq1,
                                                    const float *__restrict__ lk1,
                                                    const float *__restrict__ lq2,
                                                    const float *__restrict__ lk2, int d_lambda,
                                                    float lambda_init, float *__restrict__ out) {
    const int h = blockIdx.x;
    const int lane = threadIdx.x;
    const int64_t base = (int64_t)h * d_lambda;
    float d1 = 0.0f, d2 = 0.0f;
    for (int k = lane; k < d_lambda; k += 64) {
        d1 = fmaf(lq1[base + k], lk1[base + k], d1);
        d2 = fmaf(lq2[base + k], lk2[base + k], d2);
    }
    d1 = wave_sum(d1);
    d2 = wave_sum(d2);
    if (lane == 0) out[h] = expf(d1) - expf(d2) + lambda_init;
}

hipError_t launch_lambda(const float *lq1, const float *lk1, const float *lq2, const float *lk2,
                         int H, int d_lambda, float lambda_init, float *out, hipStream_t stream) {
    hipLaunchKernelGGL(lambda_kernel, dim3(H), dim3(64), 0, stream, lq1, lk1, lq2, lk2, d_lambda,
                       lambda_init, out);
    return hipGetLastError();
}

}  // namespace da
