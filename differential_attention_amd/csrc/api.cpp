// api.cpp -- the extern "C" entry points of libdiffattn. Validates on the host
// (plan.cpp), then enqueues the gfx950 kernels on the caller's stream.
#include <math.h>

#include <string>

#include "launch.hpp"
#include "plan.hpp"

namespace {

thread_local std::string g_last_error;

int set_error(int code, const std::string &m) {
    g_last_error = m;
    return code;
}

int hip_status(hipError_t e, const char *where) {
    if (e == hipSuccess) e = hipGetLastError();
    if (e != hipSuccess)
        return set_error(DIFFATTN_EHIP, std::string(where) + ": " + hipGetErrorString(e));
    g_last_error.clear();
    return DIFFATTN_OK;
}

}  // namespace

extern "C" {

double diffattn_lambda_init(int depth) { return da::lambda_init(depth); }

const char *diffattn_last_error(void) { return g_last_error.c_str(); }

int diffattn_lambda(const float *lq1, const float *lk1, const float *lq2, const float *lk2, int H,
                    int d_lambda, int depth, float *lambda_out, void *stream) {
    std::string msg;
    int rc = da::check_lambda(lq1, lk1, lq2, lk2, H, d_lambda, depth, lambda_out, &msg);
    if (rc != DIFFATTN_OK) return set_error(rc, msg);
    hipError_t e = da::launch_lambda(lq1, lk1, lq2, lk2, H, d_lambda, (float)da::lambda_init(depth),
                                     lambda_out, (hipStream_t)stream);
    return hip_status(e, "diffattn_lambda");
}

int diffattn_prefill(const diffattn_prefill_args *a, void *stream) {
    std::string msg;
    da::PrefillPlan plan;
    int rc = da::check_prefill(a, &plan, &msg);
    if (rc != DIFFATTN_OK) return set_error(rc, msg);
    if (plan.empty) {
        g_last_error.clear();
        return DIFFATTN_OK;
    }
    const float scale = a->scale > 0.0f ? a->scale : (float)(1.0 / sqrt((double)a->d_qk));
    const float init = (float)da::lambda_init(a->depth);
    hipError_t e = plan.kind == da::PrefillKind::Bf16
                       ? da::launch_prefill_bf16(*a, scale, init, (hipStream_t)stream)
                       : da::launch_prefill_f32(*a, scale, init, (hipStream_t)stream);
    return hip_status(e, "diffattn_prefill");
}

size_t diffattn_decode_workspace_bytes(const diffattn_decode_args *a) {
    da::DecodePlan plan;
    std::string msg;
    if (da::check_decode_sizes(a, &plan, &msg) != DIFFATTN_OK) return 0;
    return plan.ws_bytes;
}

int diffattn_decode(const diffattn_decode_args *a, void *workspace, size_t ws_bytes, void *stream) {
    std::string msg;
    da::DecodePlan plan;
    int rc = da::check_decode(a, &plan, &msg);
    if (rc != DIFFATTN_OK) return set_error(rc, msg);
    if (a->B == 0) {
        g_last_error.clear();
        return DIFFATTN_OK;
    }
    if (!workspace || ws_bytes < plan.ws_bytes)
        return set_error(DIFFATTN_EWORKSPACE, "diffattn_decode: workspace missing or smaller than "
                                              "diffattn_decode_workspace_bytes()");
    if (((uintptr_t)workspace % 256) != 0)
        return set_error(DIFFATTN_EWORKSPACE, "diffattn_decode: workspace must be 256-byte aligned");
    const float scale = a->scale > 0.0f ? a->scale : (float)(1.0 / sqrt((double)a->d_qk));
    hipError_t e = da::launch_decode_bf16(*a, plan, workspace, scale, (float)da::lambda_init(a->depth),
                                          (hipStream_t)stream);
    return hip_status(e, "diffattn_decode");
}

int diffattn_decode_noalloc(const diffattn_decode_args *a, void *stream) {
    std::string msg;
    da::DecodePlan plan;
    int rc = da::check_decode(a, &plan, &msg);
    if (rc != DIFFATTN_OK) return set_error(rc, msg);
    if (a->B == 0) {
        g_last_error.clear();
        return DIFFATTN_OK;
    }
    if (plan.ws_bytes > da::kDecodeScratchBytes)
        return set_error(DIFFATTN_EWORKSPACE,
                         "diffattn_decode_noalloc: these arguments need " + std::to_string(plan.ws_bytes) +
                             " bytes of scratch, more than the " + std::to_string(da::kDecodeScratchBytes) +
                             " of the static scratch (diffattn_decode takes a workspace of any size)");
    void *ws = nullptr;
    hipError_t e = da::decode_scratch(&ws);
    if (e != hipSuccess) return hip_status(e, "diffattn_decode_noalloc (scratch lookup)");
    const float scale = a->scale > 0.0f ? a->scale : (float)(1.0 / sqrt((double)a->d_qk));
    e = da::launch_decode_bf16(*a, plan, ws, scale, (float)da::lambda_init(a->depth), (hipStream_t)stream);
    return hip_status(e, "diffattn_decode_noalloc");
}

size_t diffattn_backward_workspace_bytes(const diffattn_backward_args *a) {
    da::BackwardPlan plan;
    std::string msg;
    if (da::check_backward_sizes(a, &plan, &msg) != DIFFATTN_OK) return 0;
    return plan.ws_bytes;
}

int diffattn_backward(const diffattn_backward_args *a, void *workspace, size_t ws_bytes, void *stream) {
    std::string msg;
    da::BackwardPlan plan;
    int rc = da::check_backward(a, &plan, &msg);
    if (rc != DIFFATTN_OK) return set_error(rc, msg);
    if (plan.empty) {
        g_last_error.clear();
        return DIFFATTN_OK;
    }
    if (!workspace || ws_bytes < plan.ws_bytes)
        return set_error(DIFFATTN_EWORKSPACE, "diffattn_backward: workspace missing or smaller than "
                                              "diffattn_backward_workspace_bytes()");
    if (((uintptr_t)workspace % 256) != 0)
        return set_error(DIFFATTN_EWORKSPACE, "diffattn_backward: workspace must be 256-byte aligned");
    const float scale = a->scale > 0.0f ? a->scale : (float)(1.0 / sqrt((double)a->d_qk));
    hipError_t e = da::launch_backward_bf16(*a, plan, workspace, scale, (float)da::lambda_init(a->depth),
                                            (hipStream_t)stream);
    return hip_status(e, "diffattn_backward");
}

int diffattn_lambda_backward(const float *lq1, const float *lk1, const float *lq2, const float *lk2, int H,
                             int d_lambda, const float *dlambda, float *dlq1, float *dlk1, float *dlq2,
                             float *dlk2, void *stream) {
    std::string msg;
    int rc = da::check_lambda_backward(lq1, lk1, lq2, lk2, H, d_lambda, dlambda, dlq1, dlk1, dlq2, dlk2, &msg);
    if (rc != DIFFATTN_OK) return set_error(rc, msg);
    hipError_t e = da::launch_lambda_backward(lq1, lk1, lq2, lk2, H, d_lambda, dlambda, dlq1, dlk1, dlq2, dlk2,
                                              (hipStream_t)stream);
    return hip_status(e, "diffattn_lambda_backward");
}

}  // extern "C"
