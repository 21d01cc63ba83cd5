// plan_driver.cpp -- runs the host-side argument validation of libdiffattn
// (plan.cpp, no HIP) over valid and invalid arguments, for a build with
// AddressSanitizer and UndefinedBehaviorSanitizer. Exits non-zero when a
// status differs from the expected one; the sanitizers abort on any memory
// error or undefined behaviour.
#include <stdint.h>
#include <stdio.h>

#include <string>

#include "plan.hpp"

namespace {

int failures = 0;

void expect(int got, int want, const char *what) {
    if (got != want) {
        fprintf(stderr, "%s: status %d, expected %d\n", what, got, want);
        ++failures;
    }
}

const uintptr_t kBase = (uintptr_t)0x7F0000000000ull;  // fake device addresses, never dereferenced
const void *fake(uintptr_t off) { return (const void *)(kBase + off); }

diffattn_prefill_args prefill_args() {
    diffattn_prefill_args a = {};
    a.dtype = DIFFATTN_BF16;
    a.B = 2, a.H = 4, a.H_kv = 2, a.N = 300, a.d_qk = 64, a.d_v = 128;
    const uintptr_t step = 1u << 24;
    a.q1 = fake(0), a.q2 = fake(step), a.k1 = fake(2 * step), a.k2 = fake(3 * step), a.v = fake(4 * step);
    const int64_t sq[3] = {4 * 300 * 64, 300 * 64, 64}, sk[3] = {2 * 300 * 64, 300 * 64, 64},
                  sv[3] = {2 * 300 * 128, 300 * 128, 128}, so[3] = {4 * 300 * 128, 300 * 128, 128};
    for (int i = 0; i < 3; ++i) {
        a.sq1[i] = a.sq2[i] = sq[i];
        a.sk1[i] = a.sk2[i] = sk[i];
        a.sv[i] = sv[i];
        a.so[i] = so[i];
    }
    a.lambda = (const float *)fake(5 * step);
    a.depth = 3, a.causal = 1, a.scale = 0.0f, a.norm = DIFFATTN_NORM_RMS;
    a.gamma = (const float *)fake(6 * step);
    a.eps = 1e-5f;
    a.out = (void *)fake(7 * step);
    return a;
}

diffattn_decode_args decode_args() {
    diffattn_decode_args a = {};
    a.dtype = DIFFATTN_BF16;
    a.B = 16, a.H = 8, a.H_kv = 2, a.d_qk = 128, a.d_v = 128, a.page_size = 64, a.max_pages = 40;
    a.num_pages = 500;
    const uintptr_t step = (uintptr_t)1 << 32;
    a.q1 = fake(0), a.q2 = fake(256);
    a.sq1[0] = a.sq2[0] = 16 * 128, a.sq1[1] = a.sq2[1] = 256;
    a.k1_cache = a.k2_cache = fake(step);
    a.v_cache = fake(2 * step);
    a.page_table = (const int32_t *)fake(3 * step);
    a.ctx_len = (const int32_t *)fake(3 * step + (1 << 20));
    a.lambda = (const float *)fake(3 * step + (2 << 20));
    a.depth = 20, a.norm = DIFFATTN_NORM_NONE, a.eps = 1e-5f;
    a.out = (void *)fake(3 * step + (3 << 20));
    a.so[0] = 8 * 128, a.so[1] = 128;
    return a;
}

diffattn_backward_args backward_args() {
    diffattn_backward_args a = {};
    a.dtype = DIFFATTN_BF16;
    a.B = 1, a.H = 4, a.H_kv = 2, a.N = 128, a.d_qk = 64, a.d_v = 128;
    const uintptr_t step = 1u << 24;
    a.q1 = fake(0), a.q2 = fake(step), a.k1 = fake(2 * step), a.k2 = fake(3 * step), a.v = fake(4 * step);
    for (int i = 0; i < 3; ++i) {
        const int64_t q[3] = {4 * 128 * 64, 128 * 64, 64}, k[3] = {2 * 128 * 64, 128 * 64, 64},
                      v[3] = {2 * 128 * 128, 128 * 128, 128}, o[3] = {4 * 128 * 128, 128 * 128, 128};
        a.sq1[i] = a.sq2[i] = q[i];
        a.sk1[i] = a.sk2[i] = k[i];
        a.sv[i] = v[i];
        a.sdo[i] = o[i];
    }
    a.lambda = (const float *)fake(5 * step);
    a.depth = 3, a.causal = 1, a.norm = DIFFATTN_NORM_NONE, a.eps = 1e-5f;
    a.o1 = (const float *)fake(6 * step), a.o2 = (const float *)fake(7 * step);
    a.lse1 = (const float *)fake(8 * step), a.lse2 = (const float *)fake(9 * step);
    a.dout = fake(10 * step);
    a.dq1 = (float *)fake(11 * step), a.dq2 = (float *)fake(12 * step), a.dk1 = (float *)fake(13 * step);
    a.dk2 = (float *)fake(14 * step), a.dv = (float *)fake(15 * step), a.dlambda = (float *)fake(16 * step);
    return a;
}

}  // namespace

int main() {
    std::string msg;
    // prefill
    {
        da::PrefillPlan plan;
        diffattn_prefill_args a = prefill_args();
        expect(da::check_prefill(&a, &plan, &msg), DIFFATTN_OK, "prefill valid");
        a = prefill_args(), a.H = 3;
        expect(da::check_prefill(&a, &plan, &msg), DIFFATTN_EINVAL, "prefill H % H_kv");
        a = prefill_args(), a.d_qk = 96;
        expect(da::check_prefill(&a, &plan, &msg), DIFFATTN_EUNSUPPORTED, "prefill d_qk 96");
        a = prefill_args(), a.out = (void *)a.q1;
        expect(da::check_prefill(&a, &plan, &msg), DIFFATTN_EINVAL, "prefill alias");
        a = prefill_args(), a.so[2] = 64;
        expect(da::check_prefill(&a, &plan, &msg), DIFFATTN_EINVAL, "prefill overlapping rows");
        a = prefill_args(), a.window = 8, a.causal = 0;
        expect(da::check_prefill(&a, &plan, &msg), DIFFATTN_EINVAL, "prefill window without causal");
        a = prefill_args(), a.N = 0, a.q1 = nullptr;
        expect(da::check_prefill(&a, &plan, &msg), DIFFATTN_OK, "prefill empty");
        a = prefill_args(), a.sq1[2] = (int64_t)1 << 62;
        expect(da::check_prefill(&a, &plan, &msg), DIFFATTN_EINVAL, "prefill huge stride");
        a = prefill_args(), a.B = 0x7fffffff, a.N = 0x7fffffff;
        (void)da::check_prefill(&a, &plan, &msg);  // must not overflow (UBSan), whatever the status
        a = prefill_args(), a.dtype = DIFFATTN_F32, a.d_qk = 48, a.d_v = 80;
        (void)da::check_prefill(&a, &plan, &msg);
    }
    // decode
    {
        da::DecodePlan plan;
        diffattn_decode_args a = decode_args();
        expect(da::check_decode(&a, &plan, &msg), DIFFATTN_OK, "decode valid");
        expect(da::check_decode_sizes(&a, &plan, &msg), DIFFATTN_OK, "decode sizes");
        if (plan.ws_bytes == 0) ++failures;
        a = decode_args(), a.page_size = 32;
        expect(da::check_decode(&a, &plan, &msg), DIFFATTN_EUNSUPPORTED, "decode page 32");
        a = decode_args(), a.split_pages = -1;
        expect(da::check_decode(&a, &plan, &msg), DIFFATTN_EINVAL, "decode split -1");
        a = decode_args(), a.kv_dtype = DIFFATTN_FP8_E4M3, a.k_scale = 0.5f, a.v_scale = 0.25f;
        expect(da::check_decode(&a, &plan, &msg), DIFFATTN_OK, "decode fp8");
        a.k_scale = 0.0f;
        expect(da::check_decode(&a, &plan, &msg), DIFFATTN_EINVAL, "decode fp8 zero scale");
        a = decode_args(), a.out = (void *)a.q1;
        expect(da::check_decode(&a, &plan, &msg), DIFFATTN_EINVAL, "decode alias");
        a = decode_args(), a.max_pages = 0x7fffffff, a.B = 0x7fffffff;
        (void)da::check_decode_sizes(&a, &plan, &msg);
    }
    // backward
    {
        da::BackwardPlan plan;
        diffattn_backward_args a = backward_args();
        expect(da::check_backward(&a, &plan, &msg), DIFFATTN_OK, "backward valid");
        a = backward_args(), a.dk2 = nullptr;
        expect(da::check_backward(&a, &plan, &msg), DIFFATTN_EINVAL, "backward missing dk2");
        a = backward_args(), a.dq2 = a.dq1;
        expect(da::check_backward(&a, &plan, &msg), DIFFATTN_EINVAL, "backward outputs overlap");
        a = backward_args(), a.norm = DIFFATTN_NORM_RMS;
        expect(da::check_backward(&a, &plan, &msg), DIFFATTN_EINVAL, "backward norm without gamma");
    }
    // lambda and its gradients
    {
        const float *p[5];
        for (int i = 0; i < 5; ++i) p[i] = (const float *)fake(4096u * (unsigned)i);
        float *o = (float *)fake(65536);
        expect(da::check_lambda(p[0], p[1], p[2], p[3], 4, 8, 1, o, &msg), DIFFATTN_OK, "lambda valid");
        expect(da::check_lambda(p[0], p[1], p[2], p[3], 4, 8, 1, (float *)p[1] + 2, &msg), DIFFATTN_EINVAL,
               "lambda alias");
        float *d[4];
        for (int i = 0; i < 4; ++i) d[i] = (float *)fake(65536 + 4096u * (unsigned)i);
        expect(da::check_lambda_backward(p[0], p[1], p[2], p[3], 4, 8, p[4], d[0], d[1], d[2], d[3], &msg),
               DIFFATTN_OK, "lambda backward valid");
        expect(da::check_lambda_backward(p[0], p[1], p[2], p[3], 4, 8, p[4], (float *)p[0], d[1], d[2], d[3], &msg),
               DIFFATTN_EINVAL, "lambda backward in place");
        expect(da::check_lambda_backward(p[0], p[1], p[2], p[3], 0x7fffffff, 4096, p[4], d[0], d[1], d[2], d[3],
                                         &msg),
               DIFFATTN_EINVAL, "lambda backward huge");
    }
    if (failures) {
        fprintf(stderr, "%d unexpected statuses\n", failures);
        return 1;
    }
    printf("plan checks ok\n");
    return 0;
}
