// prefill_f32.hip -- fp32 differential-attention prefill (the accuracy path).
//
// Computes, per (batch b, output head h, query row i), with g = h / (H / H_kv):
//   A_br = softmax(q_br . k_br[g, j] * scale)   over the visible keys j
//   y    = (A_1 - lambda[h] A_2) V[g]            (lesson "Differential
//          Attention V2", section "Concept")
//   V1:  y <- y / sqrt(mean(y^2) + eps) * gamma[h] * (1 - lambda_init)
// Visible keys: j <= i when causal (lesson "Attention Variants", "Build it",
// step 1), else all N; with a causal window W also j >= i - W + 1 (same
// lesson, step 2).
//
// One wave per query row, fp32 throughout. The softmax is exact two-pass
// per row (first the maxima of both branches, then exponentials, sums and
// the value accumulation), each lane owning one key per 64-key chunk;
// probabilities reach the value loop through cross-lane broadcasts, so no
// shared memory or block barrier is needed and rows of different lengths
// never wait for each other. Sizes: d_qk, d_v <= 128.
#include "common.hpp"
#include "launch.hpp"

namespace da {

struct PrefillF32Params {
    const float *q1, *q2, *k1, *k2, *v;
    int64_t sq1[3], sq2[3], sk1[3], sk2[3], sv[3], so[3];
    const float *lambda, *gamma;
    float *out;
    float *o1, *o2, *lse1, *lse2;  // optional statistics for the backward pass (all or none)
    int H, group, N, d_qk, d_v, causal, window, norm;
    float scale, eps, one_minus_init;
};

__device__ __forceinline__ float dot_row(const float *__restrict__ q, const float *__restrict__ k, int d) {
    float acc = 0.0f;
    for (int t = 0; t < d; ++t) acc = fmaf(q[t], k[t], acc);
    return acc;
}

__global__ __launch_bounds__(256) void prefill_f32_kernel(PrefillF32Params p) {
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int i = blockIdx.x * 4 + wave;
    if (i >= p.N) return;  // whole wave leaves; no block-level synchronisation below
    const int h = blockIdx.y, b = blockIdx.z, g = h / p.group;

    const float *q1 = p.q1 + b * p.sq1[0] + h * p.sq1[1] + (int64_t)i * p.sq1[2];
    const float *q2 = p.q2 + b * p.sq2[0] + h * p.sq2[1] + (int64_t)i * p.sq2[2];
    const float *k1 = p.k1 + b * p.sk1[0] + g * p.sk1[1];
    const float *k2 = p.k2 + b * p.sk2[0] + g * p.sk2[1];
    const float *v = p.v + b * p.sv[0] + g * p.sv[1];
    const int kend = p.causal ? i + 1 : p.N;
    const int kbeg = p.window > 0 ? max(0, i - p.window + 1) : 0;

    // pass 1: row maxima of the scaled scores of both branches
    float m1 = -INFINITY, m2 = -INFINITY;
    for (int j0 = kbeg; j0 < kend; j0 += 64) {
        const int j = j0 + lane;
        if (j < kend) {
            m1 = fmaxf(m1, dot_row(q1, k1 + (int64_t)j * p.sk1[2], p.d_qk) * p.scale);
            m2 = fmaxf(m2, dot_row(q2, k2 + (int64_t)j * p.sk2[2], p.d_qk) * p.scale);
        }
    }
    m1 = wave_max(m1);
    m2 = wave_max(m2);

    // pass 2: exponentials, sums and the value accumulation of both branches
    const int c0 = lane, c1 = lane + 64;
    float l1 = 0.0f, l2 = 0.0f;
    float o1a = 0.0f, o1b = 0.0f, o2a = 0.0f, o2b = 0.0f;
    for (int j0 = kbeg; j0 < kend; j0 += 64) {
        const int j = j0 + lane;
        float e1 = 0.0f, e2 = 0.0f;
        if (j < kend) {
            e1 = expf(dot_row(q1, k1 + (int64_t)j * p.sk1[2], p.d_qk) * p.scale - m1);
            e2 = expf(dot_row(q2, k2 + (int64_t)j * p.sk2[2], p.d_qk) * p.scale - m2);
        }
        l1 += e1;
        l2 += e2;
        const int cnt = min(64, kend - j0);
        for (int t = 0; t < cnt; ++t) {
            const float w1 = __shfl(e1, t, 64);
            const float w2 = __shfl(e2, t, 64);
            const float *vr = v + (int64_t)(j0 + t) * p.sv[2];
            if (c0 < p.d_v) {
                const float x = vr[c0];
                o1a = fmaf(w1, x, o1a);
                o2a = fmaf(w2, x, o2a);
            }
            if (c1 < p.d_v) {
                const float x = vr[c1];
                o1b = fmaf(w1, x, o1b);
                o2b = fmaf(w2, x, o2b);
            }
        }
    }
    l1 = wave_sum(l1);
    l2 = wave_sum(l2);

    if (p.o1) {
        // each branch's normalised output and natural-log log-sum-exp
        const int64_t rowid = ((int64_t)b * p.H + h) * p.N + i;
        float *a1 = p.o1 + rowid * p.d_v, *a2 = p.o2 + rowid * p.d_v;
        if (c0 < p.d_v) {
            a1[c0] = o1a / l1;
            a2[c0] = o2a / l2;
        }
        if (c1 < p.d_v) {
            a1[c1] = o1b / l1;
            a2[c1] = o2b / l2;
        }
        if (lane == 0) {
            p.lse1[rowid] = m1 + logf(l1);
            p.lse2[rowid] = m2 + logf(l2);
        }
    }
    const float lam = p.lambda[h];
    const float r1 = 1.0f / l1, r2 = lam / l2;
    float ya, yb;
    {
#pragma clang fp contract(off)
        ya = c0 < p.d_v ? o1a * r1 - o2a * r2 : 0.0f;
        yb = c1 < p.d_v ? o1b * r1 - o2b * r2 : 0.0f;
    }
    if (p.norm) {
        if (p.norm == 2) {  // GroupNorm per head: subtract the channel mean first
            const float mu = wave_sum((c0 < p.d_v ? ya : 0.0f) + (c1 < p.d_v ? yb : 0.0f)) / (float)p.d_v;
            if (c0 < p.d_v) ya -= mu;
            if (c1 < p.d_v) yb -= mu;
        }
        const float ss = wave_sum(ya * ya + yb * yb);
        const float rs = p.one_minus_init / sqrtf(ss / (float)p.d_v + p.eps);
        if (c0 < p.d_v) ya *= rs * p.gamma[(int64_t)h * p.d_v + c0];
        if (c1 < p.d_v) yb *= rs * p.gamma[(int64_t)h * p.d_v + c1];
    }
    float *o = p.out + b * p.so[0] + h * p.so[1] + (int64_t)i * p.so[2];
    if (c0 < p.d_v) o[c0] = ya;
    if (c1 < p.d_v) o[c1] = yb;
}

hipError_t launch_prefill_f32(const diffattn_prefill_args &a, float scale, float lambda_init,
                              hipStream_t stream) {
    PrefillF32Params p;
    p.q1 = (const float *)a.q1;
    p.q2 = (const float *)a.q2;
    p.k1 = (const float *)a.k1;
    p.k2 = (const float *)a.k2;
    p.v = (const float *)a.v;
    for (int k = 0; k < 3; ++k) {
        p.sq1[k] = a.sq1[k];
        p.sq2[k] = a.sq2[k];
        p.sk1[k] = a.sk1[k];
        p.sk2[k] = a.sk2[k];
        p.sv[k] = a.sv[k];
        p.so[k] = a.so[k];
    }
    p.lambda = a.lambda;
    p.gamma = a.gamma;
    p.out = (float *)a.out;
    p.o1 = a.o1;
    p.o2 = a.o2;
    p.lse1 = a.lse1;
    p.lse2 = a.lse2;
    p.H = a.H;
    p.group = a.H / a.H_kv;
    p.N = a.N;
    p.d_qk = a.d_qk;
    p.d_v = a.d_v;
    p.causal = a.causal;
    p.window = a.window;
    p.norm = a.norm;  // 0 none, 1 RMS, 2 GroupNorm
    p.scale = scale;
    p.eps = a.eps;
    p.one_minus_init = 1.0f - lambda_init;
    dim3 grid((a.N + 3) / 4, a.H, a.B);
    hipLaunchKernelGGL(prefill_f32_kernel, grid, dim3(256), 0, stream, p);
    return hipGetLastError();
}

}  // namespace da
