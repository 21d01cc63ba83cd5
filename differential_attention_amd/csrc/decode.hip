// decode.hip -- split-KV paged decode of differential attention, V2 form
// (lesson "Differential Attention V2", section "V1 vs V2": the query heads
// are doubled, the KV heads stay, so the KV cache is loaded once per step and
// every key/value byte feeds all query heads of its group, both branches).
//
// Pass 1 (decode_split_kernel), one work-group per (split s, KV head g,
// sequence b): the pages of the split stream HBM -> registers -> LDS (the
// next page's loads are in flight while the current page is used). All
// 2 * group query rows of the KV head (both branches of every pair) are one
// 16-column MFMA operand, so each K and V page is read from HBM exactly once.
// Each of the 4 waves takes 16 tokens of a page:
//   S^T = K Q^T         16 tokens x 16 query rows, v_mfma_f32_16x16x32_bf16
//   online softmax      per query row (lane % 16), running max / sum
//   O^T += V^T P^T      128 x 16, v_mfma_f32_16x16x16_bf16; the 4 scores a
//                       lane holds are exactly its B-operand k-slots, and V
//                       is transposed into LDS so V^T is read 8 bytes at a time
// At the end the 4 waves' states are merged through LDS and the split's
// (max, sum, unnormalised O) per query row is written to the workspace.
// Pass 2 (decode_combine_kernel), one work-group per (output head, sequence):
// merges the splits of each branch with the log-sum-exp rule, forms
// y = O1 - lambda O2 and, for the V1 norm, y / sqrt(mean(y^2) + eps) *
// gamma * (1 - lambda_init).
// Token t of sequence b is slot t % 64 of page page_table[b][t / 64]; tokens
// at or past ctx_len[b] are masked. A page id outside [0, num_pages) is
// never dereferenced: its tokens are masked and bit 0 of *dev_err is set.
#include "common.hpp"
#include "launch.hpp"

namespace da {

namespace {

typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));

constexpr int kD = 128;      // d_qk = d_v
constexpr int kPage = 64;    // tokens per page
constexpr int kKLd = kD + 8;         // K tile row stride (elements)
constexpr int kVtLd = kPage + 8;     // V^T tile row stride (elements)
constexpr int kKElems = kPage * kKLd;
constexpr int kVtElems = kD * kVtLd;

struct DecodeParams {
    const __bf16 *q1, *q2;
    int64_t sq1[2], sq2[2];
    const __bf16 *kc, *vc;
    const int32_t *page_table, *ctx_len;
    const float *lambda, *gamma;
    __bf16 *out;
    int64_t so[2];
    float *ws;
    int *dev_err;
    int H, H_kv, group, qrows, max_pages, num_pages, split_pages, num_splits, norm;
    float sc_log2, eps, one_minus_init;
};

__device__ __forceinline__ uint4 ldg16(const __bf16 *p) { return *(const uint4 *)p; }

__global__ __launch_bounds__(256) void decode_split_kernel(DecodeParams p) {
    __shared__ __attribute__((aligned(16))) __bf16 lds[kKElems + kVtElems];
    __shared__ float red_m[4][16], red_l[4][16];

    const int s = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int n = lane & 15, grp = lane >> 4;

    const int L = p.ctx_len[b];
    if (L < 1 || L > p.max_pages * kPage) {
        if (tid == 0 && s == 0 && g == 0 && p.dev_err) atomicOr(p.dev_err, 2);
        return;
    }
    const int npages = (L + kPage - 1) / kPage;
    const int pb = s * p.split_pages;
    const int pe = min(npages, pb + p.split_pages);
    if (pb >= pe) return;

    // Q^T fragments: lane supplies query row n, d = 32 kc + 8 grp .. +7
    bf16x8 qf[4];
    {
        const bool ok = n < p.qrows;
        const int pair = n >> 1, br = n & 1;
        const int h = g * p.group + (ok ? pair : 0);
        const __bf16 *q = br ? p.q2 + b * p.sq2[0] + h * p.sq2[1] : p.q1 + b * p.sq1[0] + h * p.sq1[1];
#pragma unroll
        for (int kc = 0; kc < 4; ++kc) {
            uint4 z = {0u, 0u, 0u, 0u};
            qf[kc] = as_bf16x8(ok ? ldg16(q + 32 * kc + 8 * grp) : z);
        }
    }

    const int32_t *table = p.page_table + (int64_t)b * p.max_pages;
    uint4 kr[4], vr[4];
    bool page_ok = true;
    auto load_page = [&](int pg) {
        const int phys = table[pg];
        page_ok = phys >= 0 && phys < p.num_pages;
        const int64_t base = page_ok ? ((int64_t)phys * p.H_kv + g) * kPage : 0;
        const __bf16 *kp = p.kc + base * kD;
        const __bf16 *vp = p.vc + base * kD;
        uint4 z = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int c = tid + 256 * i;
            kr[i] = page_ok ? ldg16(kp + (c >> 4) * kD + (c & 15) * 8) : z;
        }
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int task = tid + 256 * i;
            const int j = task & 31, cg = task >> 5;
            vr[2 * i] = page_ok ? ldg16(vp + (2 * j) * kD + 8 * cg) : z;
            vr[2 * i + 1] = page_ok ? ldg16(vp + (2 * j + 1) * kD + 8 * cg) : z;
        }
    };
    auto store_page = [&]() {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int c = tid + 256 * i;
            *(uint4 *)(lds + (c >> 4) * kKLd + (c & 15) * 8) = kr[i];
        }
        uint32_t *vt = (uint32_t *)(lds + kKElems);
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int task = tid + 256 * i;
            const int j = task & 31, cg = task >> 5;
            const uint4 a = vr[2 * i], c = vr[2 * i + 1];
            const uint32_t aw[4] = {a.x, a.y, a.z, a.w};
            const uint32_t cw[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const uint32_t lo = (e & 1) ? (aw[e >> 1] >> 16) : (aw[e >> 1] & 0xffffu);
                const uint32_t hi = (e & 1) ? (cw[e >> 1] & 0xffff0000u) : (cw[e >> 1] << 16);
                vt[(8 * cg + e) * (kVtLd / 2) + j] = lo | hi;
            }
        }
    };

    f32x4 o[8];
#pragma unroll
    for (int dc = 0; dc < 8; ++dc) o[dc] = f32x4{};
    float m = -INFINITY, l = 0.0f;
    bool bad_page = false;

    load_page(pb);
    for (int pg = pb; pg < pe; ++pg) {
        const bool cur_ok = page_ok;
        bad_page |= !cur_ok;
        __syncthreads();
        store_page();
        __syncthreads();
        if (pg + 1 < pe) load_page(pg + 1);

        // scores of this wave's 16 tokens against the 16 query rows
        f32x4 sc = f32x4{};
        const __bf16 *krp = lds + (16 * wave + n) * kKLd + 8 * grp;
#pragma unroll
        for (int kc = 0; kc < 4; ++kc) sc = mfma16(as_bf16x8(*(const uint4 *)(krp + 32 * kc)), qf[kc], sc);
        const int tok0 = pg * kPage + 16 * wave + 4 * grp;
#pragma unroll
        for (int r = 0; r < 4; ++r)
            if (!cur_ok || tok0 + r >= L) sc[r] = -INFINITY;
        float mx = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
        mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        const float mnew = fmaxf(m, mx * p.sc_log2);
        const float alpha = (m == mnew) ? 1.0f : exp2_fast(m - mnew);
        const float msub = (mnew == -INFINITY) ? 0.0f : mnew;
        m = mnew;
        float pr[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) pr[r] = exp2_fast(fmaf(sc[r], p.sc_log2, -msub));
        l = l * alpha + (pr[0] + pr[1]) + (pr[2] + pr[3]);
        if (alpha != 1.0f) {
#pragma unroll
            for (int dc = 0; dc < 8; ++dc) o[dc] *= alpha;
        }
        const bf16x2 p01 = pack2(pr[0], pr[1]), p23 = pack2(pr[2], pr[3]);
        const bf16x4_t pb4 = {p01[0], p01[1], p23[0], p23[1]};
        const __bf16 *vrp = lds + kKElems + n * kVtLd + 16 * wave + 4 * grp;
#pragma unroll
        for (int dc = 0; dc < 8; ++dc) {
            const bf16x4_t va = *(const bf16x4_t *)(vrp + 16 * dc * kVtLd);
            o[dc] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, pb4, o[dc], 0, 0, 0);
        }
    }
    if (bad_page && tid == 0 && p.dev_err) atomicOr(p.dev_err, 1);

    // row sums over the 4 lane groups that share a query row
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);

    // merge the 4 waves through LDS (the K/V staging area is free now)
    __syncthreads();
    float *ow = (float *)lds;  // [4 waves][16 rows][128 dv]
#pragma unroll
    for (int dc = 0; dc < 8; ++dc)
#pragma unroll
        for (int r = 0; r < 4; ++r) ow[(wave * 16 + n) * kD + 16 * dc + 4 * grp + r] = o[dc][r];
    if (grp == 0) {
        red_m[wave][n] = m;
        red_l[wave][n] = l;
    }
    __syncthreads();
    float *rec = p.ws + (((int64_t)b * p.H_kv + g) * p.num_splits + s) * p.qrows * (kD + 2);
    for (int idx = tid; idx < p.qrows * kD; idx += 256) {
        const int q = idx / kD, dv = idx % kD;
        float M = fmaxf(fmaxf(red_m[0][q], red_m[1][q]), fmaxf(red_m[2][q], red_m[3][q]));
        float acc = 0.0f, lsum = 0.0f;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const float mw = red_m[w][q];
            const float f = (mw == -INFINITY) ? 0.0f : exp2_fast(mw - M);
            acc += ow[(w * 16 + q) * kD + dv] * f;
            lsum += red_l[w][q] * f;
        }
        float *rq = rec + q * (kD + 2);
        rq[dv] = acc;
        if (dv == 0) {
            rq[kD] = M;
            rq[kD + 1] = lsum;
        }
    }
}

__global__ __launch_bounds__(128) void decode_combine_kernel(DecodeParams p) {
    __shared__ float red[2];
    const int h = blockIdx.x, b = blockIdx.y, dv = threadIdx.x;
    const int g = h / p.group, j = h - g * p.group;
    const int L = p.ctx_len[b];
    __bf16 *op = p.out + b * p.so[0] + h * p.so[1];
    if (L < 1 || L > p.max_pages * kPage) {
        op[dv] = (__bf16)0.0f;
        return;
    }
    const int npages = (L + kPage - 1) / kPage;
    const int ns = (npages + p.split_pages - 1) / p.split_pages;
    const float *base = p.ws + ((int64_t)b * p.H_kv + g) * p.num_splits * p.qrows * (kD + 2);
    float ob[2];
#pragma unroll
    for (int br = 0; br < 2; ++br) {
        const int q = 2 * j + br;
        float M = -INFINITY;
        for (int s = 0; s < ns; ++s) M = fmaxf(M, base[((int64_t)s * p.qrows + q) * (kD + 2) + kD]);
        float acc = 0.0f, lsum = 0.0f;
        for (int s = 0; s < ns; ++s) {
            const float *rq = base + ((int64_t)s * p.qrows + q) * (kD + 2);
            const float ms = rq[kD];
            const float f = (ms == -INFINITY) ? 0.0f : exp2_fast(ms - M);
            acc += rq[dv] * f;
            lsum += rq[kD + 1] * f;
        }
        ob[br] = lsum > 0.0f ? acc / lsum : 0.0f;
    }
    float y;
    {
#pragma clang fp contract(off)
        y = ob[0] - p.lambda[h] * ob[1];
    }
    if (p.norm) {
        float ss = wave_sum(y * y);
        if ((dv & 63) == 0) red[dv >> 6] = ss;
        __syncthreads();
        ss = red[0] + red[1];
        y *= p.one_minus_init / sqrtf(ss * (1.0f / kD) + p.eps) * p.gamma[(int64_t)h * kD + dv];
    }
    op[dv] = (__bf16)y;
}

}  // namespace

hipError_t launch_decode_bf16(const diffattn_decode_args &a, const DecodePlan &plan, void *workspace,
                              float scale, float lambda_init, hipStream_t stream) {
    DecodeParams p;
    p.q1 = (const __bf16 *)a.q1;
    p.q2 = (const __bf16 *)a.q2;
    for (int k = 0; k < 2; ++k) {
        p.sq1[k] = a.sq1[k];
        p.sq2[k] = a.sq2[k];
        p.so[k] = a.so[k];
    }
    p.kc = (const __bf16 *)a.k1_cache;
    p.vc = (const __bf16 *)a.v_cache;
    p.page_table = a.page_table;
    p.ctx_len = a.ctx_len;
    p.lambda = a.lambda;
    p.gamma = a.gamma;
    p.out = (__bf16 *)a.out;
    p.ws = (float *)workspace;
    p.dev_err = a.dev_err;
    p.H = a.H;
    p.H_kv = a.H_kv;
    p.group = a.H / a.H_kv;
    p.qrows = plan.qrows;
    p.max_pages = a.max_pages;
    p.num_pages = a.num_pages;
    p.split_pages = plan.split_pages;
    p.num_splits = plan.num_splits;
    p.norm = a.norm == DIFFATTN_NORM_RMS;
    p.sc_log2 = scale * kLog2e;
    p.eps = a.eps;
    p.one_minus_init = 1.0f - lambda_init;
    hipLaunchKernelGGL(decode_split_kernel, dim3(plan.num_splits, a.H_kv, a.B), dim3(256), 0, stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(decode_combine_kernel, dim3(a.H, a.B), dim3(128), 0, stream, p);
    return hipGetLastError();
}

}  // namespace da
