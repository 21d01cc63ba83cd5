// plan.cpp -- host-only argument validation and launch planning (no HIP).
#include "plan.hpp"

#include <math.h>
#include <string.h>

#include <algorithm>
#include <vector>

namespace da {

double lambda_init(int depth) {
    if (depth < 1) return NAN;
    return 0.8 - 0.6 * exp(-0.3 * (double)(depth - 1));
}

namespace {

int fail(std::string *msg, int code, const std::string &text) {
    if (msg) *msg = text;
    return code;
}

// A strided tensor: byte extent [lo, hi) and whether its elements are distinct.
struct Extent {
    uintptr_t lo = 0, hi = 0;
};

struct Dim {
    int64_t size, stride;
};

// Byte extent of a tensor with the given dims (element strides, all >= 0).
bool extent_of(const void *p, size_t elem, const std::vector<Dim> &dims, Extent *e) {
    int64_t last = 0;
    for (const Dim &d : dims) {
        if (d.size <= 0) return false;
        if (d.stride < 0) return false;
        if (d.stride > 0 && (d.size - 1) > INT64_MAX / d.stride) return false;
        last += (d.size - 1) * d.stride;
        if (last < 0) return false;
    }
    e->lo = (uintptr_t)p;
    e->hi = e->lo + (uintptr_t)(last + 1) * elem;
    return true;
}

// True when no two index tuples map to the same element: after sorting the
// non-trivial dims by stride, each stride covers the span of the smaller ones.
bool non_overlapping(std::vector<Dim> dims) {
    dims.erase(std::remove_if(dims.begin(), dims.end(), [](const Dim &d) { return d.size == 1; }),
               dims.end());
    std::sort(dims.begin(), dims.end(), [](const Dim &a, const Dim &b) { return a.stride < b.stride; });
    int64_t span = 1;  // elements covered by the dims seen so far
    for (const Dim &d : dims) {
        if (d.stride < span) return false;
        span = d.stride * (d.size - 1) + span;
    }
    return true;
}

bool overlaps(const Extent &a, const Extent &b) { return a.lo < b.hi && b.lo < a.hi; }

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

}  // namespace

int check_lambda(const float *lq1, const float *lk1, const float *lq2, const float *lk2, int H,
                 int d_lambda, int depth, const float *out, std::string *msg) {
    if (H < 1) return fail(msg, DIFFATTN_EINVAL, "diffattn_lambda: H must be >= 1");
    if (d_lambda < 1 || d_lambda > 4096)
        return fail(msg, DIFFATTN_EINVAL, "diffattn_lambda: d_lambda must be in [1, 4096]");
    if (depth < 1) return fail(msg, DIFFATTN_EINVAL, "diffattn_lambda: depth must be >= 1");
    if (!lq1 || !lk1 || !lq2 || !lk2 || !out)
        return fail(msg, DIFFATTN_EINVAL, "diffattn_lambda: null pointer");
    const void *ins[4] = {lq1, lk1, lq2, lk2};
    for (const void *p : ins)
        if (!aligned(p, 4)) return fail(msg, DIFFATTN_EINVAL, "diffattn_lambda: misaligned input");
    if (!aligned(out, 4)) return fail(msg, DIFFATTN_EINVAL, "diffattn_lambda: misaligned output");
    Extent eo{(uintptr_t)out, (uintptr_t)out + (uintptr_t)H * 4};
    for (const void *p : ins) {
        Extent ei{(uintptr_t)p, (uintptr_t)p + (uintptr_t)H * d_lambda * 4};
        if (overlaps(eo, ei))
            return fail(msg, DIFFATTN_EINVAL, "diffattn_lambda: output overlaps an input");
    }
    return DIFFATTN_OK;
}

int check_lambda_backward(const float *lq1, const float *lk1, const float *lq2, const float *lk2, int H,
                          int d_lambda, const float *dlambda, const float *dlq1, const float *dlk1,
                          const float *dlq2, const float *dlk2, std::string *msg) {
    if (H < 1) return fail(msg, DIFFATTN_EINVAL, "diffattn_lambda_backward: H must be >= 1");
    if (d_lambda < 1 || d_lambda > 4096)
        return fail(msg, DIFFATTN_EINVAL, "diffattn_lambda_backward: d_lambda must be in [1, 4096]");
    const float *ins[5] = {lq1, lk1, lq2, lk2, dlambda};
    const float *outs[4] = {dlq1, dlk1, dlq2, dlk2};
    for (const float *p : ins)
        if (!p) return fail(msg, DIFFATTN_EINVAL, "diffattn_lambda_backward: null pointer");
    for (const float *p : outs)
        if (!p) return fail(msg, DIFFATTN_EINVAL, "diffattn_lambda_backward: null pointer");
    for (const float *p : ins)
        if (!aligned(p, 4)) return fail(msg, DIFFATTN_EINVAL, "diffattn_lambda_backward: misaligned input");
    for (const float *p : outs)
        if (!aligned(p, 4)) return fail(msg, DIFFATTN_EINVAL, "diffattn_lambda_backward: misaligned output");
    const uintptr_t vec = (uintptr_t)H * (uintptr_t)d_lambda * 4;
    Extent ei[5], eo[4];
    for (int i = 0; i < 5; ++i)
        ei[i] = Extent{(uintptr_t)ins[i], (uintptr_t)ins[i] + (i < 4 ? vec : (uintptr_t)H * 4)};
    for (int i = 0; i < 4; ++i) eo[i] = Extent{(uintptr_t)outs[i], (uintptr_t)outs[i] + vec};
    // the kernel reads every input while it writes the outputs: no output may
    // share memory with an input or with another output
    for (int i = 0; i < 4; ++i) {
        for (int j = 0; j < 5; ++j)
            if (overlaps(eo[i], ei[j]))
                return fail(msg, DIFFATTN_EINVAL, "diffattn_lambda_backward: an output overlaps an input");
        for (int j = i + 1; j < 4; ++j)
            if (overlaps(eo[i], eo[j]))
                return fail(msg, DIFFATTN_EINVAL, "diffattn_lambda_backward: outputs overlap");
    }
    return DIFFATTN_OK;
}

int check_prefill(const diffattn_prefill_args *a, PrefillPlan *plan, std::string *msg) {
    *plan = PrefillPlan();
    if (!a) return fail(msg, DIFFATTN_EINVAL, "diffattn_prefill: null argument struct");
    if (a->dtype != DIFFATTN_BF16 && a->dtype != DIFFATTN_F32)
        return fail(msg, DIFFATTN_EINVAL, "diffattn_prefill: unknown dtype");
    if (a->B < 0 || a->N < 0) return fail(msg, DIFFATTN_EINVAL, "diffattn_prefill: B and N must be >= 0");
    if (a->H < 1 || a->H_kv < 1) return fail(msg, DIFFATTN_EINVAL, "diffattn_prefill: H and H_kv must be >= 1");
    if (a->H % a->H_kv != 0)
        return fail(msg, DIFFATTN_EINVAL, "diffattn_prefill: H must be a multiple of H_kv");
    if (a->d_qk < 1 || a->d_v < 1) return fail(msg, DIFFATTN_EINVAL, "diffattn_prefill: d_qk and d_v must be >= 1");
    if (a->depth < 1) return fail(msg, DIFFATTN_EINVAL, "diffattn_prefill: depth must be >= 1");
    if (a->causal != 0 && a->causal != 1) return fail(msg, DIFFATTN_EINVAL, "diffattn_prefill: causal must be 0 or 1");
    if (a->window < 0 || (a->window > 0 && !a->causal))
        return fail(msg, DIFFATTN_EINVAL, "diffattn_prefill: window must be 0, or > 0 with causal");
    const int nstats = (a->o1 != nullptr) + (a->o2 != nullptr) + (a->lse1 != nullptr) + (a->lse2 != nullptr);
    if (nstats != 0 && nstats != 4)
        return fail(msg, DIFFATTN_EINVAL, "diffattn_prefill: set all of o1, o2, lse1, lse2 or none");
    if (a->norm != DIFFATTN_NORM_NONE && a->norm != DIFFATTN_NORM_RMS && a->norm != DIFFATTN_NORM_GROUP)
        return fail(msg, DIFFATTN_EINVAL, "diffattn_prefill: unknown norm");
    if (!(a->scale >= 0.0f) || isinf(a->scale))
        return fail(msg, DIFFATTN_EINVAL, "diffattn_prefill: scale must be finite and >= 0");
    if (a->norm != DIFFATTN_NORM_NONE && !(a->eps > 0.0f && !isinf(a->eps)))
        return fail(msg, DIFFATTN_EINVAL, "diffattn_prefill: eps must be finite and > 0");

    if (a->dtype == DIFFATTN_BF16) {
        bool ok = (a->d_qk == 64 && a->d_v == 128) || (a->d_qk == 128 && a->d_v == 128);
        if (!ok)
            return fail(msg, DIFFATTN_EUNSUPPORTED,
                        "diffattn_prefill: bf16 supports (d_qk, d_v) = (64, 128) or (128, 128)");
        plan->kind = PrefillKind::Bf16;
    } else {
        if (a->d_qk > 128 || a->d_v > 128)
            return fail(msg, DIFFATTN_EUNSUPPORTED, "diffattn_prefill: f32 supports d_qk, d_v <= 128");
        plan->kind = PrefillKind::F32;
    }
    if (a->B == 0 || a->N == 0) {
        plan->empty = true;
        return DIFFATTN_OK;
    }
    if (!a->q1 || !a->q2 || !a->k1 || !a->k2 || !a->v || !a->lambda || !a->out)
        return fail(msg, DIFFATTN_EINVAL, "diffattn_prefill: null tensor pointer");
    if (a->norm != DIFFATTN_NORM_NONE && !a->gamma)
        return fail(msg, DIFFATTN_EINVAL, "diffattn_prefill: a norm needs gamma");

    const size_t elem = a->dtype == DIFFATTN_BF16 ? 2 : 4;
    const size_t align = a->dtype == DIFFATTN_BF16 ? 16 : 4;
    const int64_t smul = a->dtype == DIFFATTN_BF16 ? 8 : 1;
    struct T {
        const char *name;
        const void *p;
        const int64_t *s;
        int64_t h, d;
    } ts[6] = {{"q1", a->q1, a->sq1, a->H, a->d_qk},   {"q2", a->q2, a->sq2, a->H, a->d_qk},
               {"k1", a->k1, a->sk1, a->H_kv, a->d_qk}, {"k2", a->k2, a->sk2, a->H_kv, a->d_qk},
               {"v", a->v, a->sv, a->H_kv, a->d_v},     {"out", a->out, a->so, a->H, a->d_v}};
    Extent ext[6];
    for (int i = 0; i < 6; ++i) {
        const T &t = ts[i];
        for (int k = 0; k < 3; ++k)
            if (t.s[k] < 0 || t.s[k] % smul != 0)
                return fail(msg, DIFFATTN_EINVAL,
                            std::string("diffattn_prefill: stride of ") + t.name +
                                (a->dtype == DIFFATTN_BF16 ? " must be a non-negative multiple of 8"
                                                           : " must be non-negative"));
        if (!aligned(t.p, align))
            return fail(msg, DIFFATTN_EINVAL, std::string("diffattn_prefill: ") + t.name + " is misaligned");
        std::vector<Dim> dims = {{a->B, t.s[0]}, {t.h, t.s[1]}, {a->N, t.s[2]}, {t.d, 1}};
        if (!extent_of(t.p, elem, dims, &ext[i]))
            return fail(msg, DIFFATTN_EINVAL, std::string("diffattn_prefill: bad strides for ") + t.name);
        if (i == 5 && !non_overlapping(dims))
            return fail(msg, DIFFATTN_EINVAL, "diffattn_prefill: out has overlapping elements");
    }
    if (!aligned(a->lambda, 4) || (a->gamma && a->norm != DIFFATTN_NORM_NONE && !aligned(a->gamma, 4)))
        return fail(msg, DIFFATTN_EINVAL, "diffattn_prefill: lambda/gamma misaligned");
    Extent lam{(uintptr_t)a->lambda, (uintptr_t)a->lambda + (uintptr_t)a->H * 4};
    for (int i = 0; i < 5; ++i)
        if (overlaps(ext[5], ext[i]))
            return fail(msg, DIFFATTN_EINVAL, std::string("diffattn_prefill: out overlaps ") + ts[i].name);
    if (overlaps(ext[5], lam)) return fail(msg, DIFFATTN_EINVAL, "diffattn_prefill: out overlaps lambda");
    if (a->norm != DIFFATTN_NORM_NONE) {
        Extent g{(uintptr_t)a->gamma, (uintptr_t)a->gamma + (uintptr_t)a->H * a->d_v * 4};
        if (overlaps(ext[5], g)) return fail(msg, DIFFATTN_EINVAL, "diffattn_prefill: out overlaps gamma");
    }
    if (a->o1) {
        const uintptr_t rows = (uintptr_t)a->B * a->H * a->N;
        Extent st[4] = {{(uintptr_t)a->o1, (uintptr_t)a->o1 + rows * a->d_v * 4},
                        {(uintptr_t)a->o2, (uintptr_t)a->o2 + rows * a->d_v * 4},
                        {(uintptr_t)a->lse1, (uintptr_t)a->lse1 + rows * 4},
                        {(uintptr_t)a->lse2, (uintptr_t)a->lse2 + rows * 4}};
        if (!aligned(a->o1, 16) || !aligned(a->o2, 16) || !aligned(a->lse1, 4) || !aligned(a->lse2, 4))
            return fail(msg, DIFFATTN_EINVAL, "diffattn_prefill: statistics misaligned");
        for (int x = 0; x < 4; ++x) {
            for (int y = x + 1; y < 4; ++y)
                if (overlaps(st[x], st[y])) return fail(msg, DIFFATTN_EINVAL, "diffattn_prefill: statistics overlap");
            for (int t = 0; t < 6; ++t)
                if (overlaps(st[x], ext[t]))
                    return fail(msg, DIFFATTN_EINVAL, "diffattn_prefill: statistics overlap an input or out");
        }
    }
    plan->shared_k = a->k1 == a->k2 && a->sk1[0] == a->sk2[0] && a->sk1[1] == a->sk2[1] &&
                     a->sk1[2] == a->sk2[2];
    return DIFFATTN_OK;
}

int check_decode_sizes(const diffattn_decode_args *a, DecodePlan *plan, std::string *msg) {
    *plan = DecodePlan();
    if (!a) return fail(msg, DIFFATTN_EINVAL, "diffattn_decode: null argument struct");
    if (a->dtype != DIFFATTN_BF16 && a->dtype != DIFFATTN_F32)
        return fail(msg, DIFFATTN_EINVAL, "diffattn_decode: unknown dtype");
    if (a->B < 0) return fail(msg, DIFFATTN_EINVAL, "diffattn_decode: B must be >= 0");
    if (a->H < 1 || a->H_kv < 1 || a->H % a->H_kv != 0)
        return fail(msg, DIFFATTN_EINVAL, "diffattn_decode: need H >= 1, H_kv >= 1, H % H_kv == 0");
    if (a->d_qk < 1 || a->d_v < 1 || a->page_size < 1 || a->max_pages < 1 || a->num_pages < 1)
        return fail(msg, DIFFATTN_EINVAL, "diffattn_decode: sizes must be >= 1");
    if (a->depth < 1) return fail(msg, DIFFATTN_EINVAL, "diffattn_decode: depth must be >= 1");
    if (a->norm != DIFFATTN_NORM_NONE && a->norm != DIFFATTN_NORM_RMS && a->norm != DIFFATTN_NORM_GROUP)
        return fail(msg, DIFFATTN_EINVAL, "diffattn_decode: unknown norm");
    if (!(a->scale >= 0.0f) || isinf(a->scale))
        return fail(msg, DIFFATTN_EINVAL, "diffattn_decode: scale must be finite and >= 0");
    if (a->norm != DIFFATTN_NORM_NONE && !(a->eps > 0.0f && !isinf(a->eps)))
        return fail(msg, DIFFATTN_EINVAL, "diffattn_decode: eps must be finite and > 0");
    if (a->window < 0) return fail(msg, DIFFATTN_EINVAL, "diffattn_decode: window must be >= 0");
    if (a->kv_dtype != DIFFATTN_BF16 && a->kv_dtype != DIFFATTN_FP8_E4M3)
        return fail(msg, DIFFATTN_EINVAL, "diffattn_decode: kv_dtype must be bf16 or fp8 e4m3");
    if (a->kv_dtype == DIFFATTN_FP8_E4M3 && !(a->k_scale > 0.0f && !isinf(a->k_scale) && a->v_scale > 0.0f &&
                                               !isinf(a->v_scale)))
        return fail(msg, DIFFATTN_EINVAL, "diffattn_decode: fp8 caches need finite k_scale, v_scale > 0");
    if (a->split_pages < 0 || a->split_pages > kDecodeMaxTarget)
        return fail(msg, DIFFATTN_EINVAL, "diffattn_decode: split_pages must be in [0, 2^24]");
    if ((int64_t)a->B * a->max_pages > INT32_MAX)
        return fail(msg, DIFFATTN_EINVAL, "diffattn_decode: B * max_pages must fit in 31 bits");
    if ((int64_t)a->B * a->H_kv * a->max_pages > ((int64_t)1 << 40))
        return fail(msg, DIFFATTN_EINVAL, "diffattn_decode: B * H_kv * max_pages must be <= 2^40");
    if ((int64_t)a->max_pages * a->page_size > (1 << 30))
        return fail(msg, DIFFATTN_EINVAL, "diffattn_decode: max_pages * page_size too large");
    if (a->dtype != DIFFATTN_BF16 || (a->d_qk != 128 && a->d_qk != 64) || a->d_v != 128 || a->page_size != 64)
        return fail(msg, DIFFATTN_EUNSUPPORTED,
                    "diffattn_decode: supports bf16 with d_qk in {64, 128}, d_v = 128 and page_size 64");
    const int group = a->H / a->H_kv;
    if (group > 8)
        return fail(msg, DIFFATTN_EUNSUPPORTED, "diffattn_decode: at most 8 output heads per KV head");
    if (a->d_qk == 128 && a->k1_cache != a->k2_cache)
        return fail(msg, DIFFATTN_EUNSUPPORTED,
                    "diffattn_decode: with d_qk = 128 the branches must share the key cache");

    // plan: the split pass has at most max_wgs work-groups; the records hold one
    // partial state per (work-group, unit) pair, of which there are fewer than
    // work-groups + units (consecutive ranges share at most one unit)
    const int64_t units = (int64_t)a->B * a->H_kv;
    const int64_t most_pages = units * a->max_pages;
    const int64_t per_wg = a->split_pages > 0 ? a->split_pages : kDecodeMinPages;
    plan->target_pages = a->split_pages;
    plan->max_wgs = (int)std::max<int64_t>(1, std::min<int64_t>(kDecodeMaxWgs, (most_pages + per_wg - 1) / per_wg));
    plan->qrows = 2 * group;
    plan->header_bytes = ((size_t)(a->B + 1) * sizeof(int32_t) + 255) / 256 * 256;
    plan->record_bytes = (size_t)plan->qrows * (a->d_v + 2) * sizeof(float);
    plan->ws_bytes = a->B > 0 ? plan->header_bytes + (size_t)(plan->max_wgs + units) * plan->record_bytes : 0;

    return DIFFATTN_OK;
}

int check_decode(const diffattn_decode_args *a, DecodePlan *plan, std::string *msg) {
    int rc = check_decode_sizes(a, plan, msg);
    if (rc != DIFFATTN_OK || a->B == 0) return rc;
    if (!a->q1 || !a->q2 || !a->k1_cache || !a->k2_cache || !a->v_cache || !a->page_table || !a->ctx_len ||
        !a->lambda || !a->out)
        return fail(msg, DIFFATTN_EINVAL, "diffattn_decode: null pointer");
    if (a->norm != DIFFATTN_NORM_NONE && !a->gamma)
        return fail(msg, DIFFATTN_EINVAL, "diffattn_decode: a norm needs gamma");
    const int64_t strides[6] = {a->sq1[0], a->sq1[1], a->sq2[0], a->sq2[1], a->so[0], a->so[1]};
    for (int64_t s : strides)
        if (s < 0 || s % 8 != 0)
            return fail(msg, DIFFATTN_EINVAL, "diffattn_decode: strides must be non-negative multiples of 8");
    const void *al16[] = {a->q1, a->q2, a->k1_cache, a->k2_cache, a->v_cache, a->out};
    for (const void *p : al16)
        if (!aligned(p, 16)) return fail(msg, DIFFATTN_EINVAL, "diffattn_decode: tensor not 16-byte aligned");
    if (!aligned(a->page_table, 4) || !aligned(a->ctx_len, 4) || !aligned(a->lambda, 4))
        return fail(msg, DIFFATTN_EINVAL, "diffattn_decode: int/float array misaligned");
    Extent eo, e;
    std::vector<Dim> od = {{a->B, a->so[0]}, {a->H, a->so[1]}, {a->d_v, 1}};
    if (!extent_of(a->out, 2, od, &eo) || !non_overlapping(od))
        return fail(msg, DIFFATTN_EINVAL, "diffattn_decode: bad output strides");
    const int64_t kv_elems = (int64_t)a->num_pages * a->H_kv * a->page_size;
    const size_t kv_b = a->kv_dtype == DIFFATTN_FP8_E4M3 ? 1 : 2;
    struct R {
        const void *p;
        size_t bytes;
    } rs[] = {{a->k1_cache, (size_t)kv_elems * a->d_qk * kv_b},
              {a->k2_cache, (size_t)kv_elems * a->d_qk * kv_b},
              {a->v_cache, (size_t)kv_elems * a->d_v * kv_b},
              {a->page_table, (size_t)a->B * a->max_pages * 4},
              {a->ctx_len, (size_t)a->B * 4},
              {a->lambda, (size_t)a->H * 4}};
    for (const R &r : rs) {
        e.lo = (uintptr_t)r.p;
        e.hi = e.lo + r.bytes;
        if (overlaps(eo, e)) return fail(msg, DIFFATTN_EINVAL, "diffattn_decode: out overlaps an input");
    }
    const void *qs[2] = {a->q1, a->q2};
    const int64_t *qstr[2] = {a->sq1, a->sq2};
    for (int i = 0; i < 2; ++i) {
        std::vector<Dim> qd = {{a->B, qstr[i][0]}, {a->H, qstr[i][1]}, {a->d_qk, 1}};
        if (!extent_of(qs[i], 2, qd, &e)) return fail(msg, DIFFATTN_EINVAL, "diffattn_decode: bad q strides");
        if (overlaps(eo, e)) return fail(msg, DIFFATTN_EINVAL, "diffattn_decode: out overlaps q");
    }
    return DIFFATTN_OK;
}

namespace {

diffattn_prefill_args prefill_view(const diffattn_backward_args *a) {
    diffattn_prefill_args p;
    memset(&p, 0, sizeof(p));
    p.dtype = a->dtype;
    p.B = a->B;
    p.H = a->H;
    p.H_kv = a->H_kv;
    p.N = a->N;
    p.d_qk = a->d_qk;
    p.d_v = a->d_v;
    p.q1 = a->q1;
    p.q2 = a->q2;
    p.k1 = a->k1;
    p.k2 = a->k2;
    p.v = a->v;
    for (int i = 0; i < 3; ++i) {
        p.sq1[i] = a->sq1[i];
        p.sq2[i] = a->sq2[i];
        p.sk1[i] = a->sk1[i];
        p.sk2[i] = a->sk2[i];
        p.sv[i] = a->sv[i];
        p.so[i] = a->sdo[i];
    }
    p.lambda = a->lambda;
    p.depth = a->depth;
    p.causal = a->causal;
    p.window = a->window;
    p.scale = a->scale;
    p.norm = a->norm;
    p.gamma = a->gamma;
    p.eps = a->eps;
    p.out = const_cast<void *>(a->dout);  // validated like an output: shape, strides, no overlap
    return p;
}

size_t round256(size_t x) { return (x + 255) / 256 * 256; }

int backward_common(const diffattn_backward_args *a, BackwardPlan *plan, std::string *msg, bool pointers) {
    *plan = BackwardPlan();
    if (!a) return fail(msg, DIFFATTN_EINVAL, "diffattn_backward: null argument struct");
    // the inputs are those of a prefill (dout standing in for its output);
    // sizes only: the same checks on an empty batch, which stop before pointers
    diffattn_prefill_args pa = prefill_view(a);
    if (!pointers && pa.B > 0) pa.B = 0;
    PrefillPlan pp;
    std::string m;
    const int rc = check_prefill(&pa, &pp, &m);
    if (rc != DIFFATTN_OK) {
        std::string t = m;
        const std::string from = "diffattn_prefill";
        if (t.compare(0, from.size(), from) == 0) t = "diffattn_backward" + t.substr(from.size());
        return fail(msg, rc, t);
    }
    if (a->dtype != DIFFATTN_BF16)
        return fail(msg, DIFFATTN_EUNSUPPORTED, "diffattn_backward: supports bf16 inputs");
    plan->shared_k = a->k1 == a->k2 && a->sk1[0] == a->sk2[0] && a->sk1[1] == a->sk2[1] && a->sk1[2] == a->sk2[2];
    plan->rows = (int64_t)a->B * a->H * a->N;
    plan->prep_blocks = (int64_t)a->B * a->H * ((a->N + kBwdPrepRows - 1) / kBwdPrepRows);
    plan->empty = a->B == 0 || a->N == 0;
    size_t off = 0;
    plan->off_dy = off;
    off += round256((size_t)plan->rows * a->d_v * 2);
    plan->off_dt1 = off;
    off += round256((size_t)plan->rows * 4);
    plan->off_dt2 = off;
    off += round256((size_t)plan->rows * 4);
    plan->off_ls1 = off;
    off += round256((size_t)plan->rows * 4);
    plan->off_ls2 = off;
    off += round256((size_t)plan->rows * 4);
    plan->off_part = off;
    off += round256((size_t)plan->prep_blocks * (1 + a->d_v) * 4);
    plan->ws_bytes = plan->empty ? 0 : off;
    return DIFFATTN_OK;
}

}  // namespace

int check_backward_sizes(const diffattn_backward_args *a, BackwardPlan *plan, std::string *msg) {
    return backward_common(a, plan, msg, false);
}

int check_backward(const diffattn_backward_args *a, BackwardPlan *plan, std::string *msg) {
    int rc = backward_common(a, plan, msg, true);
    if (rc != DIFFATTN_OK || plan->empty) return rc;
    if (!a->o1 || !a->o2 || !a->lse1 || !a->lse2 || !a->dout)
        return fail(msg, DIFFATTN_EINVAL, "diffattn_backward: null statistics or dout");
    if (!a->dq1 || !a->dq2 || !a->dk1 || !a->dv || !a->dlambda)
        return fail(msg, DIFFATTN_EINVAL, "diffattn_backward: null gradient output");
    if (plan->shared_k) {
        if (a->dk2 && a->dk2 != a->dk1)
            return fail(msg, DIFFATTN_EINVAL, "diffattn_backward: with one key tensor dk2 must be NULL or dk1");
    } else if (!a->dk2 || a->dk2 == a->dk1) {
        return fail(msg, DIFFATTN_EINVAL, "diffattn_backward: two key tensors need two key gradients");
    }
    if (a->norm != DIFFATTN_NORM_NONE && !a->dgamma)
        return fail(msg, DIFFATTN_EINVAL, "diffattn_backward: a norm needs dgamma");
    const void *al16[] = {a->o1, a->o2, a->dq1, a->dq2, a->dk1, a->dk2 ? a->dk2 : a->dk1, a->dv};
    for (const void *p : al16)
        if (!aligned(p, 16)) return fail(msg, DIFFATTN_EINVAL, "diffattn_backward: fp32 tensor not 16-byte aligned");
    if (!aligned(a->lse1, 4) || !aligned(a->lse2, 4) || !aligned(a->dlambda, 4) ||
        (a->dgamma && !aligned(a->dgamma, 4)))
        return fail(msg, DIFFATTN_EINVAL, "diffattn_backward: fp32 array misaligned");

    // outputs must not overlap each other or any input
    const uintptr_t rows = (uintptr_t)plan->rows;
    const uintptr_t kvrows = (uintptr_t)a->B * a->H_kv * a->N;
    auto E = [](const void *p, uintptr_t bytes) { return Extent{(uintptr_t)p, (uintptr_t)p + bytes}; };
    std::vector<Extent> outs = {E(a->dq1, rows * a->d_qk * 4), E(a->dq2, rows * a->d_qk * 4),
                                E(a->dk1, kvrows * a->d_qk * 4), E(a->dv, kvrows * a->d_v * 4),
                                E(a->dlambda, (uintptr_t)a->H * 4)};
    if (!plan->shared_k) outs.push_back(E(a->dk2, kvrows * a->d_qk * 4));
    if (a->norm != DIFFATTN_NORM_NONE) outs.push_back(E(a->dgamma, (uintptr_t)a->H * a->d_v * 4));
    std::vector<Extent> ins = {E(a->o1, rows * a->d_v * 4), E(a->o2, rows * a->d_v * 4), E(a->lse1, rows * 4),
                               E(a->lse2, rows * 4), E(a->lambda, (uintptr_t)a->H * 4)};
    if (a->norm != DIFFATTN_NORM_NONE && a->gamma) ins.push_back(E(a->gamma, (uintptr_t)a->H * a->d_v * 4));
    // the strided bf16 inputs, by their extents
    struct T {
        const void *p;
        const int64_t *s;
        int64_t h, d;
    } ts[] = {{a->q1, a->sq1, a->H, a->d_qk}, {a->q2, a->sq2, a->H, a->d_qk}, {a->k1, a->sk1, a->H_kv, a->d_qk},
              {a->k2, a->sk2, a->H_kv, a->d_qk}, {a->v, a->sv, a->H_kv, a->d_v}, {a->dout, a->sdo, a->H, a->d_v}};
    for (const T &t : ts) {
        Extent e;
        std::vector<Dim> dims = {{a->B, t.s[0]}, {t.h, t.s[1]}, {a->N, t.s[2]}, {t.d, 1}};
        if (!extent_of(t.p, 2, dims, &e)) return fail(msg, DIFFATTN_EINVAL, "diffattn_backward: bad strides");
        ins.push_back(e);
    }
    for (size_t i = 0; i < outs.size(); ++i) {
        for (size_t j = i + 1; j < outs.size(); ++j)
            if (overlaps(outs[i], outs[j])) return fail(msg, DIFFATTN_EINVAL, "diffattn_backward: gradient outputs overlap");
        for (const Extent &e : ins)
            if (overlaps(outs[i], e)) return fail(msg, DIFFATTN_EINVAL, "diffattn_backward: a gradient overlaps an input");
    }
    return DIFFATTN_OK;
}

}  // namespace da
