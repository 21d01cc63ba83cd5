/*
 * diffattn.h -- C ABI of libdiffattn, differential attention on AMD Instinct
 * MI355X (gfx950).
 *
 * The operation (lesson "Differential Attention V2", AI Engineering from
 * Scratch phase 10 lesson 16, section "Concept"): for each head, two softmax
 * maps A1 = softmax(Q1 K1^T / sqrt(d)) and A2 = softmax(Q2 K2^T / sqrt(d)),
 * and the output (A1 - lambda * A2) V, with a learnable per-head scalar
 * lambda = exp(lq1 . lk1) - exp(lq2 . lk2) + lambda_init.
 * Forms (same lesson, section "V1 vs V2"):
 *   V1: the head dimension is halved (d_qk = d_v / 2 in the usual setup) and
 *       a per-head RMSNorm follows the difference; this library scales the
 *       normalised output by gamma[h] * (1 - lambda_init).
 *   V2: the query heads are doubled while the KV heads stay as in GQA; both
 *       queries of a pair read the same KV head; no norm.
 * Causal mask (lesson "Attention Variants", phase 7 lesson 15, "Build it",
 * step 1): key j is visible to query i iff j <= i. Causal sliding window of
 * W keys (same lesson, step 2 and the sliding-window figure of "Concept"):
 * key j is visible iff i - W + 1 <= j <= i; W >= N is the full causal mask.
 * Key tiles wholly outside every row's window are never loaded.
 *
 * Conventions shared by every entry point:
 *  - Every tensor pointer is DEVICE memory owned by the caller. The library
 *    never allocates, frees or synchronises; all work is enqueued on `stream`
 *    (a hipStream_t passed as void*, NULL = the default stream) and the call
 *    returns once it is enqueued.
 *  - Strides are in elements; the innermost (feature) stride is always 1.
 *  - Arguments are checked on the host before anything is launched; on an
 *    error the call returns a negative status, launches nothing and leaves
 *    every output untouched. diffattn_last_error() then describes it.
 *  - DIFFATTN_EHIP means a launch was attempted and the HIP runtime reported
 *    an error (for example, no device); outputs are then undefined.
 *  - The library holds no state between calls apart from a per-device
 *    cache of the compute-unit count and kernel occupancy and the static
 *    scratch of diffattn_decode_noalloc, and is safe to call from several
 *    host threads (the last-error message is thread-local).
 */
#ifndef DIFFATTN_H
#define DIFFATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    DIFFATTN_OK = 0,
    DIFFATTN_EINVAL = -1,       /* bad pointer, size, stride, alignment or alias */
    DIFFATTN_EUNSUPPORTED = -2, /* valid, but no kernel for this dtype/size combination */
    DIFFATTN_EWORKSPACE = -3,   /* decode workspace missing or too small */
    DIFFATTN_EHIP = -4          /* the HIP runtime reported an error */
};

enum {
    DIFFATTN_BF16 = 0,
    DIFFATTN_F32 = 1,
    DIFFATTN_FP8_E4M3 = 2  /* KV-cache storage only: OCP fp8 e4m3 (bias 7, no infinities,
                              0x7f / 0xff are NaN), one byte per element */
};
enum {
    DIFFATTN_NORM_NONE = 0,  /* V2 */
    DIFFATTN_NORM_RMS = 1,   /* V1: y / sqrt(mean(y^2) + eps) * gamma * (1 - lambda_init) */
    DIFFATTN_NORM_GROUP = 2  /* V1 variant, GroupNorm with one group per head:
                                (y - mean y) / sqrt(var(y) + eps) * gamma * (1 - lambda_init) */
};

/*
 * Prefill arguments. Shapes:
 *   q1, q2 [B, H, N, d_qk]      H = output heads (one (Q1, Q2) pair each)
 *   k1, k2 [B, H_kv, N, d_qk]   H % H_kv == 0; output head h reads KV head
 *                               h / (H / H_kv). k1 == k2 with equal strides
 *                               (V2) is allowed and loads each key tile once.
 *   v      [B, H_kv, N, d_v]
 *   out    [B, H, N, d_v]       must not overlap any input
 * s* arrays hold the element strides of dimensions (b, h, n).
 * dtype DIFFATTN_BF16: all tensors bf16, (d_qk, d_v) in {(64,128), (128,128)},
 * strides multiples of 8 and pointers 16-byte aligned.
 * dtype DIFFATTN_F32: all tensors fp32, 1 <= d_qk, d_v <= 128, 4-byte aligned.
 */
typedef struct {
    int dtype;
    int B, H, H_kv, N, d_qk, d_v;
    const void *q1, *q2;
    const void *k1, *k2;
    const void *v;
    int64_t sq1[3], sq2[3], sk1[3], sk2[3], sv[3];
    const float *lambda; /* [H] fp32 device (diffattn_lambda, or any values) */
    int depth;           /* >= 1; lambda_init(depth) feeds the V1 (1 - lambda_init) scale */
    int causal;          /* 0 or 1 */
    float scale;         /* score scale; 0 selects 1/sqrt(d_qk) */
    int norm;            /* DIFFATTN_NORM_NONE, _RMS or _GROUP */
    const float *gamma;  /* RMS / GROUP: [H, d_v] fp32 device gain; NONE: ignored (may be NULL) */
    float eps;           /* RMSNorm epsilon, > 0 */
    void *out;
    int64_t so[3];
    int window;          /* 0: none; W > 0 (causal only): row i sees keys i-W+1 .. i */
    /* Optional statistics for the backward pass (all four set, or all NULL):
     * o1, o2 fp32 [B, H, N, d_v] contiguous: each branch's normalised output
     * softmax(Q_k K_k^T scale) V; lse1, lse2 fp32 [B, H, N] contiguous: the
     * natural-log log-sum-exp of each branch's scaled, masked scores per row. */
    float *o1, *o2;
    float *lse1, *lse2;
} diffattn_prefill_args;

/*
 * Paged-decode arguments: one new query token per sequence attends to the
 * ctx_len[b] tokens held in a paged KV cache (the new token's key and value
 * already written). Token t of sequence b lives in physical page
 * page_table[b * max_pages + t / page_size], slot t % page_size.
 *   q1, q2      [B, H, d_qk]                  strides sq*[0] (b), sq*[1] (h)
 *   k1_cache,
 *   k2_cache    [num_pages, H_kv, page_size, d_qk] contiguous; one cache for
 *               both branches (V2, k1 == k2) or one per branch (V1)
 *   v_cache     [num_pages, H_kv, page_size, d_v]  contiguous, read once for
 *               both branches
 *   page_table  [B, max_pages] int32 device
 *   ctx_len     [B] int32 device, 1 <= ctx_len[b] <= max_pages * page_size
 *   out         [B, H, d_v]                   strides so[0], so[1]
 * Supported: dtype DIFFATTN_BF16, d_v 128, page_size 64, H / H_kv <= 8
 * output heads per KV head, and d_qk 128 with k1_cache == k2_cache (V2) or
 * d_qk 64 with any two key caches (V1); the caches bf16 or fp8 (kv_dtype).
 * split_pages: pages per work-group of the split-KV pass, 0..2^24. The pages
 * of all (sequence, KV head) pairs are cut into equal contiguous ranges, one
 * per work-group (at most 2048); 0 lets the library use one round of the
 * work-groups the device holds at once (at least 4 pages each).
 * window: causal sliding window (0 = none); pages wholly before the window
 * are neither counted nor read.
 * dev_err: optional device int; bit 0 is OR-ed in when a page id outside
 * [0, num_pages) is met, bit 1 when a ctx_len is out of range. Such pages or
 * sequences are skipped (never read). NULL disables the report (the checks
 * that keep reads in bounds still run).
 */
typedef struct {
    int dtype;
    int B, H, H_kv, d_qk, d_v, page_size, max_pages, num_pages;
    const void *q1, *q2;
    int64_t sq1[2], sq2[2];
    const void *k1_cache, *k2_cache, *v_cache;
    const int32_t *page_table;
    const int32_t *ctx_len;
    const float *lambda;
    int depth;
    float scale;
    int norm;
    const float *gamma;
    float eps;
    void *out;
    int64_t so[2];
    int split_pages;
    int *dev_err;
    int window;          /* 0: none; W > 0: the query sees tokens ctx_len-W .. ctx_len-1 */
    /* KV-cache storage: DIFFATTN_BF16 (0), or DIFFATTN_FP8_E4M3 with one byte
     * per element in the same layouts, the key caches dequantised as
     * k_scale * code and the value cache as v_scale * code (per-tensor scales,
     * finite and > 0; ignored for bf16). Queries and output stay bf16. */
    int kv_dtype;
    float k_scale, v_scale;
} diffattn_decode_args;

/*
 * lambda_init(depth) = 0.8 - 0.6 exp(-0.3 (depth - 1)), the default depth
 * schedule on the lesson's integrator skill page (depth = 1-based layer
 * index). Host function, fp64. Returns NaN for depth < 1.
 */
double diffattn_lambda_init(int depth);

/*
 * Per-head lambda (lesson "Differential Attention V2", section "Concept"):
 * lambda_out[h] = exp(lq1[h] . lk1[h]) - exp(lq2[h] . lk2[h]) + lambda_init(depth).
 * lq1, lk1, lq2, lk2: [H, d_lambda] fp32 device, contiguous; lambda_out [H]
 * fp32 device. 1 <= H, 1 <= d_lambda <= 4096, depth >= 1.
 */
int diffattn_lambda(const float *lq1, const float *lk1, const float *lq2, const float *lk2,
                    int H, int d_lambda, int depth, float *lambda_out, void *stream);

/* Differential-attention prefill over whole sequences (see the struct). */
int diffattn_prefill(const diffattn_prefill_args *a, void *stream);

/*
 * Bytes of device workspace diffattn_decode needs for these arguments: the
 * page prefix over the sequences and the split-KV partial results (one per
 * (work-group, sequence and KV head) pair). Only sizes and flags are examined
 * (pointers may be NULL). Returns 0 if they are invalid or B == 0.
 */
size_t diffattn_decode_workspace_bytes(const diffattn_decode_args *a);

/*
 * Paged decode (see the struct). workspace: caller-owned device memory of at
 * least diffattn_decode_workspace_bytes(a) bytes, 256-byte aligned; its
 * contents need no initialisation and are overwritten. Calls that share one
 * workspace must be ordered on one stream.
 */
int diffattn_decode(const diffattn_decode_args *a, void *workspace, size_t ws_bytes, void *stream);

/*
 * Paged decode without a workspace, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation). Same arguments, kernels and results as diffattn_decode;
 * the split-KV partial results go to a static device scratch of 32 MiB
 * (each device the library runs on holds its own until the process ends)
 * instead of a caller workspace. Allocates nothing and calls no allocating
 * routine. Returns DIFFATTN_EWORKSPACE, launching nothing, when the
 * arguments need more scratch than that (diffattn_decode_workspace_bytes(a)
 * > 32 MiB; the need is a small header plus at most 2048 + B * H_kv records
 * of 2 * (H / H_kv) * (d_v + 2) fp32 each, so with 4 query pairs per KV head
 * up to about 6000 (sequence, KV head) pairs fit). All calls on one device
 * share the scratch, which keeps the last call's contents and needs no
 * clearing: calls that overlap on one device (different streams, or host
 * threads without ordering) race; calls ordered on one stream do not.
 */
int diffattn_decode_noalloc(const diffattn_decode_args *a, void *stream);

/*
 * Backward pass of the prefill (the gradients of the function defined above;
 * the pages give the forward only, the gradients follow from it by the chain
 * rule). Inputs as in diffattn_prefill_args (bf16, d_v 128, d_qk 64 or 128),
 * plus:
 *   o1, o2, lse1, lse2  the statistics a diffattn_prefill call with the same
 *                       inputs stored (fp32, contiguous)
 *   dout, sdo[3]        gradient of the output [B, H, N, d_v], bf16, strides (b, h, n)
 * Outputs (fp32, contiguous, overwritten):
 *   dq1, dq2  [B, H, N, d_qk]
 *   dk1, dk2  [B, H_kv, N, d_qk]; when k1 == k2 (one key tensor for both
 *             branches) dk1 receives the whole key gradient and dk2 must be
 *             NULL or equal to dk1
 *   dv        [B, H_kv, N, d_v]
 *   dlambda   [H]           (feed diffattn_lambda_backward for the four vectors)
 *   dgamma    [H, d_v]      (with a norm; may be NULL otherwise)
 * The workspace (diffattn_backward_workspace_bytes) holds the output gradient
 * after the norm in bf16 and per-row reductions; 256-byte aligned.
 */
typedef struct {
    int dtype;
    int B, H, H_kv, N, d_qk, d_v;
    const void *q1, *q2;
    const void *k1, *k2;
    const void *v;
    int64_t sq1[3], sq2[3], sk1[3], sk2[3], sv[3];
    const float *lambda;
    int depth;
    int causal;
    int window;
    float scale;
    int norm;
    const float *gamma;
    float eps;
    const float *o1, *o2;
    const float *lse1, *lse2;
    const void *dout;
    int64_t sdo[3];
    float *dq1, *dq2;
    float *dk1, *dk2;
    float *dv;
    float *dlambda;
    float *dgamma;
} diffattn_backward_args;

/* Workspace bytes for diffattn_backward (sizes only; 0 if invalid). */
size_t diffattn_backward_workspace_bytes(const diffattn_backward_args *a);

int diffattn_backward(const diffattn_backward_args *a, void *workspace, size_t ws_bytes, void *stream);

/*
 * Gradients of lambda = exp(lq1 . lk1) - exp(lq2 . lk2) + lambda_init with
 * respect to the four [H, d_lambda] fp32 vectors, given dlambda [H]:
 * dlq1 = dlambda e1 lk1, dlk1 = dlambda e1 lq1, dlq2 = -dlambda e2 lk2,
 * dlk2 = -dlambda e2 lq2 with e_k = exp(lq_k . lk_k). Device pointers.
 */
int diffattn_lambda_backward(const float *lq1, const float *lk1, const float *lq2, const float *lk2, int H,
                             int d_lambda, const float *dlambda, float *dlq1, float *dlk1, float *dlq2,
                             float *dlk2, void *stream);

/* Message for the last failure on this thread ("" if none). */
const char *diffattn_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* DIFFATTN_H */
