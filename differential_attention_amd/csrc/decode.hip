// decode.hip -- split-KV paged decode of differential attention
// (lesson "Differential Attention V2", section "V1 vs V2"). V2 form: the
// query heads are doubled, the KV heads stay, so the KV cache is loaded once
// per step and every key/value byte feeds all query heads of its group, both
// branches. V1 form (d_qk 64, separate K1 and K2 caches, value width 128):
// the value cache that a two-call implementation reads once per branch is
// read once here for both, and the combine applies the V1 norm.
//
// Work decomposition. The (sequence, KV head) units, in order, with their
// pages form one global page list of T pages. Pass 1 (decode_split_kernel)
// gives work-group w the contiguous range [w T / W, (w + 1) T / W) of it, so
// every work-group streams the same number of pages whatever the mix of
// sequence lengths (no tail of long items); W is one round of resident
// work-groups unless the caller asks for a page count per work-group. A
// range can start and end inside a unit and can cross several; for each
// unit u it touches, work-group w writes one partial state to record w + u
// of the workspace (unique: a later work-group never touches an earlier
// unit). Pass 2 (decode_combine_kernel), one work-group per (output head,
// sequence), finds the work-groups that covered its unit from the same
// arithmetic and merges their records with the log-sum-exp rule, forms
// y = O1 - lambda O2 and, for the V1 norm, y / sqrt(mean(y^2) + eps) *
// gamma * (1 - lambda_init).
//
// Inside a range, all 2 * group query rows of the KV head (both branches of
// every pair) form one 16-column MFMA operand, so each K and V byte is read
// from HBM exactly once (V1: the K1 product with the branch-2 columns zeroed
// plus the K2 product with the branch-1 columns zeroed fill one accumulator). Each of the 4 waves owns a 16-token slice of every
// page and streams it independently -- no barrier inside the page loop: the
// next kBuf pages' K and V slices are loaded into registers while the current
// one is used, so every wave keeps HBM requests in flight.
//   S^T = K Q^T      16 tokens x 16 query rows, v_mfma_f32_16x16x32_bf16;
//                    each lane loads its K operand (token, 8 features)
//                    straight from HBM in MFMA operand layout
//   online softmax   per query row (lane % 16), running max / sum
//   O^T += V^T P^T   128 x 16, v_mfma_f32_16x16x16_bf16: the 4 scores a lane
//                    holds are its B-operand k-slots; the V slice goes through
//                    a wave-private LDS buffer (XOR-swizzled rows) and
//                    ds_read_b64_tr_b16 returns 4 consecutive tokens of one
//                    value column
// At the end of a unit's part the 4 waves' states are merged through LDS and
// the (max, sum, unnormalised O) of each query row is written to its record.
// Token t of sequence b is slot t % 64 of page page_table[b][t / 64]; tokens
// at or past ctx_len[b] are masked and their value rows replaced by zeros, so
// whatever an unused cache slot holds cannot reach the output. A page id
// outside [0, num_pages) is never dereferenced: page 0 is read in its place,
// all its tokens are masked and bit 0 of *dev_err is set. A sequence whose
// length is out of range has no pages; its outputs are zeros and bit 1 of
// *dev_err is set. With a causal window W the query sees tokens L-W .. L-1
// (lesson "Attention Variants", sliding window, for the last row): only the
// pages holding them enter the page list and earlier tokens are masked.
//
// fp8 caches (OCP e4m3, per-tensor scales): every lane loads 16 codes per
// 16-byte request -- half the bytes of a bf16 slice, so twice the pages are
// held in flight in the same registers -- and widens them to bf16 on the way
// to the matrix cores (exact: every e4m3 value is a bf16 value). The key
// scale is folded into the score scale and the value scale applied in the
// combine, so the loop itself runs on the codes' values. Because a dot
// product does not care in which order its features are summed, a lane loads
// 32 contiguous key features and the Q fragments use the same feature order.
#include "common.hpp"
#include "launch.hpp"

#include <algorithm>
#include <atomic>

namespace da {

namespace {

typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr int kDV = 128;     // value width (and the width of a record row)
constexpr int kPage = 64;    // tokens per page
#ifndef DIFFATTN_DECODE_KBUF
#define DIFFATTN_DECODE_KBUF 2
#endif
constexpr int kBuf = DIFFATTN_DECODE_KBUF;  // pages of K/V held in registers per wave
#ifndef DIFFATTN_DECODE_ROUNDS
#define DIFFATTN_DECODE_ROUNDS 1
#endif
constexpr int kRounds = DIFFATTN_DECODE_ROUNDS;  // rounds of resident work-groups (library's choice)
constexpr float kLazy = 8.0f;  // lazy-rescale threshold of the running max, log2 units

struct DecodeParams {
    const __bf16 *q1, *q2;
    int64_t sq1[2], sq2[2];
    const __bf16 *kc, *kc2, *vc;  // kc2: the branch-2 key cache (d_qk 64; == kc for d_qk 128)
    const int32_t *page_table, *ctx_len;
    const float *lambda, *gamma;
    __bf16 *out;
    int64_t so[2];
    int32_t *pref;  // workspace header: pages of the valid sequences before b, [B + 1]
    float *rec;     // workspace records, qrows * (kDV + 2) floats each
    int *dev_err;
    int B, H, H_kv, group, qrows, max_pages, num_pages, target, num_wgs, norm, window;
    float sc_log2, eps, one_minus_init;
    float v_scale;  // fp8 value scale (1 for bf16 caches)
};

__device__ __forceinline__ uint4 ldg16(const __bf16 *p) { return *(const uint4 *)p; }
// 16 bytes of the key/value caches: a non-temporal load (every cache line is
// read once per call, so none is worth keeping in the caches), which streams
// about 8 % faster than an ordinary load (a plain read of a large buffer:
// 6.45 against 6.0 TB/s)
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ldnt16(const void *p) {
    const u32x4_t v = __builtin_nontemporal_load((const u32x4_t *)p);
    return make_uint4(v.x, v.y, v.z, v.w);
}

// first token the query sees: L - W with a window W < L, else 0
__device__ __forceinline__ int first_token(const DecodeParams &p, int L) {
    return (p.window > 0 && L > p.window) ? L - p.window : 0;
}

// pages of sequence b holding visible tokens (those from the page of its
// first visible token on); 0 for b >= B or a length out of range
__device__ __forceinline__ int seq_pages(const DecodeParams &p, int b) {
    if (b >= p.B) return 0;
    const int L = p.ctx_len[b];
    if (L < 1 || L > p.max_pages * kPage) return 0;
    return (L + kPage - 1) / kPage - first_token(p, L) / kPage;
}

// work-groups that share the T pages (each gets at least one)
__device__ __forceinline__ int64_t active_wgs(const DecodeParams &p, int64_t T) {
    if (T <= 0) return 0;
    const int64_t want = p.target > 0 ? (T + p.target - 1) / p.target : T / kDecodeMinPages;
    return min((int64_t)p.num_wgs, max((int64_t)1, want));
}

// sum over the 256 threads of a work-group
__device__ __forceinline__ int block_sum(int x, int *sh) {
    for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, 64);
    if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = x;
    __syncthreads();
    const int t = sh[0] + sh[1] + sh[2] + sh[3];
    __syncthreads();
    return t;
}

// inclusive prefix sum over the 256 threads of a work-group; *total = the sum
__device__ __forceinline__ int block_scan(int x, int *sh, int *total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    for (int o = 1; o < 64; o <<= 1) {
        const int t = __shfl_up(x, o, 64);
        if (lane >= o) x += t;
    }
    if (lane == 63) sh[wave] = x;
    __syncthreads();
    int before = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) before += i < wave ? sh[i] : 0;
    *total = sh[0] + sh[1] + sh[2] + sh[3];
    __syncthreads();
    return x + before;
}

// one wave's 16-token slice of a page: K operands and V rows
template <bool FP8>
struct Slice {
    uint4 k[4];  // k[kc]: token 16 w + lane % 16, 8 features from 8 (lane / 16) (see the Q fragments)
    uint4 v[4];  // v[i]: token 16 w + 4 i + lane / 16, features 8 (lane % 16) .. +7
    bool ok;     // the page id was valid
};
template <>
struct Slice<true> {
    uint4 k[2];  // token 16 w + lane % 16; d_qk 128: features 32 (lane / 16) .. +31;
                 // d_qk 64: k[0] from K1, k[1] from K2, features 16 (lane / 16) .. +15
    uint4 v[2];  // v[i]: token 16 w + 8 i + lane / 8, features 16 (lane % 8) .. +15
    bool ok;
};

// 4 e4m3 codes (in memory order) -> 4 bf16 values in the same order: one
// scaled conversion (scale 1) per two codes, exact since every e4m3 value is
// a bf16 value
__device__ __forceinline__ uint2 e4m3x4_to_bf16(uint32_t w) {
    const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w, 1.0f, false);  // bytes 0, 1
    const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w, 1.0f, true);   // bytes 2, 3
    return uint2{__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b)};
}

// 8 codes (two words) -> one bf16x8 MFMA operand
__device__ __forceinline__ bf16x8 e4m3x8_to_bf16(uint32_t w0, uint32_t w1) {
    const uint2 a = e4m3x4_to_bf16(w0), b = e4m3x4_to_bf16(w1);
    return as_bf16x8(uint4{a.x, a.y, b.x, b.y});
}

template <int DQK, bool FP8>
__global__ __launch_bounds__(256) void decode_split_kernel(DecodeParams p) {
    constexpr int kBufT = FP8 ? 2 * kBuf : kBuf;  // slices in flight per wave
    __shared__ __attribute__((aligned(1024))) unsigned char lds[4 * 16 * kDV * 4];  // 32 KB
    __shared__ float red_m[4][16], red_l[4][16];
    __shared__ int sh[4], s_b, s_excl;

    const int w = blockIdx.x;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int n = lane & 15, grp = lane >> 4;

    // the global page list: T pages, W work-groups share it
    int part = 0;
    for (int b0 = 0; b0 < p.B; b0 += 256) part += seq_pages(p, b0 + tid);
    const int tseq = block_sum(part, sh);
    const int64_t T = (int64_t)tseq * p.H_kv;
    const int64_t W = active_wgs(p, T);
    if (w >= W && w != 0) return;
    const int64_t start = W > 0 ? (int64_t)w * T / W : 0;
    const int64_t end = W > 0 ? (int64_t)(w + 1) * T / W : 0;

    // find the unit holding page `start` (a prefix sum over the sequences);
    // work-group 0 also stores the prefix for the combine pass
    int carry = 0;
    for (int b0 = 0; b0 < p.B; b0 += 256) {
        const int bb = b0 + tid;
        const int c = seq_pages(p, bb);
        int tot;
        const int excl = carry + block_scan(c, sh, &tot) - c;
        if (w == 0 && bb < p.B) p.pref[bb] = excl;
        if (c > 0 && (int64_t)excl * p.H_kv <= start && start < (int64_t)(excl + c) * p.H_kv) {
            s_b = bb;
            s_excl = excl;
        }
        carry += tot;
    }
    if (w == 0 && tid == 0) p.pref[p.B] = carry;
    if (w >= W) return;
    __syncthreads();

    int b = __builtin_amdgcn_readfirstlane(s_b);
    int c = seq_pages(p, b);
    int64_t ubase = (int64_t)__builtin_amdgcn_readfirstlane(s_excl) * p.H_kv;  // first page of unit (b, g)
    int g = (int)((start - ubase) / c);
    ubase += (int64_t)g * c;

    // this wave's V buffer: 16 rows x 256 bytes, 16-byte chunks XOR-swizzled
    // by 2 (row & 7) so each transposing read pass touches 64 distinct banks
    unsigned char *vbuf = lds + wave * 4096;
    const int vrow = 4 * grp + (n >> 2);  // row this lane addresses in a transposing read
    const int vswz = (vrow & 7) << 1;

    for (int64_t pos = start;;) {
        // pages [p0, p1) of unit (b, g), counted from the page of its first
        // visible token (page index fp in the sequence)
        const int p0 = (int)(pos - ubase);
        const int p1 = (int)(min(end, ubase + c) - ubase);
        const int L = p.ctx_len[b];
        const int t0 = first_token(p, L);
        const int fp = t0 / kPage;

        // Q^T fragments: lane supplies query row n (pair n / 2, branch n % 2).
        // d_qk 128: k step kc covers features 32 kc + 8 grp .. +7 of the shared
        // keys (fp8: 32 grp + 8 kc .. +7). d_qk 64: k steps 0, 1 contract K1
        // with the branch-1 rows and steps 2, 3 contract K2 with the branch-2
        // rows (each with the other branch's rows zero), so one accumulator
        // gets each row's own scores; features 32 (kc % 2) + 8 grp .. +7
        // (fp8: 16 grp + 8 (kc % 2) .. +7).
        bf16x8 qf[4];
        {
            const bool ok = n < p.qrows;
            const int pair = n >> 1, br = n & 1;
            const int h = g * p.group + (ok ? pair : 0);
            const __bf16 *q = br ? p.q2 + b * p.sq2[0] + h * p.sq2[1] : p.q1 + b * p.sq1[0] + h * p.sq1[1];
#pragma unroll
            for (int kc = 0; kc < 4; ++kc) {
                uint4 z = {0u, 0u, 0u, 0u};
                const bool use = DQK == 128 ? ok : (ok && br == (kc >> 1));
                int f;
                if (FP8)
                    f = DQK == 128 ? 32 * grp + 8 * kc : 16 * grp + 8 * (kc & 1);
                else
                    f = 32 * (DQK == 128 ? kc : (kc & 1)) + 8 * grp;
                qf[kc] = as_bf16x8(use ? ldg16(q + f) : z);
            }
        }

        f32x4 o[8];
#pragma unroll
        for (int dc = 0; dc < 8; ++dc) o[dc] = f32x4{};
        float m = -INFINITY, l = 0.0f;
        bool bad_page = false;

        // pages in chunks of at most 64: a chunk's page ids are read once, one
        // per lane, and each page's id is then taken with v_readlane (a scalar),
        // so no vector load of the table sits between the K/V loads of pages
        const int32_t *table = p.page_table + (int64_t)b * p.max_pages + fp;
        for (int c0 = p0; c0 < p1; c0 += 64) {
            const int np = min(64, p1 - c0);
            const int ids = lane < np ? table[c0 + lane] : 0;
            auto load = [&](Slice<FP8> &S, int k) DA_INLINE {
                int phys = __builtin_amdgcn_readlane(ids, k);
                S.ok = phys >= 0 && phys < p.num_pages;
                bad_page |= !S.ok;
                phys = S.ok ? phys : 0;
                const int64_t row0 = ((int64_t)phys * p.H_kv + g) * kPage + 16 * wave;  // first token row
                if constexpr (FP8) {
                    const unsigned char *vp = (const unsigned char *)p.vc + (row0 + (lane >> 3)) * kDV + 16 * (lane & 7);
                    if (DQK == 128) {
                        const unsigned char *kp = (const unsigned char *)p.kc + (row0 + n) * DQK + 32 * grp;
                        S.k[0] = ldnt16(kp);
                        S.k[1] = ldnt16(kp + 16);
                    } else {
                        const int64_t off = (row0 + n) * DQK + 16 * grp;
                        S.k[0] = ldnt16((const unsigned char *)p.kc + off);
                        S.k[1] = ldnt16((const unsigned char *)p.kc2 + off);
                    }
                    S.v[0] = ldnt16(vp);
                    S.v[1] = ldnt16(vp + 8 * kDV);
                } else {
                    const __bf16 *vp = p.vc + row0 * kDV + grp * kDV + 8 * n;
                    if (DQK == 128) {
                        const __bf16 *kp = p.kc + (row0 + n) * DQK + 8 * grp;
#pragma unroll
                        for (int kc = 0; kc < 4; ++kc) S.k[kc] = ldnt16(kp + 32 * kc);
                    } else {
                        const __bf16 *kp1 = p.kc + (row0 + n) * DQK + 8 * grp;
                        const __bf16 *kp2 = p.kc2 + (row0 + n) * DQK + 8 * grp;
                        S.k[0] = ldnt16(kp1);
                        S.k[1] = ldnt16(kp1 + 32);
                        S.k[2] = ldnt16(kp2);
                        S.k[3] = ldnt16(kp2 + 32);
                    }
#pragma unroll
                    for (int i = 0; i < 4; ++i) S.v[i] = ldnt16(vp + 4 * i * kDV);
                }
            };

            auto process = [&](const Slice<FP8> &S, int k) DA_INLINE {
                const int pg = fp + c0 + k;                   // page index in the sequence
                const int vis = L - pg * kPage - 16 * wave;   // rows >= vis are past the end
                const int vlo = t0 - pg * kPage - 16 * wave;  // rows < vlo are before the window
                // V rows into the wave buffer (rows past the end as zeros)
                if constexpr (FP8) {
#pragma unroll
                    for (int i = 0; i < 2; ++i) {
                        const int row = 8 * i + (lane >> 3);
                        // a bad page id was replaced by page 0: none of its values may enter
                        const uint32_t keep = (S.ok && row < vis && row >= vlo) ? 0xffffffffu : 0u;
                        const uint2 a = e4m3x4_to_bf16(S.v[i].x), b2 = e4m3x4_to_bf16(S.v[i].y);
                        const uint2 c2 = e4m3x4_to_bf16(S.v[i].z), d2 = e4m3x4_to_bf16(S.v[i].w);
                        // features 16 (lane % 8) .. +15 are 16-byte chunks 2 (lane % 8) and
                        // 2 (lane % 8) + 1 of the row; the swizzle is even, so they stay adjacent
                        unsigned char *dst = vbuf + row * 256 + 16 * ((2 * (lane & 7)) ^ ((row & 7) << 1));
                        *(uint4 *)dst = uint4{a.x & keep, a.y & keep, b2.x & keep, b2.y & keep};
                        *(uint4 *)(dst + 16) = uint4{c2.x & keep, c2.y & keep, d2.x & keep, d2.y & keep};
                    }
                } else {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int row = 4 * i + grp;
                        const uint32_t keep = (S.ok && row < vis && row >= vlo) ? 0xffffffffu : 0u;  // select by value
                        uint4 v = S.v[i];
                        v.x &= keep;
                        v.y &= keep;
                        v.z &= keep;
                        v.w &= keep;
                        *(uint4 *)(vbuf + row * 256 + 16 * (n ^ ((row & 7) << 1))) = v;
                    }
                }
                // scores of the 16 tokens against the 16 query rows
                f32x4 sc = f32x4{};
#pragma unroll
                for (int kc = 0; kc < 4; ++kc) {
                    bf16x8 ka;
                    if constexpr (FP8) {
                        const uint4 &w = S.k[kc >> 1];
                        ka = (kc & 1) ? e4m3x8_to_bf16(w.z, w.w) : e4m3x8_to_bf16(w.x, w.y);
                    } else {
                        ka = as_bf16x8(S.k[kc]);
                    }
                    sc = mfma16(ka, qf[kc], sc);
                }
                if (!(S.ok && vis >= 16 && vlo <= 0)) {  // a slice with masked tokens (wave-uniform)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        if (!S.ok || 4 * grp + r >= vis || 4 * grp + r < vlo) sc[r] = -INFINITY;
                }
                float mx = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
                mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
                mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
                // lazy rescale: the reference m moves only when a score exceeds it
                // by more than kLazy (log2 units), so the weights stay <= 2^kLazy
                // and O and l are rescaled rarely; the normalisation at the end
                // divides by l built on the same reference, so the result is the
                // same softmax
                const float mxs = mx * p.sc_log2;
                const bool grow = mxs > m + kLazy;  // false while every score is masked
                if (__any(grow)) {                  // wave-uniform
                    const float mnew = grow ? mxs : m;
                    const float alpha = (m == mnew) ? 1.0f : exp2_fast(m - mnew);
                    m = mnew;
                    l *= alpha;
#pragma unroll
                    for (int dc = 0; dc < 8; ++dc) o[dc] *= alpha;
                }
                const float msub = (m == -INFINITY) ? 0.0f : m;
                float pr[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) pr[r] = exp2_fast(fmaf(sc[r], p.sc_log2, -msub));
                l += (pr[0] + pr[1]) + (pr[2] + pr[3]);
                const bf16x2 p01 = pack2(pr[0], pr[1]), p23 = pack2(pr[2], pr[3]);
                const bf16x4_t pb4 = {p01[0], p01[1], p23[0], p23[1]};
                // the V rows written above must be complete before other lanes read them
                __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
                const unsigned char *vr = vbuf + vrow * 256;
#pragma unroll
                for (int dc = 0; dc < 8; ++dc) {
                    const int col = 16 * dc + 4 * (n & 3);
                    const int cc = (col >> 3) ^ vswz;
                    const s16x4 va =
                        __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(vr + 16 * cc + 2 * (col & 7)));
                    o[dc] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(bf16x4_t, va), pb4,
                                                                      o[dc], 0, 0, 0);
                }
                // the reads must be complete before the next slice overwrites the buffer
                __builtin_amdgcn_s_waitcnt(0xC07F);
            };

            // every slot issues its next load unconditionally (past the chunk's
            // end it re-reads the chunk's last page, which is in L2), so the
            // compiler can count the loads in flight and wait for the oldest
            // slice only, keeping kBufT - 1 slices of requests outstanding
            Slice<FP8> S[kBufT];
#pragma unroll
            for (int j = 0; j < kBufT; ++j) load(S[j], min(j, np - 1));
            for (int k0 = 0; k0 < np; k0 += kBufT) {
#pragma unroll
                for (int j = 0; j < kBufT; ++j) {
                    const int k = k0 + j;
                    if (k < np) process(S[j], k);
                    load(S[j], min(k + kBufT, np - 1));
                }
            }
        }
        if (bad_page && lane == 0 && p.dev_err) atomicOr(p.dev_err, 1);

        // row sums over the 4 lane groups that share a query row
        l += __shfl_xor(l, 16, 64);
        l += __shfl_xor(l, 32, 64);

        // merge the 4 waves through LDS into record w + (b H_kv + g)
        __syncthreads();
        float *ow = (float *)lds;  // [4 waves][16 rows][128 dv]
#pragma unroll
        for (int dc = 0; dc < 8; ++dc)
#pragma unroll
            for (int r = 0; r < 4; ++r) ow[(wave * 16 + n) * kDV + 16 * dc + 4 * grp + r] = o[dc][r];
        if (grp == 0) {
            red_m[wave][n] = m;
            red_l[wave][n] = l;
        }
        __syncthreads();
        float *rec = p.rec + ((int64_t)w + (int64_t)b * p.H_kv + g) * p.qrows * (kDV + 2);
        for (int idx = tid; idx < p.qrows * kDV; idx += 256) {
            const int q = idx / kDV, dv = idx % kDV;
            float M = fmaxf(fmaxf(red_m[0][q], red_m[1][q]), fmaxf(red_m[2][q], red_m[3][q]));
            float acc = 0.0f, lsum = 0.0f;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float mw = red_m[i][q];
                const float f = (mw == -INFINITY) ? 0.0f : exp2_fast(mw - M);
                acc += ow[(i * 16 + q) * kDV + dv] * f;
                lsum += red_l[i][q] * f;
            }
            float *rq = rec + q * (kDV + 2);
            rq[dv] = acc;
            if (dv == 0) {
                rq[kDV] = M;
                rq[kDV + 1] = lsum;
            }
        }

        // next unit with pages, if the range goes on
        pos = ubase + p1;
        if (pos >= end) break;
        ubase += c;
        if (++g == p.H_kv) {
            g = 0;
            do {
                ++b;
                c = seq_pages(p, b);
            } while (c == 0 && b + 1 < p.B);
            if (c == 0) break;  // unreachable: pos < end <= T leaves pages to take
        }
        __syncthreads();  // the merge buffers are reused
    }
}

__global__ __launch_bounds__(128) void decode_combine_kernel(DecodeParams p) {
    __shared__ float red[4];
    const int h = blockIdx.x, b = blockIdx.y, dv = threadIdx.x;
    const int g = h / p.group, j = h - g * p.group;
    const int L = p.ctx_len[b];
    __bf16 *op = p.out + b * p.so[0] + h * p.so[1];
    if (L < 1 || L > p.max_pages * kPage) {
        if (h == 0 && dv == 0 && p.dev_err) atomicOr(p.dev_err, 2);
        op[dv] = (__bf16)0.0f;
        return;
    }
    // the work-groups whose ranges covered unit (b, g): those holding its first
    // and last page and every one between (work-group w holds page x iff
    // w T / W <= x < (w + 1) T / W, so w = floor(((x + 1) W - 1) / T))
    const int excl = p.pref[b], c = p.pref[b + 1] - excl;
    const int64_t T = (int64_t)p.pref[p.B] * p.H_kv, W = active_wgs(p, T);
    const int64_t ubase = (int64_t)excl * p.H_kv + (int64_t)g * c;
    const int64_t w0 = ((ubase + 1) * W - 1) / T, w1 = ((ubase + c) * W - 1) / T;
    const int ns = (int)(w1 - w0 + 1);
    const float *base = p.rec + (w0 + (int64_t)b * p.H_kv + g) * p.qrows * (kDV + 2);
    float ob[2];
#pragma unroll
    for (int br = 0; br < 2; ++br) {
        const int q = 2 * j + br;
        // the records' loads are independent: unrolled so they are in flight together
        float M = -INFINITY;
#pragma unroll 8
        for (int s = 0; s < ns; ++s) M = fmaxf(M, base[((int64_t)s * p.qrows + q) * (kDV + 2) + kDV]);
        float acc = 0.0f, lsum = 0.0f;
#pragma unroll 8
        for (int s = 0; s < ns; ++s) {
            const float *rq = base + ((int64_t)s * p.qrows + q) * (kDV + 2);
            const float ms = rq[kDV];
            const float f = (ms == -INFINITY) ? 0.0f : exp2_fast(ms - M);
            acc += rq[dv] * f;
            lsum += rq[kDV + 1] * f;
        }
        ob[br] = lsum > 0.0f ? acc / lsum * p.v_scale : 0.0f;
    }
    float y;
    {
#pragma clang fp contract(off)
        y = ob[0] - p.lambda[h] * ob[1];
    }
    if (p.norm) {
        if (p.norm == 2) {  // GroupNorm per head: subtract the channel mean first
            const float sm = wave_sum(y);
            if ((dv & 63) == 0) red[2 + (dv >> 6)] = sm;
            __syncthreads();
            y -= (red[2] + red[3]) * (1.0f / kDV);
        }
        float ss = wave_sum(y * y);
        if ((dv & 63) == 0) red[dv >> 6] = ss;
        __syncthreads();
        ss = red[0] + red[1];
        y *= p.one_minus_init / sqrtf(ss * (1.0f / kDV) + p.eps) * p.gamma[(int64_t)h * kDV + dv];
    }
    op[dv] = (__bf16)y;
}

// Work-groups of the split pass that fit on the device at once; cached per
// device (compute-unit count times the kernel's occupancy per unit).
template <int DQK, bool FP8>
int resident_split_wgs() {
    constexpr int kMaxDevices = 64;
    static std::atomic<int> cache[kMaxDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 1;
    if (dev >= 0 && dev < kMaxDevices) {
        const int c = cache[dev].load(std::memory_order_relaxed);
        if (c > 0) return c;
    }
    int cus = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, decode_split_kernel<DQK, FP8>, 256, 0) != hipSuccess)
        return 1;
    const int r = std::max(1, cus * per_cu);
    if (dev >= 0 && dev < kMaxDevices) cache[dev].store(r, std::memory_order_relaxed);
    return r;
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
    p.kc2 = (const __bf16 *)a.k2_cache;
    p.vc = (const __bf16 *)a.v_cache;
    p.page_table = a.page_table;
    p.ctx_len = a.ctx_len;
    p.lambda = a.lambda;
    p.gamma = a.gamma;
    p.out = (__bf16 *)a.out;
    p.pref = (int32_t *)workspace;
    p.rec = (float *)((unsigned char *)workspace + plan.header_bytes);
    p.dev_err = a.dev_err;
    p.B = a.B;
    p.H = a.H;
    p.H_kv = a.H_kv;
    p.group = a.H / a.H_kv;
    p.qrows = plan.qrows;
    p.max_pages = a.max_pages;
    p.num_pages = a.num_pages;
    p.target = plan.target_pages;
    const bool d64 = a.d_qk == 64, fp8 = a.kv_dtype == DIFFATTN_FP8_E4M3;
    int resident;
    if (fp8)
        resident = d64 ? resident_split_wgs<64, true>() : resident_split_wgs<128, true>();
    else
        resident = d64 ? resident_split_wgs<64, false>() : resident_split_wgs<128, false>();
    p.num_wgs = plan.target_pages > 0 ? plan.max_wgs : std::min(plan.max_wgs, kRounds * resident);
    p.norm = a.norm;  // 0 none, 1 RMS, 2 GroupNorm
    p.window = a.window;
    p.sc_log2 = scale * (fp8 ? a.k_scale : 1.0f) * kLog2e;
    p.v_scale = fp8 ? a.v_scale : 1.0f;
    p.eps = a.eps;
    p.one_minus_init = 1.0f - lambda_init;
    auto kern = fp8 ? (d64 ? decode_split_kernel<64, true> : decode_split_kernel<128, true>)
                    : (d64 ? decode_split_kernel<64, false> : decode_split_kernel<128, false>);
    hipLaunchKernelGGL(kern, dim3(p.num_wgs), dim3(256), 0, stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(decode_combine_kernel, dim3(a.H, a.B), dim3(128), 0, stream, p);
    return hipGetLastError();
}

// ---- static scratch for the allocation-free entry point
// A file-scope device array: each device that loads the library holds its
// own copy until the process ends. Host code never uses the array's name as
// an address (on the host it is only a handle); it uses the device address
// hipGetSymbolAddress returns for the current device, looked up on the first
// call on that device and kept per device. Every call on one device shares
// this array: its contents need no initialisation (the split pass writes
// every record the combine pass reads), and calls that overlap on one device
// race.
static __device__ __align__(256) unsigned char scratch[kDecodeScratchBytes];

hipError_t decode_scratch(void **ptr) {
    constexpr int kMaxDevices = 64;
    static std::atomic<void *> addr[kMaxDevices];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    void *p = addr[dev].load(std::memory_order_acquire);
    if (!p) {
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        addr[dev].store(p, std::memory_order_release);  // racing first calls store the same address
    }
    *ptr = p;
    return hipSuccess;
}

}  // namespace da
