// prefill_bf16.hip -- fused single-pass differential-attention prefill,
// bf16 inputs, fp32 accumulation, bf16 MFMA on gfx950.
//
// What it computes (lesson "Differential Attention V2", section "Concept";
// V1/V2 forms from its section "V1 vs V2"; causal mask from the lesson
// "Attention Variants", "Build it", step 1): for output head h with KV head
// g = h / (H / H_kv),
//   O_br = softmax(Q_br K_br^T * scale) V,   br = 1, 2
//   y    = O_1 - lambda[h] O_2
//   V1:  y <- y / sqrt(mean(y^2) + eps) * gamma[h] * (1 - lambda_init)
// The two maps are never materialised: by linearity (A1 - l A2) V equals
// A1 V - l A2 V, so each branch keeps its own online-softmax state (running
// max m, running sum l, unnormalised O) and the difference is taken once, in
// fp32, in the epilogue.
//
// Work decomposition (one work-group = 4 waves = 128 query rows of one head):
//  * each wave owns 32 query rows; its Q1/Q2 rows live in registers as MFMA
//    B operands for the whole sweep;
//  * key tiles of 64 keys stream HBM -> registers -> LDS, double-buffered: the
//    next tile's global loads are in flight while the current one is used;
//    one key tile feeds both branches when K1 == K2 (V2), and the value tile
//    is loaded once for both branches;
//  * per 32-key sub-block and branch: S^T = K Q^T (32 keys x 32 queries,
//    v_mfma_f32_32x32x16_bf16), so each lane holds 16 scores of ONE query:
//    the row max needs one cross-half exchange and the row sum stays
//    lane-local until the end;
//  * the probabilities go straight from the S^T accumulator registers into
//    the B operand of O^T += V^T P^T. The key order inside the sub-block is
//    permuted when K rows are read so that each lane's 8 probabilities of a
//    16-key step are 8 consecutive keys, which lets V^T be read from LDS with
//    one 16-byte load;
//  * V is transposed on its way into LDS (V^T[d_v][keys]) so both operands
//    of the PV contraction have keys as their contiguous dimension;
//  * causal: key tiles past the work-group's last row are never loaded,
//    sub-blocks past a wave's last row are skipped, masking runs only on
//    sub-blocks that straddle the diagonal or the end of the sequence; work-
//    groups with the longest rows are dispatched first.
// Grid mapping: work-groups are dispatched round-robin over the 8 XCDs; when
// the number of (batch, KV head) units is a multiple of 8, all work-groups
// reading one KV head are placed on the same XCD so its K/V stay in that
// XCD's L2.
#include "common.hpp"
#include "launch.hpp"

namespace da {

namespace {

constexpr int kDV = 128;    // value width (both forms)
constexpr int kBM = 128;    // query rows per work-group
constexpr int kWM = 32;     // query rows per wave
constexpr int kBN = 64;     // keys per LDS tile
constexpr int kVtLd = kBN + 8;  // row stride (elements) of the V^T tile

struct Bf16Params {
    const __bf16 *q1, *q2, *k1, *k2, *v;
    int64_t sq1[3], sq2[3], sk1[3], sk2[3], sv[3], so[3];
    const float *lambda, *gamma;
    __bf16 *out;
    int B, H, H_kv, group, N, causal, row_blocks, xcd_units;
    float sc_log2;  // scale * log2(e)
    float eps, one_minus_init;
};

// Physical key (within a 32-key sub-block) read by the A-operand row m:
// swap bits 2 and 3 of m.
__device__ __forceinline__ int perm_key(int m) { return (m & 0x13) | ((m & 4) << 1) | ((m & 8) >> 1); }

// Physical key (within a sub-block) held by register r of S^T in lane-half hh.
__device__ __forceinline__ int key_of_reg(int r, int hh) {
    return 16 * ((r >> 3) & 1) + 8 * hh + 4 * ((r >> 2) & 1) + (r & 3);
}

__device__ __forceinline__ uint4 ldg16(const __bf16 *p) { return *(const uint4 *)p; }

template <int DQK, bool SHARED_K>
struct Tile {
    static constexpr int kKLd = DQK + 8;                     // row stride of a K tile
    static constexpr int kNK = SHARED_K ? 1 : 2;             // K tiles per stage
    static constexpr int kKElems = kBN * kKLd;               // one K tile
    static constexpr int kVtElems = kDV * kVtLd;             // the V^T tile
    static constexpr int kStage = kNK * kKElems + kVtElems;  // elements per stage
    static constexpr int kKChunks = kBN * DQK / 8 / 256;     // 16-byte chunks per thread per K tile
};

template <int DQK, bool SHARED_K, bool NORM>
__global__ __launch_bounds__(256) void prefill_bf16_kernel(Bf16Params p) {
    using T = Tile<DQK, SHARED_K>;
    constexpr int KC = DQK / 16;  // 16-wide k steps of the QK contraction
    __shared__ __attribute__((aligned(16))) __bf16 lds[2 * T::kStage];

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int l32 = lane & 31;
    const int hh = lane >> 5;

    // ---- which (batch, head, row block) this work-group computes
    int b, h, rb;
    {
        const int L = blockIdx.x;
        const int U = p.B * p.H;
        int rank, u;
        if (p.xcd_units) {
            // per XCD: xcd_units KV units (stride 8), each with `group` heads
            const int xcd = L & 7, s = L >> 3;
            const int per = p.xcd_units * p.group;
            rank = s / per;
            const int rest = s - rank * per;
            const int kvu = (rest / p.group) * 8 + xcd;
            const int hig = rest - (rest / p.group) * p.group;
            const int bb = kvu / p.H_kv, g = kvu - bb * p.H_kv;
            u = bb * p.H + g * p.group + hig;
        } else {
            rank = L / U;
            u = L - rank * U;
        }
        b = u / p.H;
        h = u - b * p.H;
        rb = p.causal ? p.row_blocks - 1 - rank : rank;
    }
    const int g = h / p.group;
    const int q0 = rb * kBM;
    const int wrow0 = q0 + wave * kWM;  // first query row of this wave
    const int myrow = wrow0 + l32;      // the query row of this lane

    // ---- Q fragments (B operands): lane holds Q[myrow][16 kc + 8 hh .. +7]
    bf16x8 qf1[KC], qf2[KC];
    {
        const __bf16 *q1 = p.q1 + b * p.sq1[0] + h * p.sq1[1] + (int64_t)myrow * p.sq1[2] + 8 * hh;
        const __bf16 *q2 = p.q2 + b * p.sq2[0] + h * p.sq2[1] + (int64_t)myrow * p.sq2[2] + 8 * hh;
        const bool ok = myrow < p.N;
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) {
            uint4 z = {0u, 0u, 0u, 0u};
            qf1[kc] = as_bf16x8(ok ? ldg16(q1 + 16 * kc) : z);
            qf2[kc] = as_bf16x8(ok ? ldg16(q2 + 16 * kc) : z);
        }
    }

    const __bf16 *kb1 = p.k1 + b * p.sk1[0] + g * p.sk1[1];
    const __bf16 *kb2 = p.k2 + b * p.sk2[0] + g * p.sk2[1];
    const __bf16 *vb = p.v + b * p.sv[0] + g * p.sv[1];
    const int64_t sk1n = p.sk1[2], sk2n = p.sk2[2], svn = p.sv[2];

    const int kend = p.causal ? min(p.N, q0 + kBM) : p.N;
    const int ntiles = (kend + kBN - 1) / kBN;

    // ---- staging registers for one tile
    uint4 kr1[T::kKChunks], kr2[SHARED_K ? 1 : T::kKChunks], vr[4];

    auto load_tile = [&](int t) {
        const int key0 = t * kBN;
#pragma unroll
        for (int i = 0; i < T::kKChunks; ++i) {
            const int c = tid + 256 * i;
            const int key = c / (DQK / 8), col = (c % (DQK / 8)) * 8;
            const bool ok = key0 + key < p.N;
            uint4 z = {0u, 0u, 0u, 0u};
            kr1[i] = ok ? ldg16(kb1 + (int64_t)(key0 + key) * sk1n + col) : z;
            if constexpr (!SHARED_K) kr2[i] = ok ? ldg16(kb2 + (int64_t)(key0 + key) * sk2n + col) : z;
        }
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int task = tid + 256 * i;
            const int j = task & 31, cg = task >> 5;
            const int key = key0 + 2 * j;
            uint4 z = {0u, 0u, 0u, 0u};
            vr[2 * i] = key < p.N ? ldg16(vb + (int64_t)key * svn + 8 * cg) : z;
            vr[2 * i + 1] = key + 1 < p.N ? ldg16(vb + (int64_t)(key + 1) * svn + 8 * cg) : z;
        }
    };

    auto store_tile = [&](int stage) {
        __bf16 *base = lds + stage * T::kStage;
#pragma unroll
        for (int i = 0; i < T::kKChunks; ++i) {
            const int c = tid + 256 * i;
            const int key = c / (DQK / 8), col = (c % (DQK / 8)) * 8;
            *(uint4 *)(base + key * T::kKLd + col) = kr1[i];
            if constexpr (!SHARED_K) *(uint4 *)(base + T::kKElems + key * T::kKLd + col) = kr2[i];
        }
        uint32_t *vt = (uint32_t *)(base + T::kNK * T::kKElems);
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

    // ---- per-branch online-softmax state
    f32x16 o1[4], o2[4];
#pragma unroll
    for (int dc = 0; dc < 4; ++dc) {
        o1[dc] = f32x16{};
        o2[dc] = f32x16{};
    }
    float m1 = -INFINITY, m2 = -INFINITY, l1 = 0.0f, l2 = 0.0f;
    const int krow = perm_key(l32);  // key row this lane feeds to the S^T A operand

    auto branch = [&](const __bf16 *ktile, const bf16x8 *qf, const __bf16 *vt, int sb, int key0,
                      bool need_mask, float &m, float &l, f32x16 *o) {
        f32x16 s = f32x16{};
        const __bf16 *krp = ktile + (32 * sb + krow) * T::kKLd + 8 * hh;
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) s = mfma32(as_bf16x8(*(const uint4 *)(krp + 16 * kc)), qf[kc], s);
        if (need_mask) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = key0 + key_of_reg(r, hh);
                if ((p.causal && key > myrow) || key >= p.N) s[r] = -INFINITY;
            }
        }
        float mx = s[0];
#pragma unroll
        for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[r]);
        mx = fmaxf(mx, xor32(mx));
        const float mnew = fmaxf(m, mx * p.sc_log2);
        const float alpha = (m == mnew) ? 1.0f : exp2_fast(m - mnew);
        const float msub = (mnew == -INFINITY) ? 0.0f : mnew;
        m = mnew;
        float ps[16];
        float lsum = 0.0f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            ps[r] = exp2_fast(fmaf(s[r], p.sc_log2, -msub));
            lsum += ps[r];
        }
        l = l * alpha + lsum;
        if (alpha != 1.0f) {
#pragma unroll
            for (int dc = 0; dc < 4; ++dc) o[dc] *= alpha;
        }
        const bf16x8 pb0 = pack8(ps[0], ps[1], ps[2], ps[3], ps[4], ps[5], ps[6], ps[7]);
        const bf16x8 pb1 = pack8(ps[8], ps[9], ps[10], ps[11], ps[12], ps[13], ps[14], ps[15]);
        const __bf16 *vrp = vt + l32 * kVtLd + 32 * sb + 8 * hh;
#pragma unroll
        for (int dc = 0; dc < 4; ++dc) {
            o[dc] = mfma32(as_bf16x8(*(const uint4 *)(vrp + dc * 32 * kVtLd)), pb0, o[dc]);
            o[dc] = mfma32(as_bf16x8(*(const uint4 *)(vrp + dc * 32 * kVtLd + 16)), pb1, o[dc]);
        }
    };

    // ---- the key sweep
    if (ntiles > 0) {
        load_tile(0);
        store_tile(0);
    }
    __syncthreads();
    for (int t = 0; t < ntiles; ++t) {
        const int cur = t & 1;
        if (t + 1 < ntiles) load_tile(t + 1);
        const __bf16 *base = lds + cur * T::kStage;
        const __bf16 *kt1 = base;
        const __bf16 *kt2 = SHARED_K ? base : base + T::kKElems;
        const __bf16 *vt = base + T::kNK * T::kKElems;
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
            const int key0 = t * kBN + 32 * sb;
            const bool live = key0 < p.N && !(p.causal && key0 > wrow0 + kWM - 1);
            if (live) {
                const bool need_mask = (p.causal && key0 + 31 > wrow0) || key0 + 32 > p.N;
                branch(kt1, qf1, vt, sb, key0, need_mask, m1, l1, o1);
                branch(kt2, qf2, vt, sb, key0, need_mask, m2, l2, o2);
            }
        }
        if (t + 1 < ntiles) store_tile(cur ^ 1);
        __syncthreads();
    }

    // ---- epilogue: y = O1 / l1 - lambda O2 / l2 (then the V1 norm), bf16 store
    l1 += xor32(l1);
    l2 += xor32(l2);
    const float r1 = 1.0f / l1;
    const float r2 = p.lambda[h] / l2;
    f32x16 y[4];
#pragma unroll
    for (int dc = 0; dc < 4; ++dc) y[dc] = o1[dc] * r1 - o2[dc] * r2;
    if constexpr (NORM) {
        float ss = 0.0f;
#pragma unroll
        for (int dc = 0; dc < 4; ++dc)
#pragma unroll
            for (int r = 0; r < 16; ++r) ss = fmaf(y[dc][r], y[dc][r], ss);
        ss += xor32(ss);
        const float rs = p.one_minus_init / sqrtf(ss * (1.0f / kDV) + p.eps);
        const float *gm = p.gamma + (int64_t)h * kDV;
#pragma unroll
        for (int dc = 0; dc < 4; ++dc)
#pragma unroll
            for (int r = 0; r < 16; ++r) y[dc][r] *= rs * gm[32 * dc + 8 * (r >> 2) + 4 * hh + (r & 3)];
    }
    if (myrow < p.N) {
        __bf16 *op = p.out + b * p.so[0] + h * p.so[1] + (int64_t)myrow * p.so[2] + 4 * hh;
#pragma unroll
        for (int dc = 0; dc < 4; ++dc)
#pragma unroll
            for (int rq = 0; rq < 4; ++rq) {
                const bf16x2 a = pack2(y[dc][4 * rq], y[dc][4 * rq + 1]);
                const bf16x2 c = pack2(y[dc][4 * rq + 2], y[dc][4 * rq + 3]);
                const bf16x4 w = {a[0], a[1], c[0], c[1]};
                *(bf16x4 *)(op + 32 * dc + 8 * rq) = w;
            }
    }
}

template <int DQK, bool SHARED_K, bool NORM>
hipError_t launch_t(const Bf16Params &p, int blocks, hipStream_t stream) {
    hipLaunchKernelGGL((prefill_bf16_kernel<DQK, SHARED_K, NORM>), dim3(blocks), dim3(256), 0, stream, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_bf16(const diffattn_prefill_args &a, float scale, float lambda_init,
                               hipStream_t stream) {
    Bf16Params p;
    p.q1 = (const __bf16 *)a.q1;
    p.q2 = (const __bf16 *)a.q2;
    p.k1 = (const __bf16 *)a.k1;
    p.k2 = (const __bf16 *)a.k2;
    p.v = (const __bf16 *)a.v;
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
    p.out = (__bf16 *)a.out;
    p.B = a.B;
    p.H = a.H;
    p.H_kv = a.H_kv;
    p.group = a.H / a.H_kv;
    p.N = a.N;
    p.causal = a.causal;
    p.row_blocks = (a.N + kBM - 1) / kBM;
    const int kv_units = a.B * a.H_kv;
    p.xcd_units = (kv_units % 8 == 0) ? kv_units / 8 : 0;
    p.sc_log2 = scale * kLog2e;
    p.eps = a.eps;
    p.one_minus_init = 1.0f - lambda_init;
    const int64_t blocks = (int64_t)a.B * a.H * p.row_blocks;
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    const bool shared = a.k1 == a.k2 && a.sk1[0] == a.sk2[0] && a.sk1[1] == a.sk2[1] && a.sk1[2] == a.sk2[2];
    const bool norm = a.norm == DIFFATTN_NORM_RMS;
    const int nb = (int)blocks;
    if (a.d_qk == 64) {
        if (shared) return norm ? launch_t<64, true, true>(p, nb, stream) : launch_t<64, true, false>(p, nb, stream);
        return norm ? launch_t<64, false, true>(p, nb, stream) : launch_t<64, false, false>(p, nb, stream);
    }
    if (shared) return norm ? launch_t<128, true, true>(p, nb, stream) : launch_t<128, true, false>(p, nb, stream);
    return norm ? launch_t<128, false, true>(p, nb, stream) : launch_t<128, false, false>(p, nb, stream);
}

}  // namespace da
