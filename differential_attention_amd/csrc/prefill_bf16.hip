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
// Work decomposition. One work-group = 4 waves = 128 query rows of one output
// head; two work-groups share a CU (at most 128 VGPRs + 128 AGPRs per lane,
// so two waves per SIMD interleave matrix-core and vector work).
//  * Each wave owns 32 query rows. Its Q1/Q2 rows live in registers as MFMA B
//    operands for the whole sweep; O1^T, O2^T (d_v x 32) live in AGPRs.
//  * Key tiles of 64 keys stream HBM -> LDS with global_load_lds (16 bytes a
//    lane, no register staging), double-buffered: the loads of tile t+1 are
//    in flight while tile t is used. One key tile feeds both branches when
//    K1 == K2 (V2); the value tile is loaded once and read once for both
//    branches.
//  * Per 32-key sub-block and branch: S^T = K Q^T (32 keys x 32 queries,
//    v_mfma_f32_32x32x16_bf16), so a lane holds 16 scores of ONE query: the
//    row max needs one v_permlane32_swap and the row sum stays lane-local
//    until the end. The key order inside a sub-block is permuted when K rows
//    are read (bits 2 and 3 of the row index swapped) so that the 8 scores a
//    lane holds for a 16-key step are 8 consecutive keys.
//  * O^T += V^T P^T: the probabilities go straight from the S^T registers into
//    the B operand; the V^T operand is read from the row-major V tile with
//    ds_read_b64_tr_b16 (two reads give a lane 8 consecutive keys of one value
//    column).
//  * LDS tiles have no padding; 16-byte chunks are XOR-swizzled per row so the
//    K-operand reads and the transposing V reads are free of bank conflicts.
//  * Lazy rescale: a branch's reference max moves only when a block max
//    exceeds it by 2^8, so the AGPR accumulators are rarely rescaled.
//  * Causal: key tiles past the work-group's last row are never loaded; a wave
//    stops at its diagonal sub-block, the only one it masks (with the ragged
//    end of the sequence). Work-groups with the longest rows run first.
// Grid mapping: work-groups are dispatched round-robin over the 8 XCDs; when
// the number of (batch, KV head) units is a multiple of 8, all work-groups
// reading one KV head are placed on the same XCD so its K/V stay in that
// XCD's L2.
#include "common.hpp"
#include "launch.hpp"

namespace da {

namespace {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kDV = 128;              // value width (both forms)
constexpr int kBM = 128;              // query rows per work-group
constexpr int kWM = 32;               // query rows per wave
constexpr int kBN = 64;               // keys per LDS tile
constexpr float kRescaleLog2 = 8.0f;  // lazy-rescale threshold (log2 units)

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

// Key offset (within a sub-block, before adding 8 * lane-half) held by
// register r of an S^T accumulator.
__device__ __forceinline__ constexpr int key_of_reg(int r) { return 16 * ((r >> 3) & 1) + 4 * ((r >> 2) & 1) + (r & 3); }

// XOR swizzle of the 16-byte chunk index inside a K-tile row (row bytes
// 2 * DQK): keeps the 16 lanes of one ds_read_b128 pass on distinct banks.
template <int DQK>
__device__ __forceinline__ int k_swz(int row) {
    return DQK == 128 ? (row & 15) : ((row >> 1) & 7);
}
// XOR swizzle of the chunk index inside a V-tile row (256 bytes): the four
// rows read by one ds_read_b64_tr_b16 pass land on distinct banks.
__device__ __forceinline__ int v_swz(int row) { return (row & 3) << 2; }

__device__ __forceinline__ uint4 ldg16(const __bf16 *p) { return *(const uint4 *)p; }

__device__ __forceinline__ void wait_vmem_all() {
    // s_waitcnt vmcnt(0) (expcnt and lgkmcnt left at their maxima)
    __builtin_amdgcn_s_waitcnt(0x0F70);
}

template <int DQK, bool SHARED_K>
struct Tile {
    static constexpr int kKBytes = kBN * DQK * 2;             // one K tile
    static constexpr int kVBytes = kBN * kDV * 2;             // the V tile
    static constexpr int kNK = SHARED_K ? 1 : 2;              // K tiles per stage
    static constexpr int kStage = kNK * kKBytes + kVBytes;    // bytes per stage
    static constexpr int kKCh = DQK / 8;                      // 16-byte chunks per K row
    static constexpr int kKLoads = kKBytes / 1024 / 4;        // 1 KB loads per wave per K tile
};

template <int DQK, bool SHARED_K, bool NORM>
__global__ __launch_bounds__(256, DQK == 64 ? 2 : 1) void prefill_bf16_kernel(Bf16Params p) {
    using T = Tile<DQK, SHARED_K>;
    constexpr int KC = DQK / 16;  // 16-wide k steps of the QK contraction
    __shared__ __attribute__((aligned(1024))) unsigned char lds[2 * T::kStage];

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
        const int row = min(myrow, p.N - 1);  // rows past the end compute garbage, never stored
        const __bf16 *q1 = p.q1 + b * p.sq1[0] + h * p.sq1[1] + (int64_t)row * p.sq1[2] + 8 * hh;
        const __bf16 *q2 = p.q2 + b * p.sq2[0] + h * p.sq2[1] + (int64_t)row * p.sq2[2] + 8 * hh;
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) {
            qf1[kc] = as_bf16x8(ldg16(q1 + 16 * kc));
            qf2[kc] = as_bf16x8(ldg16(q2 + 16 * kc));
        }
    }

    const __bf16 *kb1 = p.k1 + b * p.sk1[0] + g * p.sk1[1];
    const __bf16 *kb2 = p.k2 + b * p.sk2[0] + g * p.sk2[1];
    const __bf16 *vb = p.v + b * p.sv[0] + g * p.sv[1];
    const int64_t sk1n = p.sk1[2], sk2n = p.sk2[2], svn = p.sv[2];

    const int kend = p.causal ? min(p.N, q0 + kBM) : p.N;
    const int ntiles = (kend + kBN - 1) / kBN;
    // sub-blocks this wave needs; the last one is the only masked one
    const int wend = p.causal ? min(p.N, wrow0 + kWM) : p.N;
    const int nsub = wrow0 < p.N ? (wend + 31) / 32 : 0;

    // ---- per-lane constants of the global -> LDS copies. Load i of wave w
    // fills the 1 KB block (4 i + w) of a region; lane l fills its 16-byte
    // slot l. Slot -> (row, physical chunk) -> logical chunk via the swizzle.
    // K (DQK 128): 16 chunks a row, 4 rows per block; (DQK 64): 8 chunks, 8 rows.
    constexpr int kRowsPerBlock = 1024 / (2 * DQK);
    const int k_row_l = lane / T::kKCh;                        // row inside the block
    const int k_pc = lane % T::kKCh;                            // physical chunk
    const int k_col = 8 * (k_pc ^ k_swz<DQK>(wave * kRowsPerBlock + k_row_l));
    const int v_row_l = lane >> 4;
    const int v_col = 8 * ((lane & 15) ^ v_swz(v_row_l));

    auto issue_tile = [&](int t, int stage) {
        const int key0 = t * kBN;
        unsigned char *base = lds + stage * T::kStage;
#pragma unroll
        for (int i = 0; i < T::kKLoads; ++i) {
            const int blk = 4 * i + wave;
            const int key = min(key0 + blk * kRowsPerBlock + k_row_l, p.N - 1);
            __builtin_amdgcn_global_load_lds(kb1 + (int64_t)key * sk1n + k_col,
                                             (lds_void *)(base + blk * 1024), 16, 0, 0);
            if constexpr (!SHARED_K)
                __builtin_amdgcn_global_load_lds(kb2 + (int64_t)key * sk2n + k_col,
                                                 (lds_void *)(base + T::kKBytes + blk * 1024), 16, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int blk = 4 * i + wave;
            const int key = min(key0 + blk * 4 + v_row_l, p.N - 1);
            __builtin_amdgcn_global_load_lds(vb + (int64_t)key * svn + v_col,
                                             (lds_void *)(base + T::kNK * T::kKBytes + blk * 1024), 16, 0, 0);
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

    // byte offset of this lane's K-operand chunk for k step kc, sub-block sb
    const int krow = perm_key(l32);
    auto k_addr = [&](int sb, int kc) {
        const int row = 32 * sb + krow;
        const int c = (2 * kc + hh) ^ k_swz<DQK>(row);
        return row * (2 * DQK) + 16 * c;
    };
    // byte offsets of this lane's two transposing V reads for (sb, k step t, dv block dc)
    const int vi = lane & 15;           // lane inside its 16-lane group
    const int vdv0 = 16 * ((lane >> 4) & 1);
    auto v_addr = [&](int sb, int t, int dc, int half) {
        const int row = 32 * sb + 16 * t + 8 * hh + 4 * half + (vi >> 2);
        const int col = 32 * dc + vdv0 + 4 * (vi & 3);
        const int c = (col >> 3) ^ v_swz(row);
        return row * 256 + 16 * c + 2 * (col & 7);
    };

    // scores of one branch for one sub-block, masked when `mask`
    auto scores = [&](const unsigned char *ktile, const bf16x8 *qf, int sb, bool mask, int lim) {
        f32x16 s = f32x16{};
#pragma unroll
        for (int kc = 0; kc < KC; ++kc)
            s = mfma32(as_bf16x8(*(const uint4 *)(ktile + k_addr(sb, kc))), qf[kc], s);
        if (mask) {
#pragma unroll
            for (int r = 0; r < 16; ++r)
                if (key_of_reg(r) >= lim) s[r] = -INFINITY;
        }
        return s;
    };
    // online softmax of one branch: returns the bf16 probabilities for the two
    // 16-key steps, updates (m, l) and rescales o when the reference max moves
    auto softmax = [&](f32x16 s, float &m, float &l, f32x16 *o, bf16x8 &pb0, bf16x8 &pb1) {
        float mx = fmaxf(fmaxf(s[0], s[1]), s[2]);
#pragma unroll
        for (int r = 3; r < 15; r += 2) mx = fmaxf(fmaxf(mx, s[r]), s[r + 1]);
        mx = fmaxf(mx, s[15]);
        const float mxs = halves_max(mx) * p.sc_log2;
        if (__any(mxs > m + kRescaleLog2)) {
            const float mnew = fmaxf(m, mxs);
            const float alpha = (m == mnew) ? 1.0f : exp2_fast(m - mnew);
            m = mnew;
            l *= alpha;
#pragma unroll
            for (int dc = 0; dc < 4; ++dc) o[dc] *= alpha;
        }
        const float msub = (m == -INFINITY) ? 0.0f : m;
        float ps[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) ps[r] = exp2_fast(fmaf(s[r], p.sc_log2, -msub));
        float a0 = (ps[0] + ps[1]) + (ps[2] + ps[3]);
        float a1 = (ps[4] + ps[5]) + (ps[6] + ps[7]);
        float a2 = (ps[8] + ps[9]) + (ps[10] + ps[11]);
        float a3 = (ps[12] + ps[13]) + (ps[14] + ps[15]);
        l += (a0 + a1) + (a2 + a3);
        pb0 = pack8(ps[0], ps[1], ps[2], ps[3], ps[4], ps[5], ps[6], ps[7]);
        pb1 = pack8(ps[8], ps[9], ps[10], ps[11], ps[12], ps[13], ps[14], ps[15]);
    };

    auto step = [&](const unsigned char *base, int sb, bool mask, int lim) {
        const unsigned char *kt1 = base;
        const unsigned char *kt2 = SHARED_K ? base : base + T::kKBytes;
        const unsigned char *vt = base + T::kNK * T::kKBytes;
        bf16x8 p10, p11, p20, p21;
        softmax(scores(kt1, qf1, sb, mask, lim), m1, l1, o1, p10, p11);
        softmax(scores(kt2, qf2, sb, mask, lim), m2, l2, o2, p20, p21);
#pragma unroll
        for (int dc = 0; dc < 4; ++dc) {
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(vt + v_addr(sb, t, dc, 0)));
                const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(vt + v_addr(sb, t, dc, 1)));
                const bf16x8 va = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
                o1[dc] = mfma32(va, t ? p11 : p10, o1[dc]);
                o2[dc] = mfma32(va, t ? p21 : p20, o2[dc]);
            }
        }
    };

    // ---- the key sweep
    if (ntiles > 0) issue_tile(0, 0);
    for (int t = 0; t < ntiles; ++t) {
        wait_vmem_all();
        __syncthreads();  // tile t visible to all waves; tile t-1 no longer read
        if (t + 1 < ntiles) issue_tile(t + 1, (t + 1) & 1);
        const unsigned char *base = lds + (t & 1) * T::kStage;
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
            const int j = 2 * t + sb;
            if (j < nsub - 1) {
                step(base, sb, false, 0);
            } else if (j == nsub - 1) {
                // diagonal / ragged-end sub-block: key index >= lim is masked
                const int key0 = j * 32 + 8 * hh;
                const int lim = (p.causal ? min(myrow + 1, p.N) : p.N) - key0;
                step(base, sb, true, lim);
            }
        }
    }

    // ---- epilogue: y = O1 / l1 - lambda O2 / l2 (then the V1 norm), bf16 store
    l1 = halves_sum(l1);
    l2 = halves_sum(l2);
    const float r1 = 1.0f / l1;
    const float r2 = p.lambda[h] / l2;
    f32x16 y[4];
    {
        // both products rounded separately (no fused multiply-add), so identical
        // branches with lambda = 1 give exactly zero
#pragma clang fp contract(off)
#pragma unroll
        for (int dc = 0; dc < 4; ++dc) y[dc] = o1[dc] * r1 - o2[dc] * r2;
    }
    if constexpr (NORM) {
        float ss = 0.0f;
#pragma unroll
        for (int dc = 0; dc < 4; ++dc)
#pragma unroll
            for (int r = 0; r < 16; ++r) ss = fmaf(y[dc][r], y[dc][r], ss);
        ss = halves_sum(ss);
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
