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
// Work decomposition. A work-group of 8 waves owns a block of query rows of
// one output head, in 32-row groups, one per wave or per pair of waves:
//  * d_qk 64 (V1 shapes): 256 rows, each wave computes both branches of its
//    32 rows (256 unified registers a lane, two waves per SIMD, one
//    work-group a CU), so one key/value tile stream feeds 256 rows;
//  * d_qk 128 (V2 shapes): 128 rows, waves 2r and 2r+1 own rows
//    32r..32r+31, the first for branch 1, the second for branch 2. Splitting
//    the branches halves each wave's state (Q rows as MFMA B operands, one
//    d_v x 32 accumulator), so two waves share a SIMD where one wave holding
//    both branches would not fit twice.
//  * Key tiles of 64 keys stream HBM -> LDS with global_load_lds (16 bytes a
//    lane, no register staging), double-buffered: the loads of tile t+1 are
//    in flight while tile t is used. One key tile feeds both branches when
//    K1 == K2 (V2); the value tile is loaded once for both branches.
//  * Per 32-key sub-block: S^T = K Q^T (32 keys x 32 queries,
//    v_mfma_f32_32x32x16_bf16), so a lane holds 16 scores of ONE query: the
//    row max needs one v_permlane32_swap and the row sum stays lane-local
//    until the end. The key order inside a sub-block is permuted when K rows
//    are read (bits 2 and 3 of the row index swapped) so that the 8 scores a
//    lane holds for a 16-key step are 8 consecutive keys.
//  * O^T += V^T P^T: the probabilities go straight from the S^T registers into
//    the B operand; the V^T operand is read from the row-major V tile with
//    ds_read_b64_tr_b16 (two reads give a lane 8 consecutive keys of one value
//    column). The row sum accumulates the bf16 probabilities the product
//    uses, two at a time (v_dot2_f32_bf16 against ones).
//  * LDS tiles have no padding; 16-byte chunks are XOR-swizzled per row so the
//    K-operand reads and the transposing V reads are free of bank conflicts.
//  * Fixed-reference sweep: when every row sees at least 256 keys and the
//    scores of 32 sampled keys span at most 12 log2 units in every row, the
//    queries are pre-scaled by scale * log2(e) (rounded once to bf16) and the
//    probabilities are 2^s against a fixed reference of 0: no running max,
//    no subtraction, no rescale (about half the softmax's VALU work). The
//    sums are checked once, after the sweep; a row out of range sends the
//    work-group through the exact sweep from the start.
//  * Exact sweep (otherwise, and with stored statistics): lazy rescale, a
//    wave's reference max moves only when a block max exceeds it by 2^8, so
//    the accumulators are rarely rescaled.
//  * Causal: key tiles past the work-group's last row are never loaded; a wave
//    stops at its diagonal sub-block, the only one it masks (with the ragged
//    end of the sequence). Work-groups with the longest rows run first.
//  * Epilogue: y = O1 / l1 - lambda O2 / l2 (when the branches live in two
//    waves, the branch-2 wave leaves lambda O2 / l2 in LDS for its partner),
//    then the V1 norm, then one bf16 store.
// Grid mapping: work-groups are dispatched round-robin over the 8 XCDs; when
// the number of (batch, KV head) units is a multiple of 8, all work-groups
// reading one KV head are placed on the same XCD so its K/V stay in that
// XCD's L2.
#include "launch.hpp"
#include "tiles.hpp"

#include <climits>
#include <type_traits>

namespace da {

namespace {

constexpr int kWM = 32;               // query rows per wave
constexpr float kRescaleLog2 = 8.0f;  // lazy-rescale threshold (log2 units)
// Fixed-reference sweep: with the queries pre-scaled by scale * log2(e) the
// products give the scores in log2 units, and the probabilities are taken as
// 2^s against a fixed reference of 0 (no running max, no subtraction, no
// rescale). That is the same softmax as long as the sums stay in range, which
// is checked once, after the sweep: a row whose sum is not within
// [kFastMinSum, kFastMaxSum] (a score above about 64 or a row whose scores are
// all below about -60, in log2 units) or whose accumulators are not finite
// sends its work-group through the exact sweep (running max, lazy rescale).
constexpr float kFastMinSum = 8.673617379884035e-19f;  // 2^-60
constexpr int kFastMinKeys = 256;     // rows with fewer visible keys take the exact sweep
constexpr float kFastMaxRange = 12.0f;  // largest sampled score span (log2 units) of the fixed-reference sweep
constexpr float kFastMaxSum = 1.8446744073709552e19f;  // 2^64

// branch-split decomposition for a head dimension (see the header comment)
template <int DQK>
struct Split {
    static constexpr bool kOn = DQK == 128;
    static constexpr int kThreads = 512;
    static constexpr int kBM = kOn ? 128 : 256;  // query rows per work-group
    static constexpr int kNBr = kOn ? 1 : 2;  // branches per wave
    static constexpr int kMinBlocks = 1;
};

struct Bf16Params {
    const __bf16 *q1, *q2, *k1, *k2, *v;
    int64_t sq1[3], sq2[3], sk1[3], sk2[3], sv[3], so[3];
    const float *lambda, *gamma;
    __bf16 *out;
    float *o1, *o2, *lse1, *lse2;  // optional statistics for the backward pass (all or none)
    int B, H, H_kv, group, N, causal, window, row_blocks, xcd_units;
    int group_norm;  // the norm subtracts the channel mean first (GroupNorm per head)
    int off32;       // each (batch, KV head) slice of K1, K2 and V spans fewer than 2^31 bytes
    float sc_log2;  // scale * log2(e)
    float eps, one_minus_init;
};

// STATS: also store each branch's normalised output and log-sum-exp for the
// backward pass (o1, o2, lse1, lse2); such calls take the exact sweep only.
template <int DQK, bool SHARED_K, bool NORM, bool WIN, bool STATS>
__global__ __launch_bounds__(Split<DQK>::kThreads, Split<DQK>::kMinBlocks) void prefill_bf16_kernel(Bf16Params p) {
    using T = Tile<DQK, SHARED_K>;
    using S = Split<DQK>;
    constexpr int KC = DQK / 16;           // 16-wide k steps of the QK contraction
    constexpr int NBR = S::kNBr;           // branches computed by one wave
    constexpr int NW = S::kThreads / 64;   // waves per work-group
    // Two stages in two distinct LDS objects: the compiler then knows that the
    // reads of one stage do not depend on the asynchronous copies into the
    // other, and does not wait for the next tile's loads before reading this
    // one. With split branches the epilogue reuses the stages for 4 waves x
    // 64 lanes x 64 floats (two row groups in each).
    constexpr int kStageBytes = (S::kOn && T::kStage < 32768) ? 32768 : T::kStage;
    __shared__ __attribute__((aligned(1024))) unsigned char st0[kStageBytes];
    __shared__ __attribute__((aligned(1024))) unsigned char st1[kStageBytes];
    __shared__ int redo_flag;  // a row left the fixed-reference range: redo the sweep exactly

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    if (tid == 0) redo_flag = 0;  // read only after the sweep's barriers
    const int l32 = lane & 31;
    const int hh = lane >> 5;
    const int br0 = S::kOn ? (wave & 1) : 0;   // first branch of this wave (0: Q1/K1, 1: Q2/K2)
    const int rg = S::kOn ? (wave >> 1) : wave;  // row group

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
    const int q0 = rb * S::kBM;
    const int wrow0 = q0 + rg * kWM;  // first query row of this wave
    const int myrow = wrow0 + l32;    // the query row of this lane

    const __bf16 *kb1 = p.k1 + b * p.sk1[0] + g * p.sk1[1];
    const __bf16 *kb2 = p.k2 + b * p.sk2[0] + g * p.sk2[1];
    const __bf16 *vb = p.v + b * p.sv[0] + g * p.sv[1];
    const int64_t sk1n = p.sk1[2], sk2n = p.sk2[2], svn = p.sv[2];

    // ---- Q fragments of this wave's branches (B operands): Q[myrow][16 kc + 8 hh .. +7]
    bf16x8 qf[NBR][KC];
    auto load_q = [&]() DA_INLINE {
        const int row = min(myrow, p.N - 1);  // rows past the end compute garbage, never stored
#pragma unroll
        for (int j = 0; j < NBR; ++j) {
            const __bf16 *q = (br0 + j) ? p.q2 + b * p.sq2[0] + h * p.sq2[1] + (int64_t)row * p.sq2[2]
                                        : p.q1 + b * p.sq1[0] + h * p.sq1[1] + (int64_t)row * p.sq1[2];
#pragma unroll
            for (int kc = 0; kc < KC; ++kc) qf[j][kc] = as_bf16x8(ldg16(q + 8 * hh + 16 * kc));
        }
    };
    load_q();

    // ---- exact or fixed-reference sweep (see kFastMinSum) for this work-group.
    // The fixed-reference sweep needs the queries pre-scaled: q * scale *
    // log2(e), rounded once to bf16, so that the products give the scores in
    // log2 units. That rounding moves each score by about 2^-10 of the spread
    // of its terms across keys, so the sweep is taken only where that stays
    // small against the rounding of the probabilities themselves:
    //  * every row sees at least kFastMinKeys keys (in rows of a few keys
    //    whose two branches nearly cancel, the V1 norm magnifies any error);
    //  * the scores of 32 keys every row sees (sampled before the sweep) span
    //    at most kFastMaxRange in every row.
    // Calls that store statistics always take the exact sweep (the backward
    // recomputes the exact scores against the stored log-sum-exp). Neither
    // test is needed for the result to be right: the exact sweep is always
    // available.
    const int min_keys = WIN ? min(p.causal ? q0 + 1 : p.N, p.window) : (p.causal ? q0 + 1 : p.N);
    // first sampled key: the window start of the work-group's last row, so
    // that keys ks .. ks+31 are visible to every row (a window that cuts no
    // row's keys samples the same keys as no window)
    const int ks = WIN ? max(0, min(q0 + S::kBM, p.N) - p.window) : 0;
    bool fast = !STATS && min_keys >= kFastMinKeys && ks + 31 <= (p.causal ? q0 : p.N - 1);
    float scl = p.sc_log2;  // multiplier from the products' scores to log2 units
    if (fast) {  // work-group-uniform
#pragma unroll
        for (int j = 0; j < NBR; ++j)
#pragma unroll
            for (int kc = 0; kc < KC; ++kc) {
                const bf16x8 x = qf[j][kc];
                qf[j][kc] = pack8((float)x[0] * p.sc_log2, (float)x[1] * p.sc_log2, (float)x[2] * p.sc_log2,
                                  (float)x[3] * p.sc_log2, (float)x[4] * p.sc_log2, (float)x[5] * p.sc_log2,
                                  (float)x[6] * p.sc_log2, (float)x[7] * p.sc_log2);
            }
        // the sample: keys ks .. ks+31 against this lane's row, straight from
        // global memory (S^T = K Q^T as in the sweep, unpermuted key order)
        float span = 0.0f;
        {
            const int key = ks + l32;
#pragma unroll
            for (int j = 0; j < NBR; ++j) {
                const __bf16 *kr = ((br0 + j) ? kb2 + (int64_t)key * sk2n : kb1 + (int64_t)key * sk1n) + 8 * hh;
                f32x16 sv = f32x16{};
#pragma unroll
                for (int kc = 0; kc < KC; ++kc) sv = mfma32(as_bf16x8(ldg16(kr + 16 * kc)), qf[j][kc], sv);
                float mx = sv[0], mn = sv[0];
#pragma unroll
                for (int r = 1; r < 16; ++r) {
                    mx = fmaxf(mx, sv[r]);
                    mn = fminf(mn, sv[r]);
                }
                span = fmaxf(span, halves_max(mx) + halves_max(-mn));
            }
        }
        const bool wide = !(span <= kFastMaxRange) && myrow < p.N;
        __syncthreads();  // redo_flag cleared
        if (__any(wide) && lane == 0) redo_flag = 1;
        __syncthreads();
        if (redo_flag) {
            fast = false;
            load_q();  // back to the exact queries
        } else {
            scl = 1.0f;
        }
        __syncthreads();  // every wave has read the flag
        if (tid == 0) redo_flag = 0;  // for the check after the sweep (read after its barriers)
    }

    const int kend = p.causal ? min(p.N, q0 + S::kBM) : p.N;
    const int ntiles = (kend + kBN - 1) / kBN;
    // causal window W: row i sees keys i-W+1 .. i, so tiles below the work-
    // group's first row's window are never loaded, sub-blocks below this
    // wave's first row's window are skipped, and sub-blocks holding a key
    // below its last row's window start are masked from below
    const int win = WIN ? p.window : 0;  // (a separate instantiation when windowed)
    const int tlo = WIN ? max(0, q0 - win + 1) / kBN : 0;
    const int jlo = WIN ? max(0, wrow0 - win + 1) / 32 : 0;
    const int jmask = WIN ? (max(0, wrow0 + kWM - win) + 31) / 32 : 0;  // sub-blocks < jmask: lower mask
    // sub-blocks this wave needs; the last one is masked from above
    const int wend = p.causal ? min(p.N, wrow0 + kWM) : p.N;
    const int nsub = wrow0 < p.N ? (wend + 31) / 32 : 0;

    // ---- global -> LDS copies: 1 KB block B of a stage is filled by wave
    // B % NW (load B / NW), lane l filling 16-byte slot l; blocks [0, kKBlocks)
    // hold the K tile(s), the rest the V tile. Slot -> (row, physical chunk)
    // -> logical chunk through the row's swizzle.
    static_assert(T::kBlocks % NW == 0, "stage blocks must divide among the waves");
    static_assert((T::kKBytes / 1024) % NW == 0, "a wave's copy i reads one tensor, fixed by i");
    constexpr int NC = T::kBlocks / NW;  // copies per wave and tile
    constexpr int KPB = T::kKBytes / 1024 / NW;  // copies per K tile
    const int wv = wave_id();            // the wave index as a scalar
    // With off32, a whole tile in range is copied by buffer loads: the
    // (batch, KV head) slice's base in a buffer descriptor, a scalar offset
    // (the tile's first key, and the copy's first row inside the tile, times
    // the row stride) and one per-lane offset per tensor, so a tile costs no
    // vector arithmetic. The copies of one tensor differ only by whole rows
    // (NW blocks apart: a multiple of every swizzle's period), so one lane
    // offset serves them all; K1 and K2 share theirs (off32 requires equal
    // row strides). The last, partial tile (rows clamped to the last key) and
    // huge strides take the general form below.
    constexpr int KRows = NW * T::kRowsPerKBlock;  // rows between a wave's consecutive K copies
    constexpr int VRows = NW * 4;                  // and between its V copies (4 rows a block)
    static_assert(KRows % 16 == 0 && VRows % 4 == 0, "copy row steps must keep the swizzles");
    uint32_t koff, voff;
    {
        const int krow = wv * T::kRowsPerKBlock + lane / T::kKCh;
        koff = 2u * (uint32_t)(krow * sk1n + 8 * ((lane % T::kKCh) ^ k_swz<DQK>(krow)));
        const int vrow = wv * 4 + (lane >> 4);
        voff = 2u * (uint32_t)(vrow * svn + 8 * ((lane & 15) ^ v_swz(vrow)));
    }
    // raw buffer descriptors (stride 0, 32-bit data format: dword 3 =
    // 0x00020000) over the three slices; range 2^31 - 1 bytes (off32)
    const __amdgpu_buffer_rsrc_t rk1 = __builtin_amdgcn_make_buffer_rsrc((void *)kb1, (short)0, 0x7fffffff, 0x00020000);
    const __amdgpu_buffer_rsrc_t rk2 = __builtin_amdgcn_make_buffer_rsrc((void *)kb2, (short)0, 0x7fffffff, 0x00020000);
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc((void *)vb, (short)0, 0x7fffffff, 0x00020000);
    auto issue_tile = [&](int t, unsigned char *base) DA_INLINE {
        const int key0 = __builtin_amdgcn_readfirstlane(t * kBN);  // uniform: keeps the offsets scalar
        if (p.off32 && key0 + kBN <= p.N) {
#pragma unroll
            for (int i = 0; i < NC; ++i) {
                const int blk = wv + NW * i;
                if (i < T::kNK * KPB) {
                    const int kt = i / KPB, j = i % KPB;  // tensor, and copy inside it
                    const uint32_t so = 2u * (uint32_t)(key0 + j * KRows) * (uint32_t)sk1n;
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(kt ? rk2 : rk1, (lds_void *)(base + blk * 1024), 16,
                                                             koff, so, 0, 0);
                } else {
                    const int j = i - T::kNK * KPB;
                    const uint32_t so = 2u * (uint32_t)(key0 + j * VRows) * (uint32_t)svn;
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void *)(base + blk * 1024), 16, voff, so, 0,
                                                             0);
                }
            }
        return;
        }
#pragma unroll
        for (int i = 0; i < NC; ++i) {
            const int blk = wave + NW * i;
            if (blk < T::kKBlocks) {
                const int kt = blk / (T::kKBytes / 1024);  // which K tile (0: K1, 1: K2)
                const int kblk = blk % (T::kKBytes / 1024);
                const int row = kblk * T::kRowsPerKBlock + lane / T::kKCh;
                const int col = 8 * ((lane % T::kKCh) ^ k_swz<DQK>(row));
                const int key = min(key0 + row, p.N - 1);
                const __bf16 *src = (kt ? kb2 + (int64_t)key * sk2n : kb1 + (int64_t)key * sk1n) + col;
                __builtin_amdgcn_global_load_lds(src, (lds_void *)(base + blk * 1024), 16, 0, 0);
            } else {
                const int vblk = blk - T::kKBlocks;
                const int row = vblk * 4 + (lane >> 4);
                const int col = 8 * ((lane & 15) ^ v_swz(row));
                const int key = min(key0 + row, p.N - 1);
                __builtin_amdgcn_global_load_lds(vb + (int64_t)key * svn + col,
                                                 (lds_void *)(base + blk * 1024), 16, 0, 0);
            }
        }
    };

    // ---- online-softmax state of this wave's branches
    // l sums the bf16-rounded probabilities the value products use (so the
    // output's weights sum to one); le (statistics only) sums them unrounded,
    // for the log-sum-exp
    f32x16 o[NBR][4];
    float m[NBR], l[NBR], le[NBR];
#pragma unroll
    for (int j = 0; j < NBR; ++j) {
#pragma unroll
        for (int dc = 0; dc < 4; ++dc) o[j][dc] = f32x16{};
        m[j] = -INFINITY;
        l[j] = 0.0f;
        le[j] = 0.0f;
    }

    // byte offset of this lane's K-operand chunk for k step kc, sub-block sb
    const int krow = perm_key(l32);
    auto k_addr = [&](int sb, int kc) DA_INLINE {
        const int row = 32 * sb + krow;
        const int c = (2 * kc + hh) ^ k_swz<DQK>(row);
        return row * (2 * DQK) + 16 * c;
    };
    // byte offset of one of this lane's two transposing V reads for
    // (sub-block sb, k step t, dv block dc, half)
    const int vi = lane & 15;  // lane inside its 16-lane group
    const int vdv0 = 16 * ((lane >> 4) & 1);
    auto v_addr = [&](int sb, int t, int dc, int half) DA_INLINE {
        const int row = 32 * sb + 16 * t + 8 * hh + 4 * half + (vi >> 2);
        const int col = 32 * dc + vdv0 + 4 * (vi & 3);
        const int c = (col >> 3) ^ v_swz(row);
        return row * 256 + 16 * c + 2 * (col & 7);
    };
    const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};

    // online softmax of one branch's scores (reference max moved lazily), bf16
    // probabilities for the two 16-key steps
    auto softmax_branch = [&](f32x16 s, bool mask, int lim, int lo, float &mr, float &lr, float &er, f32x16 *orr,
                              bf16x8 &pb0, bf16x8 &pb1) DA_INLINE {
        if (mask) {
            // an opaque statement keeps this a branch taken by the few masked
            // sub-blocks, instead of per-element selects evaluated for all
            asm volatile("");
#pragma unroll
            for (int r = 0; r < 16; ++r)
                if (key_of_reg(r) >= lim || key_of_reg(r) < lo) s[r] = -INFINITY;
        }
        float mx = fmaxf(fmaxf(s[0], s[1]), s[2]);
#pragma unroll
        for (int r = 3; r < 15; r += 2) mx = fmaxf(fmaxf(mx, s[r]), s[r + 1]);
        mx = fmaxf(mx, s[15]);
        const float mxs = halves_max(mx) * scl;
        if (__any(mxs > mr + kRescaleLog2)) {
            const float mnew = fmaxf(mr, mxs);
            const float alpha = (mr == mnew) ? 1.0f : exp2_fast(mr - mnew);
            mr = mnew;
            lr *= alpha;
            if constexpr (STATS) er *= alpha;
#pragma unroll
            for (int dc = 0; dc < 4; ++dc) orr[dc] *= alpha;
        }
        const float msub = (mr == -INFINITY) ? 0.0f : mr;
#pragma unroll
        for (int r = 0; r < 16; ++r) s[r] = exp2_fast(fmaf(s[r], scl, -msub));
        if constexpr (STATS) {
            float e0 = s[0] + s[1], e1 = s[2] + s[3];
#pragma unroll
            for (int r = 4; r < 16; r += 4) {
                e0 += s[r] + s[r + 1];
                e1 += s[r + 2] + s[r + 3];
            }
            er += e0 + e1;
        }
        bf16x2 pp[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) pp[i] = pack2(s[2 * i], s[2 * i + 1]);
        // row sum of the rounded probabilities the product uses
        float l0 = __builtin_amdgcn_fdot2_f32_bf16(pp[0], ones, 0.0f, false);
        float l1 = __builtin_amdgcn_fdot2_f32_bf16(pp[4], ones, 0.0f, false);
#pragma unroll
        for (int i = 1; i < 4; ++i) {
            l0 = __builtin_amdgcn_fdot2_f32_bf16(pp[i], ones, l0, false);
            l1 = __builtin_amdgcn_fdot2_f32_bf16(pp[4 + i], ones, l1, false);
        }
        lr += l0 + l1;
        pb0 = bf16x8{pp[0][0], pp[0][1], pp[1][0], pp[1][1], pp[2][0], pp[2][1], pp[3][0], pp[3][1]};
        pb1 = bf16x8{pp[4][0], pp[4][1], pp[5][0], pp[5][1], pp[6][0], pp[6][1], pp[7][0], pp[7][1]};
    };

    // the fixed-reference form of one branch: p = 2^s (scores already in log2
    // units), bf16 probabilities and this block's row sum lb of the rounded values
    auto softmax_fast = [&](f32x16 s, bool mask, int lim, int lo, bf16x8 &pb0, bf16x8 &pb1,
                            float &lb) DA_INLINE {
        if (mask) {
            asm volatile("");
#pragma unroll
            for (int r = 0; r < 16; ++r)
                if (key_of_reg(r) >= lim || key_of_reg(r) < lo) s[r] = -INFINITY;
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) s[r] = exp2_fast(s[r]);
        bf16x2 pp[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) pp[i] = pack2(s[2 * i], s[2 * i + 1]);
        float l0 = __builtin_amdgcn_fdot2_f32_bf16(pp[0], ones, 0.0f, false);
        float l1 = __builtin_amdgcn_fdot2_f32_bf16(pp[4], ones, 0.0f, false);
#pragma unroll
        for (int i = 1; i < 4; ++i) {
            l0 = __builtin_amdgcn_fdot2_f32_bf16(pp[i], ones, l0, false);
            l1 = __builtin_amdgcn_fdot2_f32_bf16(pp[4 + i], ones, l1, false);
        }
        lb = l0 + l1;
        pb0 = bf16x8{pp[0][0], pp[0][1], pp[1][0], pp[1][1], pp[2][0], pp[2][1], pp[3][0], pp[3][1]};
        pb1 = bf16x8{pp[4][0], pp[4][1], pp[5][0], pp[5][1], pp[6][0], pp[6][1], pp[7][0], pp[7][1]};
    };
    // one 32-key sub-block: scores, softmax (fixed-reference or exact form,
    // chosen at compile time by the tag), value products
    auto step = [&](auto fast_tag, const unsigned char *base, int sb, bool mask, int lim, int lo) DA_INLINE {
        constexpr bool kFast = decltype(fast_tag)::value;
        const unsigned char *vt = base + T::kNK * T::kKBytes;
        // every key fragment of the sub-block is read before the first product
        // (the reads then overlap each other instead of each product waiting
        // for its own read); then every branch's score products, so that with
        // two branches per wave the two product chains interleave
        bf16x8 kf[NBR][KC];
#pragma unroll
        for (int j = 0; j < NBR; ++j)
#pragma unroll
            for (int kc = 0; kc < KC; ++kc)
                kf[j][kc] = as_bf16x8(*(const uint4 *)(base + (SHARED_K ? 0 : (br0 + j) * T::kKBytes) + k_addr(sb, kc)));
        __builtin_amdgcn_sched_barrier(0);
        f32x16 sc[NBR];
#pragma unroll
        for (int j = 0; j < NBR; ++j) {
            sc[j] = f32x16{};
#pragma unroll
            for (int kc = 0; kc < KC; ++kc) sc[j] = mfma32(kf[j][kc], qf[j][kc], sc[j]);
        }
        bf16x8 pb[NBR][2];
        if constexpr (kFast) {
#pragma unroll
            for (int j = 0; j < NBR; ++j) {
                float lb;
                softmax_fast(sc[j], mask, lim, lo, pb[j][0], pb[j][1], lb);
                l[j] += lb;
            }
        } else {
#pragma unroll
            for (int j = 0; j < NBR; ++j)
                softmax_branch(sc[j], mask, lim, lo, m[j], l[j], le[j], o[j], pb[j][0], pb[j][1]);
        }
        // O^T += V^T P^T, one V read for every branch of the wave. Step i
        // covers (k step t, dv block dc). With one branch per wave the k step
        // is the outer index, so the 4 accumulators of a k step are updated
        // back to back and dependent products sit 4 apart; with two branches
        // the dv block is outer (the two branches' products already alternate).
        constexpr bool kStepOuter = NBR == 1;
        auto t_of = [](int i) DA_INLINE { return kStepOuter ? (i >> 2) : (i & 1); };
        auto dc_of = [](int i) DA_INLINE { return kStepOuter ? (i & 3) : (i >> 1); };
        auto vfrag = [&](int i) DA_INLINE {
            const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(vt + v_addr(sb, t_of(i), dc_of(i), 0)));
            const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(vt + v_addr(sb, t_of(i), dc_of(i), 1)));
            return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        };
        // every value fragment of the sub-block is read before the first
        // product (the transposing reads overlap each other)
        bf16x8 vf[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) vf[i] = vfrag(i);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int j = 0; j < NBR; ++j) o[j][dc_of(i)] = mfma32(vf[i], pb[j][t_of(i)], o[j][dc_of(i)]);
    };

    // ---- the key sweep: even tiles in stage 0, odd tiles in stage 1
    auto tile_body = [&](auto ft, const unsigned char *base, int t) DA_INLINE {
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
            const int j = 2 * t + sb;
            if (j < jlo || j >= nsub) continue;  // wholly outside every row's window / past the diagonal
            if (j < nsub - 1 && j >= jmask) {
                step(ft, base, sb, false, 0, 0);
            } else {
                // diagonal / ragged-end sub-block (keys >= lim masked) and
                // window-start sub-blocks (keys < lo masked), relative to key0
                const int key0 = j * 32 + 8 * hh;
                const int lim = (p.causal ? min(myrow + 1, p.N) : p.N) - key0;
                const int lo = WIN ? myrow - win + 1 - key0 : INT_MIN / 2;
                step(ft, base, sb, true, lim, lo);
            }
        }
    };
    // The branch-split sweep (and the two-branch sweep without a window) runs in up
    // to three phases, each its own loop: the general
    // body (all masks) for the tiles holding window-start sub-blocks (the
    // first 4 tiles, windowed kernels only), the open body (no mask code at
    // all) through the middle, and the general body again for the last
    // kBM / 64 tiles, which hold every wave's diagonal sub-block and the
    // ragged end of the keys. A mask test inside one loop would let the
    // compiler merge the two variants of a step and evaluate the mask for
    // every sub-block. Phase boundaries sit at even tile offsets from tlo, so
    // each phase starts in stage 0 with its first tile already issued.
    auto tile_body_open = [&](auto ft, const unsigned char *base, int t) DA_INLINE {
#pragma unroll
        for (int sb = 0; sb < 2; ++sb)
            if (2 * t + sb < nsub - 1) step(ft, base, sb, false, 0, 0);
    };
    auto phase = [&](auto ft, auto body, int t0, int t1) DA_INLINE {
        for (int t = t0; t < t1; t += 2) {
            wait_vmem_all();
            __syncthreads();  // tile t visible to all waves; tile t-1 no longer read
            if (t + 1 < ntiles) issue_tile(t + 1, st1);
            body(ft, st0, t);
            if (t + 1 >= t1) break;  // only the last phase can end on an odd offset
            wait_vmem_all();
            __syncthreads();  // tile t+1 visible to all waves; tile t no longer read
            if (t + 2 < ntiles) issue_tile(t + 2, st0);
            body(ft, st1, t + 1);
        }
    };
    auto sweep = [&](auto ft) DA_INLINE {
        if (tlo < ntiles) issue_tile(tlo, st0);
        if constexpr (S::kOn || !WIN) {
            constexpr int kTail = S::kBM / kBN;  // tiles holding the waves' diagonal sub-blocks
            const int ta = WIN ? min(ntiles, tlo + 4) : tlo;
            const int tb = max(ta, tlo + 2 * ((ntiles - kTail - tlo) / 2));
            if (WIN) phase(ft, tile_body, tlo, ta);
            phase(ft, tile_body_open, ta, tb);
            phase(ft, tile_body, tb, ntiles);
        } else {
            // the windowed two-branch kernels run one phase: there the second copy
            // of the step that separate phases need costs more (register spills:
            // 12-15 % slower) than the guarded mask branch it saves; without a
            // window the phases gain 2 % (longctx_v1)
            phase(ft, tile_body, tlo, ntiles);
        }
    };
    // The fixed-reference sweep first (when the queries are pre-scaled), then,
    // if any row of the work-group left its range, the exact sweep from the
    // start. The decision is the work-group's (one flag in LDS), so every wave
    // runs the same barriers.
    bool exact = true;
    if (fast) {
        sweep(std::true_type{});
        bool bad = false;
#pragma unroll
        for (int j = 0; j < NBR; ++j) {
            const float ls = halves_sum(l[j]);
            bad = bad || !(ls >= kFastMinSum && ls <= kFastMaxSum);
#pragma unroll
            for (int dc = 0; dc < 4; ++dc)
#pragma unroll
                for (int r = 0; r < 16; ++r) bad = bad || !__builtin_isfinite(o[j][dc][r]);
        }
        bad = bad && myrow < p.N;
        if (__any(bad) && lane == 0) redo_flag = 1;
        __syncthreads();  // every wave has left the sweep and set its flag
        exact = redo_flag != 0;
        if (exact) {
#pragma unroll
            for (int j = 0; j < NBR; ++j) {
#pragma unroll
                for (int dc = 0; dc < 4; ++dc) o[j][dc] = f32x16{};
                m[j] = -INFINITY;
                l[j] = 0.0f;
                le[j] = 0.0f;
            }
            load_q();  // the exact sweep takes the exact queries
            scl = p.sc_log2;
        } else {
#pragma unroll
            for (int j = 0; j < NBR; ++j) m[j] = 0.0f;  // the reference the sums were taken against
        }
    }
    if (exact) sweep(std::false_type{});

    // ---- epilogue: y = O1 / l1 - lambda O2 / l2 (then the V1 norm), bf16 store
#pragma unroll
    for (int j = 0; j < NBR; ++j) {
        l[j] = halves_sum(l[j]);
        if constexpr (STATS) le[j] = halves_sum(le[j]);
    }
    // statistics for the backward pass: each branch's normalised output and
    // natural-log log-sum-exp of its scaled scores (m is in log2 units)
    if (STATS && myrow < p.N) {
        const int64_t rowid = ((int64_t)b * p.H + h) * p.N + myrow;
#pragma unroll
        for (int j = 0; j < NBR; ++j) {
            const int brj = br0 + j;
            float *ob = (brj ? p.o2 : p.o1) + rowid * kDV + 4 * hh;
            const float rl = 1.0f / l[j];
#pragma unroll
            for (int dc = 0; dc < 4; ++dc)
#pragma unroll
                for (int rq = 0; rq < 4; ++rq) {
                    const float4 v4 = {o[j][dc][4 * rq] * rl, o[j][dc][4 * rq + 1] * rl, o[j][dc][4 * rq + 2] * rl,
                                       o[j][dc][4 * rq + 3] * rl};
                    *(float4 *)(ob + 32 * dc + 8 * rq) = v4;
                }
            if (hh == 0) (brj ? p.lse2 : p.lse1)[rowid] = (m[j] + log2f(le[j])) * 0.69314718055994531f;
        }
    }
    f32x16 y[4];
    if constexpr (S::kOn) {
        // branch-2 waves hand lambda O2 / l2 to their branch-1 partner through LDS
        __syncthreads();  // every wave is done with the key tiles
        // a row group's 64 x 64 values, stored float4 by float4 with the 64 lanes'
        // float4s of one (dc, q) contiguous, so every access is conflict-free
        float *xch = (float *)(rg < 2 ? st0 : st1) + (rg & 1) * 64 * 64 + 4 * lane;
        if (br0) {
            const float r2 = p.lambda[h] / l[0];
#pragma unroll
            for (int dc = 0; dc < 4; ++dc) {
                const f32x16 w = o[0][dc] * r2;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const float4 v4 = {w[4 * q], w[4 * q + 1], w[4 * q + 2], w[4 * q + 3]};
                    *(float4 *)(xch + 256 * (4 * dc + q)) = v4;
                }
            }
        }
        __syncthreads();
        if (br0) return;
        const float r1 = 1.0f / l[0];
#pragma unroll
        for (int dc = 0; dc < 4; ++dc) {
            // both products rounded separately (no fused multiply-add), so identical
            // branches with lambda = 1 give exactly zero
#pragma clang fp contract(off)
            f32x16 w2;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float4 v4 = *(const float4 *)(xch + 256 * (4 * dc + q));
                w2[4 * q] = v4.x;
                w2[4 * q + 1] = v4.y;
                w2[4 * q + 2] = v4.z;
                w2[4 * q + 3] = v4.w;
            }
            y[dc] = o[0][dc] * r1 - w2;
        }
    } else {
        const float r1 = 1.0f / l[0];
        const float r2 = p.lambda[h] / l[NBR - 1];
#pragma unroll
        for (int dc = 0; dc < 4; ++dc) {
#pragma clang fp contract(off)
            y[dc] = o[0][dc] * r1 - o[NBR - 1][dc] * r2;
        }
    }
    if constexpr (NORM) {
        if (p.group_norm) {
            float sm = 0.0f;
#pragma unroll
            for (int dc = 0; dc < 4; ++dc)
#pragma unroll
                for (int r = 0; r < 16; ++r) sm += y[dc][r];
            const float mu = halves_sum(sm) * (1.0f / kDV);
#pragma unroll
            for (int dc = 0; dc < 4; ++dc)
#pragma unroll
                for (int r = 0; r < 16; ++r) y[dc][r] -= mu;
        }
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

template <int DQK, bool SHARED_K, bool NORM, bool STATS>
hipError_t launch_s(const Bf16Params &p, int blocks, hipStream_t stream) {
    if (p.window > 0)
        hipLaunchKernelGGL((prefill_bf16_kernel<DQK, SHARED_K, NORM, true, STATS>), dim3(blocks),
                           dim3(Split<DQK>::kThreads), 0, stream, p);
    else
        hipLaunchKernelGGL((prefill_bf16_kernel<DQK, SHARED_K, NORM, false, STATS>), dim3(blocks),
                           dim3(Split<DQK>::kThreads), 0, stream, p);
    return hipGetLastError();
}

template <int DQK, bool SHARED_K, bool NORM>
hipError_t launch_t(const Bf16Params &p, int blocks, hipStream_t stream) {
    return p.o1 ? launch_s<DQK, SHARED_K, NORM, true>(p, blocks, stream)
                : launch_s<DQK, SHARED_K, NORM, false>(p, blocks, stream);
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
    p.o1 = a.o1;
    p.o2 = a.o2;
    p.lse1 = a.lse1;
    p.lse2 = a.lse2;
    p.B = a.B;
    p.H = a.H;
    p.H_kv = a.H_kv;
    p.group = a.H / a.H_kv;
    p.N = a.N;
    p.causal = a.causal;
    p.window = a.window;
    const int bm = a.d_qk == 64 ? Split<64>::kBM : Split<128>::kBM;
    p.row_blocks = (a.N + bm - 1) / bm;
    const int kv_units = a.B * a.H_kv;
    p.xcd_units = (kv_units % 8 == 0) ? kv_units / 8 : 0;
    p.sc_log2 = scale * kLog2e;
    p.eps = a.eps;
    p.one_minus_init = 1.0f - lambda_init;
    const int64_t blocks = (int64_t)a.B * a.H * p.row_blocks;
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    const bool shared = a.k1 == a.k2 && a.sk1[0] == a.sk2[0] && a.sk1[1] == a.sk2[1] && a.sk1[2] == a.sk2[2];
    const bool norm = a.norm != DIFFATTN_NORM_NONE;
    p.group_norm = a.norm == DIFFATTN_NORM_GROUP;
    {
        // bytes from a slice's first row to the end of its last: the buffer
        // offsets (scalar tile offset + per-lane offset) stay below 2^31
        const int64_t n1 = std::max<int64_t>(a.N - 1, 63);
        int64_t most = a.sv[2] * n1 + a.d_v;
        most = std::max(most, a.sk1[2] * n1 + a.d_qk);
        most = std::max(most, a.sk2[2] * n1 + a.d_qk);
        p.off32 = 2 * most <= INT32_MAX && a.sk1[2] == a.sk2[2];
    }
    const int nb = (int)blocks;
    if (a.d_qk == 64) {
        if (shared) return norm ? launch_t<64, true, true>(p, nb, stream) : launch_t<64, true, false>(p, nb, stream);
        return norm ? launch_t<64, false, true>(p, nb, stream) : launch_t<64, false, false>(p, nb, stream);
    }
    if (shared) return norm ? launch_t<128, true, true>(p, nb, stream) : launch_t<128, true, false>(p, nb, stream);
    return norm ? launch_t<128, false, true>(p, nb, stream) : launch_t<128, false, false>(p, nb, stream);
}

}  // namespace da
