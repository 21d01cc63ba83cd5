// backward.hip -- gradients of the differential-attention prefill, bf16
// inputs, fp32 accumulation and gradients, bf16 MFMA on gfx950.
//
// The pages define the forward only (lesson "Differential Attention V2",
// section "Concept": the two maps A_k = softmax(Q_k K_k^T scale), the output
// (A_1 - lambda A_2) V; section "V1 vs V2": the V1 RMSNorm; lesson
// "Attention Variants": the causal mask and the sliding window). The
// gradients follow by the chain rule:
//   V1:  dy = c r (gamma dz) - y r^3 / d_v sum(c gamma dz y),
//        dgamma = sum_rows c dz y r        (r = 1/sqrt(mean(y^2) + eps), c = 1 - lambda_init)
//   dlambda = -sum(dy o_2),  dO_1 = dy,  dO_2 = -lambda dy   (o_k = O_k / l_k)
//   dV  = sum_q (P_1 - lambda P_2)^T dy                 one product for both branches
//   G   = dy V^T                                        shared by both branches
//   dS_k = w_k P_k (G - rowsum(dy o_k)),  w_1 = 1, w_2 = -lambda
//   dQ_k = scale dS_k K_k,  dK_k = scale dS_k^T Q_k
// with P_k = exp(S_k - lse_k) recomputed from the statistics the forward
// stored (each branch's normalised output o_k and log-sum-exp lse_k).
//
// Kernels:
//  bwd_prep_kernel      one wave per row: dy (stored bf16, the MFMA operand),
//                       rowsum(dy o_k) from the rounded dy, and per block of
//                       64 rows the partial sums of dlambda and dgamma
//  bwd_dq_kernel        query-major, like the forward: a work-group owns 128
//                       rows of one head (the heads of one KV group on one
//                       XCD), 4 waves of 32 rows, both branches per wave
//                       (one wave per SIMD); per 32-key sub-block
//                       S_k^T = K_k Q_k^T, G^T = V dy^T once for both
//                       branches, dS_k^T, dQ_k^T += K_k^T dS_k^T (K^T by
//                       transposing LDS reads; shared keys read once)
//  bwd_dkdv_kernel      key-major: a work-group owns 128 keys of one KV head
//                       (causal, no window: two mirrored blocks of 128 keys,
//                       one after the other, so every work-group does about
//                       the same work), 4 waves x 32 keys, both branches per
//                       wave, and sweeps the query tiles of every head of
//                       the group: S = Q K^T,
//                       G = dy V^T, dV^T += dy^T (P_1 - lambda P_2),
//                       dK^T += Q^T dS (Q^T and dy^T by transposing reads)
//  bwd_finalize_kernel  sums the partials per head (fixed order: deterministic)
// Masks as the forward: causal j <= i, window j >= i - W + 1, rows and keys
// past N. Tiles have the forward's LDS shapes, with the swizzles that keep
// both row and transposed reads free of bank conflicts (tiles.hpp), since
// every backward tile is read both ways.
#include "launch.hpp"
#include "tiles.hpp"

#include <climits>

namespace da {

namespace {

constexpr int kBM = 128;  // query rows per dQ work-group
constexpr int kWM = 32;   // rows (dQ) or keys (dK/dV) per wave
constexpr int kKB = 128;  // keys per dK/dV work-group

struct BwdParams {
    const __bf16 *q1, *q2, *k1, *k2, *v, *dout;
    int64_t sq1[3], sq2[3], sk1[3], sk2[3], sv[3], sdo[3];
    const float *lambda, *gamma, *o1, *o2, *lse1, *lse2;
    float *dq1, *dq2, *dk1, *dk2, *dv, *dlambda, *dgamma;
    __bf16 *dy;        // workspace: output gradient after the norm, [B, H, N, 128]
    float *dt1, *dt2;  // workspace: rowsum(dy * o_1) and sign(lambda) rowsum(dy * o_2), [B, H, N]
    float *ls1, *ls2;  // workspace: lse_1 log2(e) and lse_2 log2(e) - log2|lambda|, [B, H, N]
    float *part;       // workspace: per prep block [dlambda, dgamma[128]]
    int B, H, H_kv, group, N, causal, window, norm, prep_nblk, row_blocks, key_blocks;
    int xcd_units;  // dQ grid: B * H_kv / 8 when B * H_kv is a multiple of 8, else 0
    int qoff32;  // Q1 and Q2 share their strides and one batch of each spans fewer than 2^31 bytes
    int koff32;  // K1 and K2 share their row stride and each (batch, KV head) slice of K1, K2, V spans < 2^31 bytes
    float scale, sc_log2, eps, one_minus_init;
};

// ---------------------------------------------------------------- prep

// Sums over the 64 lanes of a wave of K independent values at once (the
// cross-lane steps of the K sums interleave).
template <int K>
__device__ __forceinline__ void wave_sums(float (&x)[K]) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1)
#pragma unroll
        for (int k = 0; k < K; ++k) x[k] += __shfl_xor(x[k], o, 64);
}

__global__ __launch_bounds__(256) void bwd_prep_kernel(BwdParams p) {
    // a block of kBwdPrepRows rows of one (batch, head): each wave takes every
    // 4th row, lane l channels 2l and 2l + 1; the block's dlambda and dgamma
    // sums go to one partial record
    __shared__ float red[4][kDV + 1];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int blk = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int c0 = 2 * lane;
    const float lam = p.lambda[h];
    const float c = p.one_minus_init;
    float gm0 = 0.0f, gm1 = 0.0f;
    if (p.norm) {
        // two scalar loads: gamma is only required to be 4-byte aligned
        gm0 = c * p.gamma[(int64_t)h * kDV + c0];
        gm1 = c * p.gamma[(int64_t)h * kDV + c0 + 1];
    }
    float dl = 0.0f, pg0 = 0.0f, pg1 = 0.0f;
    const int iend = min(p.N, (blk + 1) * kBwdPrepRows);
    for (int i = blk * kBwdPrepRows + wave; i < iend; i += 4) {
        const int64_t rowid = ((int64_t)b * p.H + h) * p.N + i;
        const float2 av = *(const float2 *)(p.o1 + rowid * kDV + c0);
        const float2 ev = *(const float2 *)(p.o2 + rowid * kDV + c0);
        const bf16x2 zv = *(const bf16x2 *)(p.dout + b * p.sdo[0] + h * p.sdo[1] + (int64_t)i * p.sdo[2] + c0);
        const float a0 = av.x, a1 = av.y, e0 = ev.x, e1 = ev.y;
        const float z0 = (float)zv[0], z1 = (float)zv[1];
        float y0, y1;
        {
#pragma clang fp contract(off)
            y0 = a0 - lam * e0;
            y1 = a1 - lam * e1;
        }
        float d0 = z0, d1 = z1;
        if (p.norm) {
            // RMS: z = y r gamma c; GroupNorm: z = u r gamma c with u = y - mean(y)
            // (r from the mean square of y, resp. u); with gd = c gamma dz:
            //   RMS:   dy = r gd - y r^3 mean(gd y)
            //   group: dy = r (gd - mean(gd)) - u r^3 mean(gd u)
            float g0 = gm0 * z0, g1 = gm1 * z1;
            if (p.norm == 2) {
                float m[2] = {y0 + y1, g0 + g1};
                wave_sums(m);
                const float mu = m[0] * (1.0f / kDV), gmean = m[1] * (1.0f / kDV);
                y0 -= mu;
                y1 -= mu;
                float q[2] = {y0 * y0 + y1 * y1, g0 * y0 + g1 * y1};
                wave_sums(q);
                const float r = 1.0f / sqrtf(q[0] * (1.0f / kDV) + p.eps);
                const float k3 = r * r * r * (1.0f / kDV) * q[1];
                d0 = r * (g0 - gmean) - y0 * k3;
                d1 = r * (g1 - gmean) - y1 * k3;
                pg0 += z0 * y0 * r * c;
                pg1 += z1 * y1 * r * c;
            } else {
                float q[2] = {y0 * y0 + y1 * y1, g0 * y0 + g1 * y1};
                wave_sums(q);
                const float r = 1.0f / sqrtf(q[0] * (1.0f / kDV) + p.eps);
                const float k3 = r * r * r * (1.0f / kDV) * q[1];
                d0 = r * g0 - y0 * k3;
                d1 = r * g1 - y1 * k3;
                pg0 += z0 * y0 * r * c;
                pg1 += z1 * y1 * r * c;
            }
        }
        const bf16x2 bd = pack2(d0, d1);
        *(bf16x2 *)(p.dy + rowid * kDV + c0) = bd;
        // the softmax-backward row sums use the rounded dy the products use
        const float f0 = (float)bd[0], f1 = (float)bd[1];
        float t[3] = {d0 * e0 + d1 * e1, f0 * a0 + f1 * a1, f0 * e0 + f1 * e1};
        wave_sums(t);
        dl -= t[0];
        // per row, for the score-gradient kernels: the log-sum-exp in log2
        // units, with |lambda| folded into branch 2's (2^(s - ls2) = |lambda| P_2;
        // lambda = 0 gives 2^-inf = 0), and branch 2's row sum times sign(lambda)
        if (lane == 0) {
            p.dt1[rowid] = t[1];
            p.dt2[rowid] = lam > 0.0f ? t[2] : (lam < 0.0f ? -t[2] : 0.0f);
            p.ls1[rowid] = p.lse1[rowid] * kLog2e;
            p.ls2[rowid] = p.lse2[rowid] * kLog2e - log2f(fabsf(lam));
        }
    }
    red[wave][c0] = pg0;
    red[wave][c0 + 1] = pg1;
    if (lane == 0) red[wave][kDV] = dl;
    __syncthreads();
    float *pp = p.part + (((int64_t)b * p.H + h) * p.prep_nblk + blk) * (kDV + 1);
    for (int k = threadIdx.x; k <= kDV; k += 256) {
        const float s = (red[0][k] + red[1][k]) + (red[2][k] + red[3][k]);
        pp[k == kDV ? 0 : 1 + k] = s;
    }
}

__global__ __launch_bounds__(512) void bwd_finalize_kernel(BwdParams p) {
    // per head: the partial records summed in a fixed order (deterministic).
    // Wave w sums its contiguous share of the records, in record order, lane
    // l holding values l and 64 + l of each record (value 128 in lane 0;
    // value 0 is dlambda, value t > 0 dgamma[t - 1]); the 8 wave sums are
    // then added in wave order.
    __shared__ float red[8][kDV + 1];
    const int h = blockIdx.x, wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t n = (int64_t)p.B * p.prep_nblk;
    const int64_t r0 = n * wave / 8, r1 = n * (wave + 1) / 8;
    float a0 = 0.0f, a1 = 0.0f, a2 = 0.0f;
#pragma unroll 4
    for (int64_t r = r0; r < r1; ++r) {
        const int64_t bb = r / p.prep_nblk, kb = r - bb * p.prep_nblk;
        const float *rec = p.part + (((int64_t)bb * p.H + h) * p.prep_nblk + kb) * (kDV + 1);
        a0 += rec[lane];
        a1 += rec[64 + lane];
        if (lane == 0) a2 += rec[kDV];
    }
    red[wave][lane] = a0;
    red[wave][64 + lane] = a1;
    if (lane == 0) red[wave][kDV] = a2;
    __syncthreads();
    const int t = threadIdx.x;
    if (t > kDV) return;
    float s = red[0][t];
#pragma unroll
    for (int w = 1; w < 8; ++w) s += red[w][t];
    if (t == 0)
        p.dlambda[h] = s;
    else if (p.norm)
        p.dgamma[(int64_t)h * kDV + t - 1] = s;
}

// ---------------------------------------------------------------- dQ

template <int DQK, bool SHARED_K, bool WIN>
__global__ __launch_bounds__(256, 1) void bwd_dq_kernel(BwdParams p) {
    using T = Tile<DQK, SHARED_K>;
    constexpr int KC = DQK / 16;
    constexpr int NW = 4;
    __shared__ __attribute__((aligned(1024))) unsigned char st0[T::kStage];
    __shared__ __attribute__((aligned(1024))) unsigned char st1[T::kStage];

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int l32 = lane & 31, hh = lane >> 5;
    const int rg = wave;  // row group: both branches of 32 rows in one wave

    const int U = p.B * p.H;
    int rank, u;
    if (p.xcd_units) {
        // work-groups go round-robin over the 8 XCDs: XCD L % 8 takes the
        // xcd_units KV units L % 8, L % 8 + 8, ..., each with every head of
        // its group, so the work-groups on one XCD stream the key/value
        // tiles of few KV heads and its L2 serves them
        const int L = blockIdx.x, xcd = L & 7, sidx = L >> 3;
        const int per = p.xcd_units * p.group;
        rank = sidx / per;
        const int rest = sidx - rank * per;
        const int kvu = (rest / p.group) * 8 + xcd;
        const int hig = rest - (rest / p.group) * p.group;
        const int bb = kvu / p.H_kv, gg = kvu - bb * p.H_kv;
        u = bb * p.H + gg * p.group + hig;
    } else {
        rank = blockIdx.x / U;
        u = blockIdx.x - rank * U;
    }
    const int b = u / p.H, h = u - b * p.H;
    const int rb = p.causal ? p.row_blocks - 1 - rank : rank;  // longest rows first
    const int g = h / p.group;
    const int q0 = rb * kBM;
    const int wrow0 = q0 + rg * kWM;
    const int myrow = wrow0 + l32;
    const int row = min(myrow, p.N - 1);  // rows past the end compute garbage, never stored
    const int64_t rowid = ((int64_t)b * p.H + h) * p.N + row;

    // B operands: both branches of Q, and dy, for the lane's row
    bf16x8 qf[2][KC], df[8];
    {
        const __bf16 *q1 = p.q1 + b * p.sq1[0] + h * p.sq1[1] + (int64_t)row * p.sq1[2];
        const __bf16 *q2 = p.q2 + b * p.sq2[0] + h * p.sq2[1] + (int64_t)row * p.sq2[2];
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) {
            qf[0][kc] = as_bf16x8(ldg16(q1 + 8 * hh + 16 * kc));
            qf[1][kc] = as_bf16x8(ldg16(q2 + 8 * hh + 16 * kc));
        }
        const __bf16 *d = p.dy + rowid * kDV;
#pragma unroll
        for (int kc = 0; kc < 8; ++kc) df[kc] = as_bf16x8(ldg16(d + 8 * hh + 16 * kc));
    }
    // dS_1 = P_1 (G - D_1) and dS_2 = -lambda P_2 (G - D_2), with G = dy V^T
    // formed once for both branches. With the prep kernel's per-row values
    // (log2 units: ls1, and ls2 with |lambda| folded, so 2^(s_2 - ls2) =
    // |lambda| P_2; dt2 = sign(lambda) D_2) the second is
    // 2^(s_2 - ls2) (sg G + dt2) with sg = -sign(lambda), as in the dK/dV kernel
    const float lamh = p.lambda[h];
    const float sg = lamh > 0.0f ? -1.0f : (lamh < 0.0f ? 1.0f : 0.0f);
    const float ls1 = p.ls1[rowid], ls2 = p.ls2[rowid];
    const float dt1 = p.dt1[rowid], dt2 = p.dt2[rowid];

    const __bf16 *kb1 = p.k1 + b * p.sk1[0] + g * p.sk1[1];
    const __bf16 *kb2 = p.k2 + b * p.sk2[0] + g * p.sk2[1];
    const __bf16 *vb = p.v + b * p.sv[0] + g * p.sv[1];
    const int64_t sk1n = p.sk1[2], sk2n = p.sk2[2], svn = p.sv[2];

    const int kend = p.causal ? min(p.N, q0 + kBM) : p.N;
    const int ntiles = (kend + kBN - 1) / kBN;
    const int win = WIN ? p.window : 0;
    const int tlo = WIN ? max(0, q0 - win + 1) / kBN : 0;
    const int jlo = WIN ? max(0, wrow0 - win + 1) / 32 : 0;
    const int jmask = WIN ? (max(0, wrow0 + kWM - win) + 31) / 32 : 0;
    const int wend = p.causal ? min(p.N, wrow0 + kWM) : p.N;
    const int nsub = wrow0 < p.N ? (wend + 31) / 32 : 0;

    static_assert(T::kBlocks % NW == 0, "stage blocks must divide among the waves");
    // With koff32, a tile wholly inside the sequence is copied by buffer
    // loads (descriptors over this (batch, KV head) slice, the tile's first
    // row times the stride as a scalar offset, one per-lane offset per tensor:
    // a wave's copies of one tensor are whole swizzle periods apart, and K1
    // and K2 share their strides); the last, partial tile and huge strides
    // take the general form.
    static_assert((T::kKBytes / 1024) % NW == 0, "copy i reads one tensor, fixed by i");
    constexpr int KPB = T::kKBytes / 1024 / NW;
    constexpr int KRows = NW * T::kRowsPerKBlock, VRows = NW * 4;
    static_assert(KRows % 16 == 0 && VRows % 16 == 0, "copy row steps must keep the swizzles");
    const int wv = wave_id();
    uint32_t koff, voff;
    {
        const int kr = wv * T::kRowsPerKBlock + lane / T::kKCh;
        koff = 2u * (uint32_t)(kr * sk1n + 8 * ((lane % T::kKCh) ^ bk_swz<DQK>(kr)));
        const int vr = wv * 4 + (lane >> 4);
        voff = 2u * (uint32_t)(vr * svn + 8 * ((lane & 15) ^ bv_swz(vr)));
    }
    const __amdgpu_buffer_rsrc_t rk1 = __builtin_amdgcn_make_buffer_rsrc((void *)kb1, (short)0, 0x7fffffff, 0x00020000);
    const __amdgpu_buffer_rsrc_t rk2 = __builtin_amdgcn_make_buffer_rsrc((void *)kb2, (short)0, 0x7fffffff, 0x00020000);
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc((void *)vb, (short)0, 0x7fffffff, 0x00020000);
    auto issue_tile = [&](int t, unsigned char *base) DA_INLINE {
        const int key0 = __builtin_amdgcn_readfirstlane(t * kBN);
        if (p.koff32 && key0 + kBN <= p.N) {
#pragma unroll
            for (int i = 0; i < T::kBlocks / NW; ++i) {
                const int blk = wv + NW * i;
                if (i < T::kNK * KPB) {
                    const int j = i % KPB;
                    const uint32_t so = 2u * (uint32_t)(key0 + j * KRows) * (uint32_t)sk1n;
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(i < KPB ? rk1 : rk2, (lds_void *)(base + blk * 1024), 16,
                                                             koff, so, 0, 0);
                } else {
                    const int j = i - T::kNK * KPB;
                    const uint32_t so = 2u * (uint32_t)(key0 + j * VRows) * (uint32_t)svn;
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void *)(base + blk * 1024), 16, voff, so, 0, 0);
                }
            }
            return;
        }
#pragma unroll
        for (int i = 0; i < T::kBlocks / NW; ++i) {
            const int blk = wave + NW * i;
            if (blk < T::kKBlocks) {
                const int kt = blk / (T::kKBytes / 1024);
                const int kblk = blk % (T::kKBytes / 1024);
                const int r = kblk * T::kRowsPerKBlock + lane / T::kKCh;
                const int col = 8 * ((lane % T::kKCh) ^ bk_swz<DQK>(r));
                const int key = min(key0 + r, p.N - 1);
                const __bf16 *src = (kt ? kb2 + (int64_t)key * sk2n : kb1 + (int64_t)key * sk1n) + col;
                __builtin_amdgcn_global_load_lds(src, (lds_void *)(base + blk * 1024), 16, 0, 0);
            } else {
                const int vblk = blk - T::kKBlocks;
                const int r = vblk * 4 + (lane >> 4);
                const int col = 8 * ((lane & 15) ^ bv_swz(r));
                const int key = min(key0 + r, p.N - 1);
                __builtin_amdgcn_global_load_lds(vb + (int64_t)key * svn + col, (lds_void *)(base + blk * 1024), 16,
                                                 0, 0);
            }
        }
    };

    f32x16 dq[2][DQK / 32];
#pragma unroll
    for (int dc = 0; dc < DQK / 32; ++dc) {
        dq[0][dc] = f32x16{};
        dq[1][dc] = f32x16{};
    }
    const int krow = perm_key(l32);

    auto step = [&](const unsigned char *base, int sb, bool mask, int lim, int lo) DA_INLINE {
        const unsigned char *kt1 = base;
        const unsigned char *kt2 = base + (SHARED_K ? 0 : T::kKBytes);
        const unsigned char *vt = base + T::kNK * T::kKBytes;
        const int r0 = 32 * sb + krow;
        // all key fragments (one set feeds both branches when the keys are
        // shared), then all value fragments, then each half's transposed key
        // fragments, read before the products that use them (the reads overlap
        // instead of each product waiting for its own)
        constexpr int NKT = SHARED_K ? 1 : 2;
        bf16x8 kf[NKT][KC];
#pragma unroll
        for (int j = 0; j < NKT; ++j)
#pragma unroll
            for (int kc = 0; kc < KC; ++kc)
                kf[j][kc] = as_bf16x8(
                    *(const uint4 *)((j ? kt2 : kt1) + r0 * (2 * DQK) + 16 * ((2 * kc + hh) ^ bk_swz<DQK>(r0))));
        __builtin_amdgcn_sched_barrier(0);
        f32x16 s1 = f32x16{}, s2 = f32x16{};
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) {
            s1 = mfma32(kf[0][kc], qf[0][kc], s1);
            s2 = mfma32(kf[NKT - 1][kc], qf[1][kc], s2);
        }
        f32x16 gq = f32x16{};
        bf16x8 vf[8];
#pragma unroll
        for (int kc = 0; kc < 8; ++kc) vf[kc] = as_bf16x8(*(const uint4 *)(vt + r0 * 256 + 16 * ((2 * kc + hh) ^ bv_swz(r0))));
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int kc = 0; kc < 8; ++kc) gq = mfma32(vf[kc], df[kc], gq);
        float p1[16], p2[16], d1[16], d2[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            p1[r] = exp2_fast(fmaf(s1[r], p.sc_log2, -ls1));
            p2[r] = exp2_fast(fmaf(s2[r], p.sc_log2, -ls2));
        }
        if (mask) {
            // an opaque statement keeps this a branch taken by the few masked
            // sub-blocks, instead of per-element selects evaluated for all
            asm volatile("");
#pragma unroll
            for (int r = 0; r < 16; ++r)
                if (key_of_reg(r) >= lim || key_of_reg(r) < lo) {
                    p1[r] = 0.0f;
                    p2[r] = 0.0f;
                }
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            d1[r] = p1[r] * (gq[r] - dt1);
            d2[r] = p2[r] * fmaf(sg, gq[r], dt2);
        }
        auto pack16 = [](const float *x, bf16x8 *out) DA_INLINE {
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const bf16x2 a = pack2(x[8 * t + 0], x[8 * t + 1]), c = pack2(x[8 * t + 2], x[8 * t + 3]);
                const bf16x2 e = pack2(x[8 * t + 4], x[8 * t + 5]), f = pack2(x[8 * t + 6], x[8 * t + 7]);
                out[t] = bf16x8{a[0], a[1], c[0], c[1], e[0], e[1], f[0], f[1]};
            }
        };
        bf16x8 pb1[2], pb2[2];
        pack16(d1, pb1);
        pack16(d2, pb2);
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            bf16x8 kq[NKT][DQK / 32];
#pragma unroll
            for (int j = 0; j < NKT; ++j)
#pragma unroll
                for (int dc = 0; dc < DQK / 32; ++dc)
                    kq[j][dc] = tr_frag(j ? kt2 : kt1, lane, 2 * DQK, BSwzK<DQK>(), sb, t, dc);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int dc = 0; dc < DQK / 32; ++dc) {
                dq[0][dc] = mfma32(kq[0][dc], pb1[t], dq[0][dc]);
                dq[1][dc] = mfma32(kq[NKT - 1][dc], pb2[t], dq[1][dc]);
            }
        }
    };

    auto tile_body = [&](const unsigned char *base, int t) DA_INLINE {
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
            const int j = 2 * t + sb;
            if (j < jlo || j >= nsub) continue;
            if (j < nsub - 1 && j >= jmask) {
                step(base, sb, false, 0, 0);
            } else {
                const int key0 = j * 32 + 8 * hh;
                const int lim = (p.causal ? min(myrow + 1, p.N) : p.N) - key0;
                const int lo = WIN ? myrow - win + 1 - key0 : INT_MIN / 2;
                step(base, sb, true, lim, lo);
            }
        }
    };
    if (tlo < ntiles) issue_tile(tlo, st0);
    for (int t = tlo; t < ntiles; t += 2) {
        wait_vmem_all();
        __syncthreads();
        if (t + 1 < ntiles) issue_tile(t + 1, st1);
        tile_body(st0, t);
        if (t + 1 >= ntiles) break;
        wait_vmem_all();
        __syncthreads();
        if (t + 2 < ntiles) issue_tile(t + 2, st0);
        tile_body(st1, t + 1);
    }

    if (myrow < p.N) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            float *o = (j ? p.dq2 : p.dq1) + (((int64_t)b * p.H + h) * p.N + myrow) * DQK + 4 * hh;
#pragma unroll
            for (int dc = 0; dc < DQK / 32; ++dc)
#pragma unroll
                for (int rq = 0; rq < 4; ++rq) {
                    const float4 v4 = {dq[j][dc][4 * rq] * p.scale, dq[j][dc][4 * rq + 1] * p.scale,
                                       dq[j][dc][4 * rq + 2] * p.scale, dq[j][dc][4 * rq + 3] * p.scale};
                    *(float4 *)(o + 32 * dc + 8 * rq) = v4;
                }
        }
    }
}

// ---------------------------------------------------------------- dK, dV

template <int DQK, bool SHARED_K, bool WIN>
__global__ __launch_bounds__(256, 1) void bwd_dkdv_kernel(BwdParams p) {
    constexpr int KC = DQK / 16;
    constexpr int NW = 4;
    constexpr int kQBytes = kBN * DQK * 2;      // one Q tile
    constexpr int kDBytes = kBN * kDV * 2;      // the dy tile
    constexpr int kSBytes = 4 * kBN * 4;        // statistics: lse_1, lse_2, dt_1, dt_2 of the tile's rows
    constexpr int kQBlocks = 2 * kQBytes / 1024;
    constexpr int kDBlocks = kDBytes / 1024;
    constexpr int kBlocks = kQBlocks + kDBlocks;  // 1 KB blocks (the statistics are loaded apart)
    constexpr int kStage = 2 * kQBytes + kDBytes + kSBytes;
    constexpr int kRowsPerQBlock = 1024 / (2 * DQK);
    constexpr int kQCh = DQK / 8;
    __shared__ __attribute__((aligned(1024))) unsigned char st0[kStage];
    __shared__ __attribute__((aligned(1024))) unsigned char st1[kStage];

    const int tid = threadIdx.x, wave = wave_id(), lane = tid & 63;
    const int l32 = lane & 31, hh = lane >> 5;

    const int U = p.B * p.H_kv;
    const int item = blockIdx.x / U, u = blockIdx.x - item * U;
    const int b = u / p.H_kv, g = u - b * p.H_kv;
    // Causal without a window: work-group `item` takes key block `item` (its
    // query tiles swept from the last down) and then the mirror block
    // key_blocks - 1 - item (swept from its first tile up). Every work-group
    // then sweeps about the same number of tiles, so a batch of work-groups
    // starts and ends together, and at any moment the work-groups of one XCD
    // read at most two tiles: (T steps in) tile T_last - T going down and
    // tile T going up, for all of them alike.
    const int npass = !WIN && p.causal && p.key_blocks - 1 - item != item ? 2 : 1;
#pragma unroll 1
    for (int pass = 0; pass < npass; ++pass) {
        const int kblk = pass ? p.key_blocks - 1 - item : item;
        const bool asc = pass == 1;
        if (pass) __syncthreads();  // every wave is done with the first block's stages
        const int k0 = kblk * kKB;
        const int kw0 = k0 + wave * kWM;
        const int mykey = kw0 + l32;
        const int key = min(mykey, p.N - 1);

        // B operands: the lane's key of K1, K2 and V
        bf16x8 kf1[KC], kf2[KC], vf[8];
        {
            const __bf16 *k1 = p.k1 + b * p.sk1[0] + g * p.sk1[1] + (int64_t)key * p.sk1[2];
            const __bf16 *k2 = p.k2 + b * p.sk2[0] + g * p.sk2[1] + (int64_t)key * p.sk2[2];
            const __bf16 *vv = p.v + b * p.sv[0] + g * p.sv[1] + (int64_t)key * p.sv[2];
#pragma unroll
            for (int kc = 0; kc < KC; ++kc) {
                kf1[kc] = as_bf16x8(ldg16(k1 + 8 * hh + 16 * kc));
                kf2[kc] = SHARED_K ? kf1[kc] : as_bf16x8(ldg16(k2 + 8 * hh + 16 * kc));
            }
#pragma unroll
            for (int kc = 0; kc < 8; ++kc) vf[kc] = as_bf16x8(ldg16(vv + 8 * hh + 16 * kc));
        }

        // query rows that see some key of the block: q >= k0 (causal) and, with
        // a window, q <= k0 + kKB - 1 + W - 1
        const int win = WIN ? p.window : 0;
        const int qlo = p.causal ? min(k0, p.N) : 0;
        const int qhi = WIN ? min(p.N, k0 + kKB - 1 + win) : p.N;
        const int tlo = qlo / kBN;
        const int nt = qhi > qlo ? (qhi + kBN - 1) / kBN - tlo : 0;  // query tiles per head
        const int total = nt * p.group;                                // (head, tile) pairs
        // step x visits query tile tlo + nt - 1 - x / group of head x % group:
        // tiles from the last down, every head of the group at each tile. The
        // work-groups running together on one XCD hold the same KV head's key
        // blocks (the KV unit is the fastest-varying part of the block index, so
        // with B * H_kv a multiple of 8 a unit's blocks all land on one XCD) and
        // all need the last tiles, so they read the same tiles at about the same
        // time and that XCD's L2 serves most of them
        auto tile_of = [&](int x, int &hg) DA_INLINE {
            const int tt = x / p.group;
            hg = x - tt * p.group;
            return asc ? tlo + tt : tlo + nt - 1 - tt;
        };

        // With qoff32, a tile wholly inside the sequence is copied by buffer
        // loads: one descriptor per tensor over this batch, the head and first
        // row (times the strides) as a scalar offset and one per-lane offset per
        // tensor; a wave's copies of one tensor are whole 16-row steps apart (the
        // swizzles' period), so Q1 and Q2 share one lane offset and dy has one.
        // The tile holding the end of the sequence (rows clamped) and huge
        // strides take the general form.
        static_assert((kQBytes / 1024) % NW == 0 && (kDBytes / 1024) % NW == 0, "copy i reads one tensor, fixed by i");
        constexpr int QPB = kQBytes / 1024 / NW;        // a wave's copies per Q tile
        constexpr int QRows = NW * kRowsPerQBlock;      // rows between them
        constexpr int DRows = NW * 4;                   // rows between a wave's dy copies
        static_assert(QRows % 16 == 0 && DRows % 16 == 0, "copy row steps must keep the swizzles");
        uint32_t qoff, doff;
        {
            const int qr = wave * kRowsPerQBlock + lane / kQCh;
            qoff = 2u * (uint32_t)(qr * p.sq1[2] + 8 * ((lane % kQCh) ^ bk_swz<DQK>(qr)));
            const int dr = wave * 4 + (lane >> 4);
            doff = 2u * (uint32_t)(dr * kDV + 8 * ((lane & 15) ^ bv_swz(dr)));
        }
        // raw buffer descriptors (stride 0, 32-bit data format: dword 3 = 0x00020000)
        const __amdgpu_buffer_rsrc_t rq1 =
            __builtin_amdgcn_make_buffer_rsrc((void *)(p.q1 + b * p.sq1[0]), (short)0, 0x7fffffff, 0x00020000);
        const __amdgpu_buffer_rsrc_t rq2 =
            __builtin_amdgcn_make_buffer_rsrc((void *)(p.q2 + b * p.sq2[0]), (short)0, 0x7fffffff, 0x00020000);
        const __amdgpu_buffer_rsrc_t rdy = __builtin_amdgcn_make_buffer_rsrc(
            (void *)(p.dy + (int64_t)b * p.H * p.N * kDV), (short)0, 0x7fffffff, 0x00020000);
        const float *stat_arr = wave == 0 ? p.ls1 : wave == 1 ? p.ls2 : wave == 2 ? p.dt1 : p.dt2;
        const __amdgpu_buffer_rsrc_t rst = __builtin_amdgcn_make_buffer_rsrc(
            (void *)(stat_arr + (int64_t)b * p.H * p.N), (short)0, 0x7fffffff, 0x00020000);

        auto issue_tile = [&](int x, unsigned char *base) DA_INLINE {
            int hg;
            const int t = tile_of(x, hg);
            const int h = g * p.group + hg;
            const int r0 = t * kBN;
            if (p.qoff32 && r0 + kBN <= p.N) {
                const int hs = __builtin_amdgcn_readfirstlane(h), rs = __builtin_amdgcn_readfirstlane(r0);
#pragma unroll
                for (int i = 0; i < kBlocks / NW; ++i) {
                    const int blk = wave + NW * i;
                    if (i < 2 * QPB) {
                        const int j = i % QPB;
                        const uint32_t so = 2u * (uint32_t)(hs * p.sq1[1] + (rs + j * QRows) * p.sq1[2]);
                        __builtin_amdgcn_raw_ptr_buffer_load_lds(i < QPB ? rq1 : rq2, (lds_void *)(base + blk * 1024),
                                                                 16, qoff, so, 0, 0);
                    } else {
                        const int j = i - 2 * QPB;
                        const uint32_t so = 2u * (uint32_t)((hs * p.N + rs + j * DRows) * kDV);
                        __builtin_amdgcn_raw_ptr_buffer_load_lds(rdy, (lds_void *)(base + blk * 1024), 16, doff, so,
                                                                 0, 0);
                    }
                }
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rst, (lds_void *)(base + kBlocks * 1024 + wave * 256), 4,
                                                         4u * (uint32_t)lane, 4u * (uint32_t)(hs * p.N + rs), 0, 0);
                return;
            }
            const __bf16 *qb1 = p.q1 + b * p.sq1[0] + h * p.sq1[1];
            const __bf16 *qb2 = p.q2 + b * p.sq2[0] + h * p.sq2[1];
            const __bf16 *db = p.dy + ((int64_t)b * p.H + h) * p.N * kDV;
            for (int blk = wave; blk < kBlocks; blk += NW) {
                if (blk < kQBlocks) {
                    const int qt = blk / (kQBytes / 1024);
                    const int qbk = blk % (kQBytes / 1024);
                    const int r = qbk * kRowsPerQBlock + lane / kQCh;
                    const int col = 8 * ((lane % kQCh) ^ bk_swz<DQK>(r));
                    const int q = min(r0 + r, p.N - 1);
                    const __bf16 *src = (qt ? qb2 + (int64_t)q * p.sq2[2] : qb1 + (int64_t)q * p.sq1[2]) + col;
                    __builtin_amdgcn_global_load_lds(src, (lds_void *)(base + blk * 1024), 16, 0, 0);
                } else {
                    const int dbk = blk - kQBlocks;
                    const int r = dbk * 4 + (lane >> 4);
                    const int col = 8 * ((lane & 15) ^ bv_swz(r));
                    const int q = min(r0 + r, p.N - 1);
                    __builtin_amdgcn_global_load_lds(db + (int64_t)q * kDV + col, (lds_void *)(base + blk * 1024),
                                                     16, 0, 0);
                }
            }
            // statistics: wave w loads array w (lse_1, lse_2, dt_1, dt_2), lane = row
            {
                const int q = min(r0 + lane, p.N - 1);
                const int64_t rid = ((int64_t)b * p.H + h) * p.N + q;
                const float *src = wave == 0 ? p.ls1 : wave == 1 ? p.ls2 : wave == 2 ? p.dt1 : p.dt2;
                __builtin_amdgcn_global_load_lds(src + rid, (lds_void *)(base + kBlocks * 1024 + wave * 256), 4, 0, 0);
            }
        };

        f32x16 dva[4], dk1a[DQK / 32], dk2a[DQK / 32];
#pragma unroll
        for (int dc = 0; dc < 4; ++dc) dva[dc] = f32x16{};
#pragma unroll
        for (int dc = 0; dc < DQK / 32; ++dc) {
            dk1a[dc] = f32x16{};
            dk2a[dc] = f32x16{};
        }
        const int qrow = perm_key(l32);

        // the transposed A operands of one 16-row half t of a sub-block: dy^T for
        // dV and Q1^T, Q2^T for dK, each 32 columns wide. Read in one batch ahead
        // of the products (one wave per SIMD: a read issued just before its
        // product would expose its whole latency to every product).
        constexpr int KD = DQK / 32;
        auto read_tr = [&](const unsigned char *base, int sb, int t, bf16x8 *fv, bf16x8 *fk1, bf16x8 *fk2) DA_INLINE {
            const unsigned char *t1 = base, *t2 = base + kQBytes, *td = base + 2 * kQBytes;
#pragma unroll
            for (int dc = 0; dc < 4; ++dc) fv[dc] = tr_frag(td, lane, 256, BSwzV(), sb, t, dc);
#pragma unroll
            for (int dc = 0; dc < KD; ++dc) {
                fk1[dc] = tr_frag(t1, lane, 2 * DQK, BSwzK<DQK>(), sb, t, dc);
                fk2[dc] = tr_frag(t2, lane, 2 * DQK, BSwzK<DQK>(), sb, t, dc);
            }
        };
        auto products = [&](bf16x8 wbt, bf16x8 s1t, bf16x8 s2t, const bf16x8 *fv, const bf16x8 *fk1,
                            const bf16x8 *fk2) DA_INLINE {
#pragma unroll
            for (int dc = 0; dc < 4; ++dc) dva[dc] = mfma32(fv[dc], wbt, dva[dc]);
#pragma unroll
            for (int dc = 0; dc < KD; ++dc) {
                dk1a[dc] = mfma32(fk1[dc], s1t, dk1a[dc]);
                if (SHARED_K)
                    dk1a[dc] = mfma32(fk2[dc], s2t, dk1a[dc]);
                else
                    dk2a[dc] = mfma32(fk2[dc], s2t, dk2a[dc]);
            }
        };

        // one 32-row query sub-block of the tile at `base` (query rows qb .. qb+31)
        // sg = -sign(lambda) of the head: with the prep kernel's folding,
        // P_2 |lambda| = 2^(s_2 - ls2), so the combined weight P_1 - lambda P_2 is
        // P_1 + sg 2^(s_2 - ls2) and dS_2 = -lambda P_2 (G - D_2) is
        // 2^(s_2 - ls2) (sg G + sign(lambda) D_2), the last term as stored
        auto step = [&](const unsigned char *base, int sb, int qb, float sg, bool mask) DA_INLINE {
            const unsigned char *t1 = base;
            const unsigned char *t2 = base + kQBytes;
            const unsigned char *td = base + 2 * kQBytes;
            const float *stat = (const float *)(base + 2 * kQBytes + kDBytes);
            const int r0 = 32 * sb + qrow;
            // the A operands of the three products are read in one batch ahead of
            // them: with one wave per SIMD nothing else hides an LDS read's latency,
            // so a read issued just before its product would stall every product
            bf16x8 a1[KC], a2[KC], ad[8];
#pragma unroll
            for (int kc = 0; kc < KC; ++kc) {
                const int off = r0 * (2 * DQK) + 16 * ((2 * kc + hh) ^ bk_swz<DQK>(r0));
                a1[kc] = as_bf16x8(*(const uint4 *)(t1 + off));
                a2[kc] = as_bf16x8(*(const uint4 *)(t2 + off));
            }
#pragma unroll
            for (int kc = 0; kc < 8; ++kc)
                ad[kc] = as_bf16x8(*(const uint4 *)(td + r0 * 256 + 16 * ((2 * kc + hh) ^ bv_swz(r0))));
            __builtin_amdgcn_sched_barrier(0);
            f32x16 s1 = f32x16{}, s2 = f32x16{}, gq = f32x16{};
#pragma unroll
            for (int kc = 0; kc < KC; ++kc) {
                s1 = mfma32(a1[kc], kf1[kc], s1);
                s2 = mfma32(a2[kc], kf2[kc], s2);
            }
#pragma unroll
            for (int kc = 0; kc < 8; ++kc) gq = mfma32(ad[kc], vf[kc], gq);
            if constexpr (DQK == 64) {
                // d_qk 64: each 16-row half t of the sub-block (registers 8t .. 8t+7)
                // is finished and its products issued before the next half's
                // arithmetic, so that arithmetic can run beside those products (4 %
                // faster on backward_v1; 2 % slower for d_qk 128, which keeps the
                // whole-sub-block form below)
                const float *statc = stat;
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    float p1[8], p2[8], D1[8], D2[8];
#pragma unroll
                    for (int r4 = 0; r4 < 2; ++r4) {
                        const int rr = 32 * sb + key_of_reg(8 * t + 4 * r4) + 8 * hh;  // 4 consecutive rows
                        const float4 l1 = *(const float4 *)(statc + rr);
                        const float4 l2 = *(const float4 *)(statc + 64 + rr);
                        const float4 t1v = *(const float4 *)(statc + 128 + rr);
                        const float4 t2v = *(const float4 *)(statc + 192 + rr);
                        const float L1[4] = {l1.x, l1.y, l1.z, l1.w}, L2[4] = {l2.x, l2.y, l2.z, l2.w};
                        const float T1[4] = {t1v.x, t1v.y, t1v.z, t1v.w}, T2[4] = {t2v.x, t2v.y, t2v.z, t2v.w};
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const int r = 4 * r4 + e;
                            p1[r] = exp2_fast(fmaf(s1[8 * t + r], p.sc_log2, -L1[e]));
                            p2[r] = exp2_fast(fmaf(s2[8 * t + r], p.sc_log2, -L2[e]));
                            D1[r] = T1[e];
                            D2[r] = T2[e];
                        }
                    }
                    if (mask) {
                        asm volatile("");
#pragma unroll
                        for (int r = 0; r < 8; ++r) {
                            const int q = qb + key_of_reg(8 * t + r) + 8 * hh;
                            const bool vis = q < p.N && (!p.causal || q >= mykey) && (!WIN || q - mykey < win);
                            if (!vis) {
                                p1[r] = 0.0f;
                                p2[r] = 0.0f;
                            }
                        }
                    }
                    float pw[8], d1[8], d2[8];
#pragma unroll
                    for (int r = 0; r < 8; ++r) {
                        const float gr = gq[8 * t + r];
                        pw[r] = fmaf(sg, p2[r], p1[r]);
                        d1[r] = p1[r] * (gr - D1[r]);
                        d2[r] = p2[r] * fmaf(sg, gr, D2[r]);
                    }
                    auto pack8f = [](const float *x) DA_INLINE {
                        const bf16x2 a = pack2(x[0], x[1]), c = pack2(x[2], x[3]);
                        const bf16x2 e = pack2(x[4], x[5]), f = pack2(x[6], x[7]);
                        return bf16x8{a[0], a[1], c[0], c[1], e[0], e[1], f[0], f[1]};
                    };
                    const bf16x8 wbt = pack8f(pw), s1t = pack8f(d1), s2t = pack8f(d2);
#pragma unroll
                    for (int dc = 0; dc < 4; ++dc)
                        dva[dc] = mfma32(tr_frag(td, lane, 256, BSwzV(), sb, t, dc), wbt, dva[dc]);
#pragma unroll
                    for (int dc = 0; dc < DQK / 32; ++dc) {
                        dk1a[dc] = mfma32(tr_frag(t1, lane, 2 * DQK, BSwzK<DQK>(), sb, t, dc), s1t, dk1a[dc]);
                        if (SHARED_K)
                            dk1a[dc] = mfma32(tr_frag(t2, lane, 2 * DQK, BSwzK<DQK>(), sb, t, dc), s2t, dk1a[dc]);
                        else
                            dk2a[dc] = mfma32(tr_frag(t2, lane, 2 * DQK, BSwzK<DQK>(), sb, t, dc), s2t, dk2a[dc]);
                    }
                }
            } else {
                // the first half's transposed operands are read now, under the
                // arithmetic below, and the second half's after it, all before the
                // products (backward_v2 7 % faster; the d_qk 64 form above keeps
                // its reads beside each product, where batching was 1.5 % slower)
                bf16x8 fv0[4], fk10[KD], fk20[KD];
                read_tr(base, sb, 0, fv0, fk10, fk20);
                __builtin_amdgcn_sched_barrier(0);
                // register r holds query row 32 sb + key_of_reg(r) + 8 hh of the tile
                float p1[16], p2[16], D1[16], D2[16];
#pragma unroll
                for (int r4 = 0; r4 < 4; ++r4) {
                    const int rr = 32 * sb + key_of_reg(4 * r4) + 8 * hh;  // 4 consecutive rows
                    const float4 l1 = *(const float4 *)(stat + rr);
                    const float4 l2 = *(const float4 *)(stat + 64 + rr);
                    const float4 t1v = *(const float4 *)(stat + 128 + rr);
                    const float4 t2v = *(const float4 *)(stat + 192 + rr);
                    const float L1[4] = {l1.x, l1.y, l1.z, l1.w}, L2[4] = {l2.x, l2.y, l2.z, l2.w};
                    const float T1[4] = {t1v.x, t1v.y, t1v.z, t1v.w}, T2[4] = {t2v.x, t2v.y, t2v.z, t2v.w};
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int r = 4 * r4 + e;
                        p1[r] = exp2_fast(fmaf(s1[r], p.sc_log2, -L1[e]));
                        p2[r] = exp2_fast(fmaf(s2[r], p.sc_log2, -L2[e]));
                        D1[r] = T1[e];
                        D2[r] = T2[e];
                    }
                }
                if (mask) {
                    // an opaque statement keeps this a branch taken by the few masked
                    // sub-blocks, instead of per-element selects evaluated for all
                    asm volatile("");
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int q = qb + key_of_reg(r) + 8 * hh;
                        const bool vis = q < p.N && (!p.causal || q >= mykey) && (!WIN || q - mykey < win);
                        if (!vis) {
                            p1[r] = 0.0f;
                            p2[r] = 0.0f;
                        }
                    }
                }
                float pw[16], d1[16], d2[16];
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    pw[r] = fmaf(sg, p2[r], p1[r]);
                    d1[r] = p1[r] * (gq[r] - D1[r]);
                    d2[r] = p2[r] * fmaf(sg, gq[r], D2[r]);
                }
                auto pack16 = [](const float *x, bf16x8 *out) DA_INLINE {
#pragma unroll
                    for (int t = 0; t < 2; ++t) {
                        const bf16x2 a = pack2(x[8 * t + 0], x[8 * t + 1]), c = pack2(x[8 * t + 2], x[8 * t + 3]);
                        const bf16x2 e = pack2(x[8 * t + 4], x[8 * t + 5]), f = pack2(x[8 * t + 6], x[8 * t + 7]);
                        out[t] = bf16x8{a[0], a[1], c[0], c[1], e[0], e[1], f[0], f[1]};
                    }
                };
                bf16x8 wb[2], s1b[2], s2b[2];
                pack16(pw, wb);
                pack16(d1, s1b);
                pack16(d2, s2b);
                bf16x8 fv1[4], fk11[KD], fk21[KD];
                read_tr(base, sb, 1, fv1, fk11, fk21);
                __builtin_amdgcn_sched_barrier(0);
                products(wb[0], s1b[0], s2b[0], fv0, fk10, fk20);
                products(wb[1], s1b[1], s2b[1], fv1, fk11, fk21);
            }
        };

        auto tile_body = [&](const unsigned char *base, int x) DA_INLINE {
            int hg;
            const int t = tile_of(x, hg);
            const float lamh = ld_uniform(p.lambda + g * p.group + hg);
            const float sg = lamh > 0.0f ? -1.0f : (lamh < 0.0f ? 1.0f : 0.0f);
#pragma unroll
            for (int sb = 0; sb < 2; ++sb) {
                const int qb = t * kBN + 32 * sb;  // first query row of the sub-block
                // wholly invisible to this wave's keys: skip
                if (qb >= p.N) continue;
                if (p.causal && qb + 31 < kw0) continue;
                if (WIN && qb > kw0 + kWM - 1 + win - 1) continue;
                const bool mask = qb + 31 >= p.N || (p.causal && qb < kw0 + kWM - 1) ||
                                  (WIN && qb + 31 > kw0 + win - 1);
                step(base, sb, qb, sg, mask);
            }
        };
        if constexpr (DQK == 128 && SHARED_K) {
            // Three phases, each its own loop: the general body (masks) for the tiles
            // at the ends of the sweep, and an open body (no mask code) for the tiles
            // every row of which every wave of the work-group sees in full: below the
            // ragged end, above the key block's diagonal (causal) and inside every
            // key's window. A mask test inside one loop splits the step into blocks
            // the scheduler cannot move work across. Phase boundaries sit at even
            // steps, so each phase starts in stage 0 with its first tile issued. (The
            // d_qk 64 kernels and the two-key d_qk 128 kernel run no faster this way,
            // and the latter spills: they keep one loop.)
            auto tile_body_open = [&](const unsigned char *base, int x) DA_INLINE {
                int hg;
                const int t = tile_of(x, hg);
                const float lamh = ld_uniform(p.lambda + g * p.group + hg);
                const float sg = lamh > 0.0f ? -1.0f : (lamh < 0.0f ? 1.0f : 0.0f);
#pragma unroll
                for (int sb = 0; sb < 2; ++sb) step(base, sb, t * kBN + 32 * sb, sg, false);
            };
            auto phase = [&](auto body, int x0, int x1) DA_INLINE {
                for (int x = x0; x < x1; x += 2) {
                    wait_vmem_all();
                    __syncthreads();
                    if (x + 1 < total) issue_tile(x + 1, st1);
                    body(st0, x);
                    if (x + 1 >= x1) break;  // only the last phase can end on an odd step
                    wait_vmem_all();
                    __syncthreads();
                    if (x + 2 < total) issue_tile(x + 2, st0);
                    body(st1, x + 1);
                }
            };
            // open tiles: t in [o_lo, o_hi]
            const int o_hi0 = p.N / kBN - 1;  // (rows past N: the ragged tile is general)
            const int o_hi = WIN ? min(o_hi0, (k0 + win) / kBN - 1) : o_hi0;
            const int o_lo = p.causal ? (k0 + kKB - 1 + kBN - 1) / kBN : tlo;
            const int t_top = tlo + nt - 1;
            int xa = asc ? max(0, (o_lo - tlo) * p.group) : max(0, (t_top - o_hi) * p.group);
            int xb = asc ? (o_hi - tlo + 1) * p.group : (t_top - o_lo + 1) * p.group;
            xa = min(total, (xa + 1) & ~1);
            xb = max(xa, min(total, xb) & ~1);
            if (o_lo > o_hi) xb = xa;
            if (total > 0) issue_tile(0, st0);
            phase(tile_body, 0, xa);
            phase(tile_body_open, xa, xb);
            phase(tile_body, xb, total);
        } else {
            if (total > 0) issue_tile(0, st0);
            for (int x = 0; x < total; x += 2) {
                wait_vmem_all();
                __syncthreads();
                if (x + 1 < total) issue_tile(x + 1, st1);
                tile_body(st0, x);
                if (x + 1 >= total) break;
                wait_vmem_all();
                __syncthreads();
                if (x + 2 < total) issue_tile(x + 2, st0);
                tile_body(st1, x + 1);
            }
        }

        if (mykey < p.N) {
            const int64_t kid = ((int64_t)b * p.H_kv + g) * p.N + mykey;
            float *ov = p.dv + kid * kDV + 4 * hh;
#pragma unroll
            for (int dc = 0; dc < 4; ++dc)
#pragma unroll
                for (int rq = 0; rq < 4; ++rq) {
                    const float4 v4 = {dva[dc][4 * rq], dva[dc][4 * rq + 1], dva[dc][4 * rq + 2], dva[dc][4 * rq + 3]};
                    *(float4 *)(ov + 32 * dc + 8 * rq) = v4;
                }
#pragma unroll
            for (int kk = 0; kk < (SHARED_K ? 1 : 2); ++kk) {
                float *ok = (kk ? p.dk2 : p.dk1) + kid * DQK + 4 * hh;
#pragma unroll
                for (int dc = 0; dc < DQK / 32; ++dc) {
                    const f32x16 a = kk ? dk2a[dc] : dk1a[dc];
#pragma unroll
                    for (int rq = 0; rq < 4; ++rq) {
                        const float4 v4 = {a[4 * rq] * p.scale, a[4 * rq + 1] * p.scale, a[4 * rq + 2] * p.scale,
                                           a[4 * rq + 3] * p.scale};
                        *(float4 *)(ok + 32 * dc + 8 * rq) = v4;
                    }
                }
            }
        }
    }
}

template <int DQK, bool SHARED_K, bool WIN>
hipError_t launch_main(const BwdParams &p, hipStream_t stream) {
    const int64_t dq_blocks = (int64_t)p.B * p.H * p.row_blocks;
    const int64_t kv_blocks = (int64_t)p.B * p.H_kv * (!WIN && p.causal ? (p.key_blocks + 1) / 2 : p.key_blocks);
    if (dq_blocks > 0x7fffffff || kv_blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((bwd_dq_kernel<DQK, SHARED_K, WIN>), dim3((int)dq_blocks), dim3(256), 0, stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((bwd_dkdv_kernel<DQK, SHARED_K, WIN>), dim3((int)kv_blocks), dim3(256), 0, stream, p);
    return hipGetLastError();
}

template <int DQK, bool SHARED_K>
hipError_t launch_w(const BwdParams &p, hipStream_t stream) {
    return p.window > 0 ? launch_main<DQK, SHARED_K, true>(p, stream) : launch_main<DQK, SHARED_K, false>(p, stream);
}

__global__ __launch_bounds__(256) void lambda_backward_kernel(const float *lq1, const float *lk1, const float *lq2,
                                                              const float *lk2, int d_l, const float *dlambda,
                                                              float *dlq1, float *dlk1, float *dlq2, float *dlk2) {
    // one work-group per head: the two dot products, then the four gradients
    __shared__ float red[2][4];
    const int h = blockIdx.x, tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int64_t o = (int64_t)h * d_l;
    float a = 0.0f, c = 0.0f;
    for (int k = tid; k < d_l; k += 256) {
        a = fmaf(lq1[o + k], lk1[o + k], a);
        c = fmaf(lq2[o + k], lk2[o + k], c);
    }
    a = wave_sum(a);
    c = wave_sum(c);
    if (lane == 0) {
        red[0][wave] = a;
        red[1][wave] = c;
    }
    __syncthreads();
    const float d = dlambda[h];
    const float e1 = d * expf((red[0][0] + red[0][1]) + (red[0][2] + red[0][3]));
    const float e2 = -d * expf((red[1][0] + red[1][1]) + (red[1][2] + red[1][3]));
    for (int k = tid; k < d_l; k += 256) {
        dlq1[o + k] = e1 * lk1[o + k];
        dlk1[o + k] = e1 * lq1[o + k];
        dlq2[o + k] = e2 * lk2[o + k];
        dlk2[o + k] = e2 * lq2[o + k];
    }
}

}  // namespace

hipError_t launch_backward_bf16(const diffattn_backward_args &a, const BackwardPlan &plan, void *workspace,
                                float scale, float lambda_init, hipStream_t stream) {
    BwdParams p;
    p.q1 = (const __bf16 *)a.q1;
    p.q2 = (const __bf16 *)a.q2;
    p.k1 = (const __bf16 *)a.k1;
    p.k2 = (const __bf16 *)a.k2;
    p.v = (const __bf16 *)a.v;
    p.dout = (const __bf16 *)a.dout;
    for (int k = 0; k < 3; ++k) {
        p.sq1[k] = a.sq1[k];
        p.sq2[k] = a.sq2[k];
        p.sk1[k] = a.sk1[k];
        p.sk2[k] = a.sk2[k];
        p.sv[k] = a.sv[k];
        p.sdo[k] = a.sdo[k];
    }
    p.lambda = a.lambda;
    p.gamma = a.gamma;
    p.o1 = a.o1;
    p.o2 = a.o2;
    p.lse1 = a.lse1;
    p.lse2 = a.lse2;
    p.dq1 = a.dq1;
    p.dq2 = a.dq2;
    p.dk1 = a.dk1;
    p.dk2 = plan.shared_k ? a.dk1 : a.dk2;
    p.dv = a.dv;
    p.dlambda = a.dlambda;
    p.dgamma = a.dgamma;
    unsigned char *ws = (unsigned char *)workspace;
    p.dy = (__bf16 *)(ws + plan.off_dy);
    p.dt1 = (float *)(ws + plan.off_dt1);
    p.dt2 = (float *)(ws + plan.off_dt2);
    p.ls1 = (float *)(ws + plan.off_ls1);
    p.ls2 = (float *)(ws + plan.off_ls2);
    p.part = (float *)(ws + plan.off_part);
    p.B = a.B;
    p.H = a.H;
    p.H_kv = a.H_kv;
    p.group = a.H / a.H_kv;
    p.N = a.N;
    p.causal = a.causal;
    p.window = a.window;
    p.norm = a.norm;  // 0 none, 1 RMS, 2 GroupNorm
    p.prep_nblk = (a.N + kBwdPrepRows - 1) / kBwdPrepRows;
    p.row_blocks = (a.N + kBM - 1) / kBM;
    p.key_blocks = (a.N + kKB - 1) / kKB;
    p.xcd_units = (a.B * a.H_kv) % 8 == 0 ? a.B * a.H_kv / 8 : 0;
    {
        // the buffer-load copies keep every offset inside one batch below 2^31
        // bytes: Q1 and Q2 (equal strides), dy (bf16, [H, N, 128]) and the
        // fp32 statistics ([H, N])
        const int64_t qmost = a.sq1[1] * (a.H - 1) + a.sq1[2] * (a.N - 1) + a.d_qk;
        const bool same = a.sq1[1] == a.sq2[1] && a.sq1[2] == a.sq2[2];
        p.qoff32 = same && 2 * qmost <= INT32_MAX && (int64_t)a.H * a.N * kDV * 2 <= INT32_MAX;
        const int64_t n1 = std::max<int64_t>(a.N - 1, 63);
        const int64_t kmost = std::max(std::max(a.sk1[2], a.sk2[2]) * n1 + a.d_qk, a.sv[2] * n1 + kDV);
        p.koff32 = a.sk1[2] == a.sk2[2] && 2 * kmost <= INT32_MAX;
    }
    p.scale = scale;
    p.sc_log2 = scale * kLog2e;
    p.eps = a.eps;
    p.one_minus_init = 1.0f - lambda_init;

    hipLaunchKernelGGL(bwd_prep_kernel, dim3(p.prep_nblk, a.H, a.B), dim3(256), 0, stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(bwd_finalize_kernel, dim3(a.H), dim3(512), 0, stream, p);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (a.d_qk == 64) return plan.shared_k ? launch_w<64, true>(p, stream) : launch_w<64, false>(p, stream);
    return plan.shared_k ? launch_w<128, true>(p, stream) : launch_w<128, false>(p, stream);
}

hipError_t launch_lambda_backward(const float *lq1, const float *lk1, const float *lq2, const float *lk2, int H,
                                  int d_lambda, const float *dlambda, float *dlq1, float *dlk1, float *dlq2,
                                  float *dlk2, hipStream_t stream) {
    hipLaunchKernelGGL(lambda_backward_kernel, dim3(H), dim3(256), 0, stream, lq1, lk1, lq2, lk2, d_lambda, dlambda,
                       dlq1, dlk1, dlq2, dlk2);
    return hipGetLastError();
}

}  // namespace da
