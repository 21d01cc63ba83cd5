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
//                       rows of one head, 8 waves = 4 row groups x 2 branches;
//                       per 32-key sub-block S^T = K Q^T, G^T = V dy^T,
//                       dS^T, dQ^T += K^T dS^T (K^T by transposing LDS reads)
//  bwd_dkdv_kernel      key-major: a work-group owns 128 keys of one KV head,
//                       4 waves x 32 keys, both branches per wave, and sweeps
//                       the query tiles of every head of the group: S = Q K^T,
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
    float *dt1, *dt2;  // workspace: rowsum(dy * o_k), [B, H, N]
    float *part;       // workspace: per prep block [dlambda, dgamma[128]]
    int B, H, H_kv, group, N, causal, window, norm, prep_nblk, row_blocks, key_blocks;
    float scale, sc_log2, eps, one_minus_init;
};

// ---------------------------------------------------------------- prep

__global__ __launch_bounds__(256) void bwd_prep_kernel(BwdParams p) {
    // a block of kBwdPrepRows rows of one (batch, head): each wave takes every
    // 4th row; the block's dlambda and dgamma sums go to one partial record
    __shared__ float red[4][kDV + 1];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int blk = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int c0 = lane, c1 = lane + 64;
    const float lam = p.lambda[h];
    const float c = p.one_minus_init;
    const float gm0 = p.norm ? c * p.gamma[(int64_t)h * kDV + c0] : 0.0f;
    const float gm1 = p.norm ? c * p.gamma[(int64_t)h * kDV + c1] : 0.0f;
    float dl = 0.0f, pg0 = 0.0f, pg1 = 0.0f;
    const int iend = min(p.N, (blk + 1) * kBwdPrepRows);
    for (int i = blk * kBwdPrepRows + wave; i < iend; i += 4) {
        const int64_t rowid = ((int64_t)b * p.H + h) * p.N + i;
        const float a0 = p.o1[rowid * kDV + c0], a1 = p.o1[rowid * kDV + c1];
        const float e0 = p.o2[rowid * kDV + c0], e1 = p.o2[rowid * kDV + c1];
        const __bf16 *dz = p.dout + b * p.sdo[0] + h * p.sdo[1] + (int64_t)i * p.sdo[2];
        const float z0 = (float)dz[c0], z1 = (float)dz[c1];
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
            if (p.norm == 2) {
                const float mu = wave_sum(y0 + y1) * (1.0f / kDV);
                y0 -= mu;
                y1 -= mu;
            }
            const float r = 1.0f / sqrtf(wave_sum(y0 * y0 + y1 * y1) * (1.0f / kDV) + p.eps);
            float g0 = gm0 * z0, g1 = gm1 * z1;
            const float k3 = r * r * r * (1.0f / kDV) * wave_sum(g0 * y0 + g1 * y1);
            if (p.norm == 2) {
                const float gmean = wave_sum(g0 + g1) * (1.0f / kDV);
                g0 -= gmean;
                g1 -= gmean;
            }
            d0 = r * g0 - y0 * k3;
            d1 = r * g1 - y1 * k3;
            pg0 += z0 * y0 * r * c;
            pg1 += z1 * y1 * r * c;
        }
        dl -= wave_sum(d0 * e0 + d1 * e1);
        const __bf16 b0 = (__bf16)d0, b1 = (__bf16)d1;
        p.dy[rowid * kDV + c0] = b0;
        p.dy[rowid * kDV + c1] = b1;
        // the softmax-backward row sums use the rounded dy the products use
        const float f0 = (float)b0, f1 = (float)b1;
        const float t1 = wave_sum(f0 * a0 + f1 * a1);
        const float t2 = wave_sum(f0 * e0 + f1 * e1);
        if (lane == 0) {
            p.dt1[rowid] = t1;
            p.dt2[rowid] = t2;
        }
    }
    red[wave][c0] = pg0;
    red[wave][c1] = pg1;
    if (lane == 0) red[wave][kDV] = dl;
    __syncthreads();
    float *pp = p.part + (((int64_t)b * p.H + h) * p.prep_nblk + blk) * (kDV + 1);
    for (int k = threadIdx.x; k <= kDV; k += 256) {
        const float s = (red[0][k] + red[1][k]) + (red[2][k] + red[3][k]);
        pp[k == kDV ? 0 : 1 + k] = s;
    }
}

__global__ __launch_bounds__(256) void bwd_finalize_kernel(BwdParams p) {
    // per head: the partial records summed in a fixed order (deterministic);
    // thread t < 129 owns value t of every record (t = 0: dlambda, else
    // dgamma[t - 1]) and keeps 8 independent running sums
    const int h = blockIdx.x, t = threadIdx.x;
    if (t > kDV) return;
    const int64_t n = (int64_t)p.B * p.prep_nblk;
    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    int64_t k = 0;
    for (; k + 8 <= n; k += 8)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int64_t r = k + e, bb = r / p.prep_nblk, kb = r - bb * p.prep_nblk;
            acc[e] += p.part[(((int64_t)bb * p.H + h) * p.prep_nblk + kb) * (kDV + 1) + t];
        }
    for (; k < n; ++k) {
        const int64_t bb = k / p.prep_nblk, kb = k - bb * p.prep_nblk;
        acc[0] += p.part[(((int64_t)bb * p.H + h) * p.prep_nblk + kb) * (kDV + 1) + t];
    }
    const float s = ((acc[0] + acc[1]) + (acc[2] + acc[3])) + ((acc[4] + acc[5]) + (acc[6] + acc[7]));
    if (t == 0)
        p.dlambda[h] = s;
    else if (p.norm)
        p.dgamma[(int64_t)h * kDV + t - 1] = s;
}

// ---------------------------------------------------------------- dQ

template <int DQK, bool SHARED_K, bool WIN>
__global__ __launch_bounds__(512, 1) void bwd_dq_kernel(BwdParams p) {
    using T = Tile<DQK, SHARED_K>;
    constexpr int KC = DQK / 16;
    constexpr int NW = 8;
    __shared__ __attribute__((aligned(1024))) unsigned char st0[T::kStage];
    __shared__ __attribute__((aligned(1024))) unsigned char st1[T::kStage];

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int l32 = lane & 31, hh = lane >> 5;
    const int br = wave & 1, rg = wave >> 1;

    const int U = p.B * p.H;
    const int rank = blockIdx.x / U, u = blockIdx.x - rank * U;
    const int b = u / p.H, h = u - b * p.H;
    const int rb = p.causal ? p.row_blocks - 1 - rank : rank;  // longest rows first
    const int g = h / p.group;
    const int q0 = rb * kBM;
    const int wrow0 = q0 + rg * kWM;
    const int myrow = wrow0 + l32;
    const int row = min(myrow, p.N - 1);  // rows past the end compute garbage, never stored
    const int64_t rowid = ((int64_t)b * p.H + h) * p.N + row;

    // B operands: this wave's branch of Q, and dy, for the lane's row
    bf16x8 qf[KC], df[8];
    {
        const __bf16 *q = br ? p.q2 + b * p.sq2[0] + h * p.sq2[1] + (int64_t)row * p.sq2[2]
                             : p.q1 + b * p.sq1[0] + h * p.sq1[1] + (int64_t)row * p.sq1[2];
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) qf[kc] = as_bf16x8(ldg16(q + 8 * hh + 16 * kc));
        const __bf16 *d = p.dy + rowid * kDV;
#pragma unroll
        for (int kc = 0; kc < 8; ++kc) df[kc] = as_bf16x8(ldg16(d + 8 * hh + 16 * kc));
    }
    const float lse2 = (br ? p.lse2 : p.lse1)[rowid] * kLog2e;  // log2 units
    const float dtr = (br ? p.dt2 : p.dt1)[rowid];
    const float w = br ? -p.lambda[h] : 1.0f;

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
    auto issue_tile = [&](int t, unsigned char *base) DA_INLINE {
        const int key0 = t * kBN;
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

    f32x16 dq[DQK / 32];
#pragma unroll
    for (int dc = 0; dc < DQK / 32; ++dc) dq[dc] = f32x16{};
    const int krow = perm_key(l32);
    const int kt_off = SHARED_K ? 0 : br * T::kKBytes;

    auto step = [&](const unsigned char *base, int sb, bool mask, int lim, int lo) DA_INLINE {
        const unsigned char *kt = base + kt_off;
        const unsigned char *vt = base + T::kNK * T::kKBytes;
        const int r0 = 32 * sb + krow;
        bf16x8 kf[KC];
#pragma unroll
        for (int kc = 0; kc < KC; ++kc)
            kf[kc] = as_bf16x8(*(const uint4 *)(kt + r0 * (2 * DQK) + 16 * ((2 * kc + hh) ^ bk_swz<DQK>(r0))));
        f32x16 s = f32x16{};
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) s = mfma32(kf[kc], qf[kc], s);
        f32x16 gq = f32x16{};
#pragma unroll
        for (int kc = 0; kc < 8; ++kc)
            gq = mfma32(as_bf16x8(*(const uint4 *)(vt + r0 * 256 + 16 * ((2 * kc + hh) ^ bv_swz(r0)))), df[kc], gq);
        float pr[16], ds[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) pr[r] = exp2_fast(fmaf(s[r], p.sc_log2, -lse2));
        if (mask) {
            // an opaque statement keeps this a branch taken by the few masked
            // sub-blocks, instead of per-element selects evaluated for all
            asm volatile("");
#pragma unroll
            for (int r = 0; r < 16; ++r)
                if (key_of_reg(r) >= lim || key_of_reg(r) < lo) pr[r] = 0.0f;
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) ds[r] = w * pr[r] * (gq[r] - dtr);
        bf16x8 pb[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const bf16x2 a = pack2(ds[8 * t + 0], ds[8 * t + 1]), c = pack2(ds[8 * t + 2], ds[8 * t + 3]);
            const bf16x2 e = pack2(ds[8 * t + 4], ds[8 * t + 5]), f = pack2(ds[8 * t + 6], ds[8 * t + 7]);
            pb[t] = bf16x8{a[0], a[1], c[0], c[1], e[0], e[1], f[0], f[1]};
        }
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int dc = 0; dc < DQK / 32; ++dc)
                dq[dc] = mfma32(tr_frag(kt, lane, 2 * DQK, BSwzK<DQK>(), sb, t, dc), pb[t], dq[dc]);
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
        float *o = (br ? p.dq2 : p.dq1) + (((int64_t)b * p.H + h) * p.N + myrow) * DQK + 4 * hh;
#pragma unroll
        for (int dc = 0; dc < DQK / 32; ++dc)
#pragma unroll
            for (int rq = 0; rq < 4; ++rq) {
                const float4 v4 = {dq[dc][4 * rq] * p.scale, dq[dc][4 * rq + 1] * p.scale, dq[dc][4 * rq + 2] * p.scale,
                                   dq[dc][4 * rq + 3] * p.scale};
                *(float4 *)(o + 32 * dc + 8 * rq) = v4;
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
    const int kblk = blockIdx.x / U, u = blockIdx.x - kblk * U;  // key blocks with the most queries first
    const int b = u / p.H_kv, g = u - b * p.H_kv;
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

    auto issue_tile = [&](int x, unsigned char *base) DA_INLINE {
        const int hg = x / nt, t = tlo + x - hg * nt;
        const int h = g * p.group + hg;
        const int r0 = t * kBN;
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
                __builtin_amdgcn_global_load_lds(db + (int64_t)q * kDV + col, (lds_void *)(base + blk * 1024), 16, 0,
                                                 0);
            }
        }
        // statistics: wave w loads array w (lse_1, lse_2, dt_1, dt_2), lane = row
        {
            const int q = min(r0 + lane, p.N - 1);
            const int64_t rid = ((int64_t)b * p.H + h) * p.N + q;
            const float *src = wave == 0 ? p.lse1 : wave == 1 ? p.lse2 : wave == 2 ? p.dt1 : p.dt2;
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

    // one 32-row query sub-block of the tile at `base` (query rows qb .. qb+31)
    auto step = [&](const unsigned char *base, int sb, int qb, float lamh, bool mask) DA_INLINE {
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
        for (int kc = 0; kc < 8; ++kc) ad[kc] = as_bf16x8(*(const uint4 *)(td + r0 * 256 + 16 * ((2 * kc + hh) ^ bv_swz(r0))));
        __builtin_amdgcn_sched_barrier(0);
        f32x16 s1 = f32x16{}, s2 = f32x16{}, gq = f32x16{};
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) {
            s1 = mfma32(a1[kc], kf1[kc], s1);
            s2 = mfma32(a2[kc], kf2[kc], s2);
        }
#pragma unroll
        for (int kc = 0; kc < 8; ++kc) gq = mfma32(ad[kc], vf[kc], gq);
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
                p1[r] = exp2_fast(fmaf(s1[r], p.sc_log2, -L1[e] * kLog2e));
                p2[r] = exp2_fast(fmaf(s2[r], p.sc_log2, -L2[e] * kLog2e));
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
            pw[r] = p1[r] - lamh * p2[r];
            d1[r] = p1[r] * (gq[r] - D1[r]);
            d2[r] = -lamh * p2[r] * (gq[r] - D2[r]);
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
#pragma unroll
        for (int t = 0; t < 2; ++t) {
#pragma unroll
            for (int dc = 0; dc < 4; ++dc) dva[dc] = mfma32(tr_frag(td, lane, 256, BSwzV(), sb, t, dc), wb[t], dva[dc]);
#pragma unroll
            for (int dc = 0; dc < DQK / 32; ++dc) {
                dk1a[dc] = mfma32(tr_frag(t1, lane, 2 * DQK, BSwzK<DQK>(), sb, t, dc), s1b[t], dk1a[dc]);
                if (SHARED_K)
                    dk1a[dc] = mfma32(tr_frag(t2, lane, 2 * DQK, BSwzK<DQK>(), sb, t, dc), s2b[t], dk1a[dc]);
                else
                    dk2a[dc] = mfma32(tr_frag(t2, lane, 2 * DQK, BSwzK<DQK>(), sb, t, dc), s2b[t], dk2a[dc]);
            }
        }
    };

    auto tile_body = [&](const unsigned char *base, int x) DA_INLINE {
        const int hg = x / nt, t = tlo + x - hg * nt;
        const float lamh = ld_uniform(p.lambda + g * p.group + hg);
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
            const int qb = t * kBN + 32 * sb;  // first query row of the sub-block
            // wholly invisible to this wave's keys: skip
            if (qb >= p.N) continue;
            if (p.causal && qb + 31 < kw0) continue;
            if (WIN && qb > kw0 + kWM - 1 + win - 1) continue;
            const bool mask = qb + 31 >= p.N || (p.causal && qb < kw0 + kWM - 1) ||
                              (WIN && qb + 31 > kw0 + win - 1);
            step(base, sb, qb, lamh, mask);
        }
    };
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

template <int DQK, bool SHARED_K, bool WIN>
hipError_t launch_main(const BwdParams &p, hipStream_t stream) {
    const int64_t dq_blocks = (int64_t)p.B * p.H * p.row_blocks;
    const int64_t kv_blocks = (int64_t)p.B * p.H_kv * p.key_blocks;
    if (dq_blocks > 0x7fffffff || kv_blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((bwd_dq_kernel<DQK, SHARED_K, WIN>), dim3((int)dq_blocks), dim3(512), 0, stream, p);
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
    p.scale = scale;
    p.sc_log2 = scale * kLog2e;
    p.eps = a.eps;
    p.one_minus_init = 1.0f - lambda_init;

    hipLaunchKernelGGL(bwd_prep_kernel, dim3(p.prep_nblk, a.H, a.B), dim3(256), 0, stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(bwd_finalize_kernel, dim3(a.H), dim3(256), 0, stream, p);
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
