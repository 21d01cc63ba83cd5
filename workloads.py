"""Seeded synthetic inputs for differential attention.

This module is shared by the tests, the benchmark and the smoke check. It
holds random draws, bf16 rounding of the draws, page-table construction and
the planting of signal keys: nothing of the attention arithmetic itself, so
neither the CPU oracle nor the HIP path gets any of its math from here.

Every array is produced by ``numpy.random.default_rng(seed)`` (PCG64) in a
fixed draw order. bf16 inputs are drawn in fp32, rounded to bf16 with
round-to-nearest-even on the integer bits, and kept as ``uint16`` bit
patterns; ``bf16_to_f32`` widens them exactly, so the oracle (fp64) and the
kernels (bf16) see the same numbers.

Workloads (shapes follow the lesson "Differential Attention (V2)", sections
"V1 vs V2" and "Build it, step 5" for the 7B-class hidden 4096 / 32 heads /
d_head 128 shape, and its exercise on GQA with 8 KV heads and 32 query heads):

* ``tiny_v1``      V1, 1 head, N 128, causal, fp32, d_qk 64, d_v 128, depth 1.
* ``prefill_v1``   V1, B 2, H 16, N 4096, causal, bf16, d_qk 64, d_v 128, depth 12.
* ``prefill_v2``   V2 GQA, B 1, 64 query heads (32 pairs), 8 KV heads, N 16384,
                   causal, bf16, d 128, depth 20.
* ``decode_v2``    V2 paged decode, 64 sequences, context U{8192..32768},
                   page 64, 8 KV heads, 64 query heads, bf16, d 128, depth 20.
* ``decode_v2_fp8`` the V2 decode with an fp8 (e4m3) KV cache, per-tensor
                   scale 1/56 for K and for V.
* ``decode_v1``    V1 paged decode, the same sequences and pages as the V2
                   decode's shape family with d_qk 64 (separate K1, K2 caches),
                   d_v 128, 32 heads over 8 KV heads, RMS norm, depth 12.
* ``longctx_v1``   V1, B 1, H 8, N 65536, causal, bf16, d_qk 64, d_v 128,
                   16 planted signal keys per head (the lesson's signal-plus-
                   noise toy, section "Build it, step 4", at 64K scale).

Each maker accepts overrides of its sizes so tests can build small instances
with the same value distributions and structure.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Dict, Optional

import numpy as np

# --------------------------------------------------------------------------
# bf16 bit handling (round-to-nearest-even on the fp32 bit pattern)
# --------------------------------------------------------------------------


def f32_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (RNE) and return the uint16 bit patterns."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    out = np.empty(u.shape, dtype=np.uint16)
    # chunked to bound temporary memory on very large arrays
    flat_u = u.reshape(-1)
    flat_o = out.reshape(-1)
    step = 1 << 24
    for s in range(0, flat_u.size, step):
        c = flat_u[s:s + step]
        r = ((c >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
        flat_o[s:s + step] = ((c + r) >> np.uint32(16)).astype(np.uint16)
    return out


def bf16_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen uint16 bf16 bit patterns to fp32 (exact)."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _normal(rng: np.random.Generator, shape, std: float = 1.0) -> np.ndarray:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return x


# --------------------------------------------------------------------------
# containers
# --------------------------------------------------------------------------


@dataclass
class Prefill:
    """One prefill problem. Arrays are fp32 (dtype 'f32') or uint16 bf16 bits ('bf16').

    q1, q2 : [B, H, N, d_qk]   (for V2 they are views of one [B, 2H, N, d] tensor)
    k1, k2 : [B, H_kv, N, d_qk] (k2 is k1 when the branches share keys)
    v      : [B, H_kv, N, d_v]
    lam_*  : [H, d_lambda] fp32 lambda re-parameterisation vectors
    gamma  : [H, d_v] fp32 norm gain, or None (no norm)
    """
    name: str
    dtype: str
    B: int
    H: int
    H_kv: int
    N: int
    d_qk: int
    d_v: int
    q1: np.ndarray
    q2: np.ndarray
    k1: np.ndarray
    k2: np.ndarray
    v: np.ndarray
    lam_q1: np.ndarray
    lam_k1: np.ndarray
    lam_q2: np.ndarray
    lam_k2: np.ndarray
    depth: int
    causal: bool
    norm: bool
    gamma: Optional[np.ndarray]
    eps: float = 1e-5
    shared_k: bool = False
    q_full: Optional[np.ndarray] = None  # V2: the [B, 2H, N, d] query tensor
    probes: Optional[np.ndarray] = None  # longctx: [H, 16, 2] (planted key, probe row)
    extra: Dict = field(default_factory=dict)

    def f32(self, name: str) -> np.ndarray:
        a = getattr(self, name)
        return bf16_to_f32(a) if self.dtype == "bf16" else a


@dataclass
class Decode:
    """One paged decode step (one new query token per sequence).

    q1, q2   : [B, H, d_qk]
    k_cache  : [P, H_kv, page, d_qk] (shared by both branches in V2)
    v_cache  : [P, H_kv, page, d_v]
    page_table : [B, max_pages] int32, -1 for unused slots
    ctx_len  : [B] int32
    """
    name: str
    dtype: str
    B: int
    H: int
    H_kv: int
    d_qk: int
    d_v: int
    page: int
    max_pages: int
    num_pages: int
    q1: np.ndarray
    q2: np.ndarray
    k1_cache: np.ndarray
    k2_cache: np.ndarray
    v_cache: np.ndarray
    page_table: np.ndarray
    ctx_len: np.ndarray
    lam_q1: np.ndarray
    lam_k1: np.ndarray
    lam_q2: np.ndarray
    lam_k2: np.ndarray
    depth: int
    norm: bool
    gamma: Optional[np.ndarray]
    eps: float = 1e-5
    shared_k: bool = True
    q_full: Optional[np.ndarray] = None  # [B, 2H, d]
    kv_dtype: str = "bf16"               # or "fp8": the caches hold e4m3 codes (uint8)
    k_scale: float = 1.0                 # fp8: key = k_scale * value of the code
    v_scale: float = 1.0                 # fp8: value = v_scale * value of the code

    @property
    def kv_bytes(self) -> int:
        return 1 if self.kv_dtype == "fp8" else 2

    def f32(self, name: str) -> np.ndarray:
        return self.values(name, getattr(self, name))

    def values(self, name: str, a: np.ndarray) -> np.ndarray:
        """fp32 values of array ``a`` stored as field ``name`` (a slice of a
        cache, say): fp8 caches dequantised with their scale."""
        if name.endswith("_cache") and self.kv_dtype == "fp8":
            scale = self.v_scale if name == "v_cache" else self.k_scale
            return fp8_to_f32(a) * np.float32(scale)
        return bf16_to_f32(a) if self.dtype == "bf16" else a


# --------------------------------------------------------------------------
# fp8, OCP e4m3: sign, 4 exponent bits (bias 7), 3 mantissa bits; no
# infinities; S.1111.111 is NaN; the largest finite magnitude is 448
# --------------------------------------------------------------------------

FP8_MAX = 448.0


def f32_to_fp8(x: np.ndarray) -> np.ndarray:
    """Round fp32 values inside [-448, 448] to e4m3 (nearest, ties to even);
    returns the uint8 codes."""
    import torch
    x = np.ascontiguousarray(x, dtype=np.float32)
    assert np.all(np.abs(x) <= FP8_MAX)
    return torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _fp8_table() -> np.ndarray:
    """The value of every e4m3 code, from the format's definition."""
    t = np.empty(256, np.float32)
    for c in range(256):
        s, e, m = c >> 7, (c >> 3) & 15, c & 7
        if e == 15 and m == 7:
            v = float("nan")
        elif e == 0:
            v = m / 8.0 * 2.0 ** -6
        else:
            v = (1.0 + m / 8.0) * 2.0 ** (e - 7)
        t[c] = -v if s else v
    return t


FP8_TABLE = _fp8_table()


def fp8_to_f32(codes: np.ndarray) -> np.ndarray:
    """Exact values of e4m3 codes."""
    return FP8_TABLE[np.asarray(codes, np.uint8)]


def _lambda_vectors(rng, H, d_l):
    return tuple(_normal(rng, (H, d_l), 0.1) for _ in range(4))


# --------------------------------------------------------------------------
# the workloads
# --------------------------------------------------------------------------


def tiny_v1(seed: int = 1, N: int = 128, d_qk: int = 64, d_v: int = 128,
            B: int = 1, H: int = 1, causal: bool = True) -> Prefill:
    """V1, fp32: Q1, K1, Q2, K2 [B,H,N,d_qk] and V [B,H,N,d_v] ~ N(0,1); lambda
    vectors [H, d_qk] ~ N(0, 0.1^2); gamma = 1; depth 1; causal."""
    rng = np.random.default_rng(seed)
    q1 = _normal(rng, (B, H, N, d_qk))
    k1 = _normal(rng, (B, H, N, d_qk))
    q2 = _normal(rng, (B, H, N, d_qk))
    k2 = _normal(rng, (B, H, N, d_qk))
    v = _normal(rng, (B, H, N, d_v))
    lq1, lk1, lq2, lk2 = _lambda_vectors(rng, H, d_qk)
    gamma = np.ones((H, d_v), np.float32)
    return Prefill("tiny_v1", "f32", B, H, H, N, d_qk, d_v, q1, q2, k1, k2, v,
                   lq1, lk1, lq2, lk2, depth=1, causal=causal, norm=True, gamma=gamma)


def prefill_v1(seed: int = 2, B: int = 2, H: int = 16, N: int = 4096,
               d_qk: int = 64, d_v: int = 128, causal: bool = True,
               depth: int = 12) -> Prefill:
    """V1, bf16: all of Q1, K1, Q2, K2, V ~ 0.5 N(0,1); lambda vectors
    [H, d_qk] ~ N(0, 0.1^2); gamma ~ U(0.9, 1.1); depth 12; causal."""
    rng = np.random.default_rng(seed)
    q1 = f32_to_bf16(_normal(rng, (B, H, N, d_qk), 0.5))
    k1 = f32_to_bf16(_normal(rng, (B, H, N, d_qk), 0.5))
    q2 = f32_to_bf16(_normal(rng, (B, H, N, d_qk), 0.5))
    k2 = f32_to_bf16(_normal(rng, (B, H, N, d_qk), 0.5))
    v = f32_to_bf16(_normal(rng, (B, H, N, d_v), 0.5))
    lq1, lk1, lq2, lk2 = _lambda_vectors(rng, H, d_qk)
    gamma = rng.uniform(0.9, 1.1, size=(H, d_v)).astype(np.float32)
    return Prefill("prefill_v1", "bf16", B, H, H, N, d_qk, d_v, q1, q2, k1, k2, v,
                   lq1, lk1, lq2, lk2, depth=depth, causal=causal, norm=True, gamma=gamma)


def prefill_v2(seed: int = 3, B: int = 1, H: int = 32, H_kv: int = 8, N: int = 16384,
               d: int = 128, causal: bool = True, depth: int = 20) -> Prefill:
    """V2 GQA, bf16: Q [B, 2H, N, d] ~ N(0,1)/sqrt(2); K, V [B, H_kv, N, d] ~ N(0,1);
    lambda vectors [H, d] ~ N(0, 0.1^2); no norm; depth 20; causal.

    Query head 2p is branch 1 and 2p+1 is branch 2 of output head p, so
    q1 = Q[:, 0::2], q2 = Q[:, 1::2]; both branches read KV head p // (H / H_kv)."""
    rng = np.random.default_rng(seed)
    q = f32_to_bf16(_normal(rng, (B, 2 * H, N, d), 1.0 / math.sqrt(2.0)))
    k = f32_to_bf16(_normal(rng, (B, H_kv, N, d)))
    v = f32_to_bf16(_normal(rng, (B, H_kv, N, d)))
    lq1, lk1, lq2, lk2 = _lambda_vectors(rng, H, d)
    return Prefill("prefill_v2", "bf16", B, H, H_kv, N, d, d, q[:, 0::2], q[:, 1::2], k, k, v,
                   lq1, lk1, lq2, lk2, depth=depth, causal=causal, norm=False, gamma=None,
                   shared_k=True, q_full=q)


def decode_v2_fp8(**kw) -> Decode:
    """decode_v2 with an fp8 (e4m3) KV cache: the same draws, each K and V
    sample divided by the per-tensor scale 1/56 (|x| <= 8 stays inside the
    e4m3 range; larger samples clip to the +-448 codes) and rounded to e4m3."""
    return decode_v2(kv_dtype="fp8", **kw)


def decode_v2(seed: int = 4, B: int = 64, H: int = 32, H_kv: int = 8, d: int = 128,
              page: int = 64, max_pages: int = 512, ctx_lo: int = 8192, ctx_hi: int = 32768,
              depth: int = 20, ctx_len: Optional[np.ndarray] = None, kv_dtype: str = "bf16") -> Decode:
    """V2 paged decode, bf16. Draw order: ctx_len ~ U{ctx_lo..ctx_hi}; a random
    permutation of the P = sum ceil(L_b/page) physical pages, assigned to
    (sequence, logical page) in order (unused table slots are -1); K and V pools
    [P, H_kv, page, d] ~ N(0,1) (slots past a sequence's length are random and
    must be masked); Q [B, 2H, d] ~ N(0,1)/sqrt(2); lambda vectors [H, d]."""
    rng = np.random.default_rng(seed)
    if ctx_len is None:
        ctx_len = rng.integers(ctx_lo, ctx_hi + 1, size=B).astype(np.int32)
    else:
        ctx_len = np.asarray(ctx_len, np.int32)
        assert ctx_len.shape == (B,)
    npg = (ctx_len.astype(np.int64) + page - 1) // page
    assert int(npg.max()) <= max_pages
    P = int(npg.sum())
    perm = rng.permutation(P).astype(np.int32)
    table = np.full((B, max_pages), -1, np.int32)
    pos = 0
    for b in range(B):
        n = int(npg[b])
        table[b, :n] = perm[pos:pos + n]
        pos += n
    fp8 = kv_dtype == "fp8"
    kv_scale = 1.0 / 56.0
    if fp8:
        enc = lambda x: f32_to_fp8(np.clip(x / np.float32(kv_scale), -FP8_MAX, FP8_MAX))
    else:
        enc = f32_to_bf16
    k_cache = np.empty((P, H_kv, page, d), np.uint8 if fp8 else np.uint16)
    v_cache = np.empty((P, H_kv, page, d), np.uint8 if fp8 else np.uint16)
    chunk = max(1, (1 << 24) // (H_kv * page * d))
    for s in range(0, P, chunk):
        e = min(P, s + chunk)
        k_cache[s:e] = enc(_normal(rng, (e - s, H_kv, page, d)))
    for s in range(0, P, chunk):
        e = min(P, s + chunk)
        v_cache[s:e] = enc(_normal(rng, (e - s, H_kv, page, d)))
    q = f32_to_bf16(_normal(rng, (B, 2 * H, d), 1.0 / math.sqrt(2.0)))
    lq1, lk1, lq2, lk2 = _lambda_vectors(rng, H, d)
    return Decode("decode_v2_fp8" if fp8 else "decode_v2", "bf16", B, H, H_kv, d, d, page, max_pages,
                  P, q[:, 0::2], q[:, 1::2], k_cache, k_cache, v_cache, table, ctx_len,
                  lq1, lk1, lq2, lk2, depth=depth, norm=False, gamma=None, q_full=q,
                  kv_dtype=kv_dtype, k_scale=kv_scale if fp8 else 1.0,
                  v_scale=kv_scale if fp8 else 1.0)


def decode_v1(seed: int = 6, B: int = 64, H: int = 32, H_kv: int = 8, d_qk: int = 64,
              d_v: int = 128, page: int = 64, max_pages: int = 512, ctx_lo: int = 8192,
              ctx_hi: int = 32768, depth: int = 12, ctx_len: Optional[np.ndarray] = None,
              kv_dtype: str = "bf16") -> Decode:
    """V1 paged decode, bf16 (kv_dtype "fp8": the pools' samples divided by the
    per-tensor scale 1/112 and rounded to e4m3 codes): the V2 decode's shape family with the V1 head
    split (d_qk 64 per branch, separate K1 and K2 caches, one V cache of width
    128) and the V1 norm. Draw order: ctx_len ~ U{ctx_lo..ctx_hi}; a random
    permutation of the P = sum ceil(L_b/page) physical pages assigned to
    (sequence, logical page) in order (unused table slots -1); K1, K2 pools
    [P, H_kv, page, d_qk] and the V pool [P, H_kv, page, d_v], each
    0.5 N(0,1) (slots past a sequence's length are random and must be masked);
    Q1, Q2 [B, H, d_qk] ~ 0.5 N(0,1); lambda vectors [H, d_qk] ~ N(0, 0.1^2);
    gamma [H, d_v] ~ U(0.9, 1.1); depth 12; RMS norm."""
    rng = np.random.default_rng(seed)
    if ctx_len is None:
        ctx_len = rng.integers(ctx_lo, ctx_hi + 1, size=B).astype(np.int32)
    else:
        ctx_len = np.asarray(ctx_len, np.int32)
        assert ctx_len.shape == (B,)
    npg = (ctx_len.astype(np.int64) + page - 1) // page
    assert int(npg.max()) <= max_pages
    P = int(npg.sum())
    perm = rng.permutation(P).astype(np.int32)
    table = np.full((B, max_pages), -1, np.int32)
    pos = 0
    for b in range(B):
        n = int(npg[b])
        table[b, :n] = perm[pos:pos + n]
        pos += n

    fp8 = kv_dtype == "fp8"
    kv_scale = 1.0 / 112.0

    def pool(d):
        out = np.empty((P, H_kv, page, d), np.uint8 if fp8 else np.uint16)
        chunk = max(1, (1 << 24) // (H_kv * page * d))
        for s in range(0, P, chunk):
            e = min(P, s + chunk)
            x = _normal(rng, (e - s, H_kv, page, d), 0.5)
            if fp8:
                out[s:e] = f32_to_fp8(np.clip(x / np.float32(kv_scale), -FP8_MAX, FP8_MAX))
            else:
                out[s:e] = f32_to_bf16(x)
        return out

    k1_cache, k2_cache, v_cache = pool(d_qk), pool(d_qk), pool(d_v)
    q1 = f32_to_bf16(_normal(rng, (B, H, d_qk), 0.5))
    q2 = f32_to_bf16(_normal(rng, (B, H, d_qk), 0.5))
    lq1, lk1, lq2, lk2 = _lambda_vectors(rng, H, d_qk)
    gamma = rng.uniform(0.9, 1.1, size=(H, d_v)).astype(np.float32)
    return Decode("decode_v1_fp8" if fp8 else "decode_v1", "bf16", B, H, H_kv, d_qk, d_v, page,
                  max_pages, P, q1, q2, k1_cache, k2_cache, v_cache, table, ctx_len,
                  lq1, lk1, lq2, lk2, depth=depth, norm=True, gamma=gamma, shared_k=False,
                  kv_dtype=kv_dtype, k_scale=kv_scale if fp8 else 1.0,
                  v_scale=kv_scale if fp8 else 1.0)


def longctx_v1(seed: int = 5, B: int = 1, H: int = 8, N: int = 65536, d_qk: int = 64,
               d_v: int = 128, n_planted: int = 16, depth: int = 12) -> Prefill:
    """V1 long context, bf16, signal-plus-noise keys.

    Q1, Q2, K1, K2 [B,H,N,d_qk] and V [B,H,N,d_v] ~ N(0,1). Per (batch, head),
    n_planted distinct key positions p ~ U[0, N-1), each with a probe row
    t ~ U{p+1..N-1}; K1[p] is replaced by sqrt(d_qk) * (0.9 q1_hat[t] +
    sqrt(0.19) u), u a random unit vector orthogonal to q1_hat[t] (cosine 0.9
    with the probe query, norm sqrt(d_qk)). K2 stays noise, so the planted key
    is signal for branch 1 only. All tensors are then rounded to bf16."""
    rng = np.random.default_rng(seed)
    q1 = _normal(rng, (B, H, N, d_qk))
    q2 = _normal(rng, (B, H, N, d_qk))
    k1 = _normal(rng, (B, H, N, d_qk))
    k2 = _normal(rng, (B, H, N, d_qk))
    v = _normal(rng, (B, H, N, d_v))
    probes = np.zeros((B, H, n_planted, 2), np.int64)
    for b in range(B):
        for h in range(H):
            ps = rng.choice(N - 1, size=n_planted, replace=False)
            for i, p in enumerate(ps):
                t = int(rng.integers(p + 1, N))
                qh = q1[b, h, t].astype(np.float64)
                qh /= np.linalg.norm(qh)
                u = rng.standard_normal(d_qk)
                u -= (u @ qh) * qh
                u /= np.linalg.norm(u)
                key = math.sqrt(d_qk) * (0.9 * qh + math.sqrt(0.19) * u)
                k1[b, h, p] = key.astype(np.float32)
                probes[b, h, i] = (p, t)
    lq1, lk1, lq2, lk2 = _lambda_vectors(rng, H, d_qk)
    gamma = rng.uniform(0.9, 1.1, size=(H, d_v)).astype(np.float32)
    return Prefill("longctx_v1", "bf16", B, H, H, N, d_qk, d_v,
                   f32_to_bf16(q1), f32_to_bf16(q2), f32_to_bf16(k1), f32_to_bf16(k2),
                   f32_to_bf16(v), lq1, lk1, lq2, lk2, depth=depth, causal=True, norm=True,
                   gamma=gamma, probes=probes)


WORKLOADS = {
    "tiny_v1": tiny_v1,
    "prefill_v1": prefill_v1,
    "prefill_v2": prefill_v2,
    "decode_v2": decode_v2,
    "longctx_v1": longctx_v1,
}


def sample_rows(N: int, rng: np.random.Generator, n_rand: int = 64, edge: int = 32) -> np.ndarray:
    """Row indices to spot-check in a full-size problem: the first and last
    ``edge`` rows plus ``n_rand`` seeded random rows (sorted, unique)."""
    rows = set(range(min(edge, N)))
    rows.update(range(max(0, N - edge), N))
    if N > 0:
        rows.update(int(r) for r in rng.integers(0, N, size=n_rand))
    return np.array(sorted(rows), np.int64)
