"""Brute-force differential attention in standard-library Python. TEST INFRASTRUCTURE ONLY.

A second implementation, for tiny shapes, whose only job is to pin the C
oracle. It works on nested lists of Python floats, written from the
definitions in the lesson "Differential Attention (V2)" (section "Concept":
two softmax maps, their difference scaled by lambda, times V; section "V1 vs
V2": the per-head RMSNorm of V1) and the causal mask of the lesson
"Attention Variants" ("Build it", step 1: key j visible to query i iff j <= i).

Unlike the C oracle, it materialises the whole masked score matrix with -inf
entries and forms the full weight matrix before multiplying by V, so the two
implementations share neither structure nor association order.
"""
from __future__ import annotations

import math
from typing import List, Optional, Sequence

Matrix = List[List[float]]


def _scores(Q: Matrix, K: Matrix, scale: float, causal: bool, window: int = 0) -> Matrix:
    n_q, n_k = len(Q), len(K)
    S = [[0.0] * n_k for _ in range(n_q)]
    for i in range(n_q):
        for j in range(n_k):
            # causal: j <= i; a sliding window W also needs j >= i - W + 1
            if (causal and j > i) or (window > 0 and j < i - window + 1):
                S[i][j] = -math.inf
            else:
                S[i][j] = math.fsum(a * b for a, b in zip(Q[i], K[j])) * scale
    return S


def _softmax_rows(S: Matrix) -> Matrix:
    A = []
    for row in S:
        top = max(row)
        e = [0.0 if x == -math.inf else math.exp(x - top) for x in row]
        z = math.fsum(e)
        A.append([x / z for x in e])
    return A


def diff_attention(Q1: Matrix, K1: Matrix, Q2: Matrix, K2: Matrix, V: Matrix, lam: float,
                   *, causal: bool, scale: Optional[float] = None, norm: bool = False,
                   gamma: Optional[Sequence[float]] = None, eps: float = 1e-5,
                   lambda_init: float = 0.0, window: int = 0) -> Matrix:
    """One head. Q*, K* are [n, d_qk] lists; V is [n, d_v]. Returns [n, d_v].
    window > 0 (with causal) keeps keys i - window + 1 .. i of row i."""
    d = len(Q1[0])
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    A1 = _softmax_rows(_scores(Q1, K1, scale, causal, window))
    A2 = _softmax_rows(_scores(Q2, K2, scale, causal, window))
    W = [[a - lam * b for a, b in zip(r1, r2)] for r1, r2 in zip(A1, A2)]
    d_v = len(V[0])
    out = []
    for i in range(len(W)):
        row = [math.fsum(W[i][j] * V[j][c] for j in range(len(V))) for c in range(d_v)]
        if norm:
            if norm == "group":  # mean-subtracting variant, one group per head
                mu = math.fsum(row) / d_v
                row = [x - mu for x in row]
            rms = math.sqrt(math.fsum(x * x for x in row) / d_v + eps)
            row = [x / rms * gamma[c] * (1.0 - lambda_init) for c, x in enumerate(row)]
        out.append(row)
    return out


def lambda_init(depth: int) -> float:
    return 0.8 - 0.6 * math.exp(-0.3 * (depth - 1))


def lambda_value(lq1, lk1, lq2, lk2, depth: int) -> float:
    return (math.exp(math.fsum(a * b for a, b in zip(lq1, lk1)))
            - math.exp(math.fsum(a * b for a, b in zip(lq2, lk2))) + lambda_init(depth))
