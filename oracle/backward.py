"""Gradients of differential attention, fp64. TEST INFRASTRUCTURE ONLY.

Only ``tests/`` import this module. It shares no code with the HIP path.

The function differentiated is the forward the C oracle computes (lesson
"Differential Attention (V2)", section "Concept": two softmax maps of scaled
scores, their difference weighted by lambda times V; section "V1 vs V2": the
V1 per-head RMSNorm; lesson "Attention Variants", "Build it", steps 1 and 2:
the causal mask and the causal sliding window). The pages give no backward;
this module applies the chain rule to that definition step by step, in the
forward's own order reversed, with every N x N map materialised (small and
medium shapes only):

  forward, per (batch b, output head h, KV head g):
    S_k = Q_k K_k^T * scale (masked to -inf)      k = 1, 2
    A_k = softmax(S_k) per row
    O_k = A_k V
    y   = O_1 - lambda O_2
    V1: z = y * r * gamma * c,  r = 1/sqrt(mean(y^2) + eps), c = 1 - lambda_init
        (GroupNorm variant: y - mean(y) in place of y, its variance in r)
  backward, given dz:
    V1: dgamma += sum_rows dz * y * r * c
        dy = c r (gamma dz) - y r^3 / d_v * sum_c(c gamma dz y)
    dlambda = -sum(dy * O_2)
    dO_1 = dy, dO_2 = -lambda dy
    dV += A_1^T dO_1 + A_2^T dO_2
    dA_k = dO_k V^T;  dS_k = A_k * (dA_k - rowsum(dA_k * A_k))
    dQ_k = scale dS_k K_k;  dK_k += scale dS_k^T Q_k
  and for lambda = exp(lq1.lk1) - exp(lq2.lk2) + lambda_init:
    dlq1 = dlambda exp(lq1.lk1) lk1,  dlk1 = dlambda exp(lq1.lk1) lq1,
    dlq2 = -dlambda exp(lq2.lk2) lk2, dlk2 = -dlambda exp(lq2.lk2) lq2.

Parity status: pinned by central finite differences of the C oracle's forward
(an independent implementation) along random directions, per input; and by
invariants the mathematics fixes (tests/test_oracle_backward.py).
"""
from __future__ import annotations

import math
from typing import Dict, Optional

import numpy as np


def _lambda_init(depth: int) -> float:
    return 0.8 - 0.6 * math.exp(-0.3 * (depth - 1))


def prefill_backward(q1, q2, k1, k2, v, lam, dout, *, depth: int, causal: bool, norm: bool,
                     gamma=None, eps: float = 1e-5, scale: Optional[float] = None,
                     window: int = 0) -> Dict[str, np.ndarray]:
    """Gradients of the prefill output w.r.t. its inputs, given dout (the
    gradient of the output). Shapes as oracle.prefill; dout [B, H, N, d_v].
    Returns dq1, dq2 [B, H, N, d_qk]; dk1, dk2 [B, H_kv, N, d_qk];
    dv [B, H_kv, N, d_v]; dlambda [H]; dgamma [H, d_v] (zeros without norm);
    the forward's per-branch normalised outputs o1, o2 [B, H, N, d_v] and
    natural-log log-sum-exp of the scaled scores lse1, lse2 [B, H, N]; and dy
    [B, H, N, d_v], the gradient at y = O_1 - lambda O_2 (dout itself without
    a norm), whose products with O_2 dlambda sums."""
    f = lambda a: np.asarray(a, np.float64)
    q1, q2, k1, k2, v, dout = (f(x) for x in (q1, q2, k1, k2, v, dout))
    lam = f(lam).reshape(-1)
    B, H, N, dqk = q1.shape
    Hkv, dv_ = k1.shape[1], v.shape[3]
    group = H // Hkv
    if scale is None:
        scale = 1.0 / math.sqrt(dqk)
    c = 1.0 - _lambda_init(depth)
    g = f(gamma).reshape(H, dv_) if norm else None

    i = np.arange(N)[:, None]
    j = np.arange(N)[None, :]
    visible = np.ones((N, N), bool)
    if causal:
        visible &= j <= i
    if window > 0:
        visible &= j >= i - window + 1

    out = {name: np.zeros_like(x) for name, x in (("dq1", q1), ("dq2", q2), ("dk1", k1), ("dk2", k2),
                                                    ("dv", v))}
    out["dlambda"] = np.zeros(H)
    out["dgamma"] = np.zeros((H, dv_))
    out["o1"] = np.zeros((B, H, N, dv_))
    out["o2"] = np.zeros((B, H, N, dv_))
    out["dy"] = np.zeros((B, H, N, dv_))
    out["lse1"] = np.zeros((B, H, N))
    out["lse2"] = np.zeros((B, H, N))

    def softmax(s):
        s = np.where(visible, s, -np.inf)
        m = s.max(axis=1, keepdims=True)
        e = np.exp(s - m)
        z = e.sum(axis=1, keepdims=True)
        return e / z, (m + np.log(z))[:, 0]

    for b in range(B):
        for h in range(H):
            kv = h // group
            s1 = q1[b, h] @ k1[b, kv].T * scale
            s2 = q2[b, h] @ k2[b, kv].T * scale
            a1, lse1 = softmax(s1)
            a2, lse2 = softmax(s2)
            o1 = a1 @ v[b, kv]
            o2 = a2 @ v[b, kv]
            y = o1 - lam[h] * o2
            out["o1"][b, h], out["o2"][b, h] = o1, o2
            out["lse1"][b, h], out["lse2"][b, h] = lse1, lse2

            dz = dout[b, h]
            if norm == "group":
                # z = (y - mean y) r gamma c with r = 1/sqrt(var + eps):
                # with u = y - mean y and gd = c gamma dz,
                # dy = r (gd - mean(gd)) - u r^3 mean(gd u)
                u = y - y.mean(axis=1, keepdims=True)
                r = 1.0 / np.sqrt((u * u).mean(axis=1, keepdims=True) + eps)
                out["dgamma"][h] += (dz * u * r * c).sum(axis=0)
                gd = c * g[h][None, :] * dz
                dy = r * (gd - gd.mean(axis=1, keepdims=True)) - u * r ** 3 * (gd * u).mean(axis=1, keepdims=True)
            elif norm:
                r = 1.0 / np.sqrt((y * y).mean(axis=1, keepdims=True) + eps)
                out["dgamma"][h] += (dz * y * r * c).sum(axis=0)
                gd = c * g[h][None, :] * dz
                dy = r * gd - y * r ** 3 / dv_ * (gd * y).sum(axis=1, keepdims=True)
            else:
                dy = dz
            out["dy"][b, h] = dy
            out["dlambda"][h] += -(dy * o2).sum()
            do1, do2 = dy, -lam[h] * dy
            out["dv"][b, kv] += a1.T @ do1 + a2.T @ do2
            for a, do, q, k, dq, dk in ((a1, do1, q1, k1, "dq1", "dk1"), (a2, do2, q2, k2, "dq2", "dk2")):
                da = do @ v[b, kv].T
                ds = a * (da - (da * a).sum(axis=1, keepdims=True))
                out[dq][b, h] += scale * ds @ k[b, kv]
                out[dk][b, kv] += scale * ds.T @ q[b, h]
    return out


def lambda_backward(lq1, lk1, lq2, lk2, dlambda) -> Dict[str, np.ndarray]:
    """Gradients of lambda = exp(lq1.lk1) - exp(lq2.lk2) + lambda_init w.r.t.
    the four [H, d_l] vectors, given dlambda [H]."""
    lq1, lk1, lq2, lk2 = (np.asarray(x, np.float64) for x in (lq1, lk1, lq2, lk2))
    d = np.asarray(dlambda, np.float64).reshape(-1, 1)
    e1 = np.exp((lq1 * lk1).sum(axis=1, keepdims=True))
    e2 = np.exp((lq2 * lk2).sum(axis=1, keepdims=True))
    return {"dlq1": d * e1 * lk1, "dlk1": d * e1 * lq1, "dlq2": -d * e2 * lk2, "dlk2": -d * e2 * lq2}
