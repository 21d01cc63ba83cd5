"""Pins of the gradient oracle (oracle/backward.py), CPU only.

The gradients are checked against central finite differences of the stdlib
brute-force forward (oracle/brute.py: fp64 Python floats, an implementation
that shares nothing with the gradient code), along random directions for
every input, and against invariants the definition fixes."""
import math

import numpy as np
import pytest

import oracle
from oracle import backward as bw
from oracle import brute


def rnd(rng, *shape, std=1.0):
    return rng.standard_normal(shape) * std


def _forward_brute(q1, q2, k1, k2, v, lam, gamma, *, causal, norm, depth, window, scale=None):
    """Whole-tensor forward through the brute-force oracle (per head)."""
    B, H, N, _ = q1.shape
    Hkv, dv = k1.shape[1], v.shape[3]
    out = np.zeros((B, H, N, dv))
    init = brute.lambda_init(depth)
    for b in range(B):
        for h in range(H):
            g = h // (H // Hkv)
            L = lambda x: x.tolist()
            out[b, h] = np.array(brute.diff_attention(
                L(q1[b, h]), L(k1[b, g]), L(q2[b, h]), L(k2[b, g]), L(v[b, g]), float(lam[h]),
                causal=causal, scale=scale, norm=norm, gamma=L(gamma[h]) if norm else None,
                lambda_init=init, window=window))
    return out


CASES = [
    dict(B=1, H=1, Hkv=1, N=5, dqk=3, dv=4, causal=True, norm=False, window=0),
    dict(B=1, H=2, Hkv=1, N=6, dqk=4, dv=3, causal=True, norm=True, window=0),
    dict(B=2, H=2, Hkv=2, N=4, dqk=2, dv=3, causal=False, norm=True, window=0),
    dict(B=1, H=2, Hkv=2, N=7, dqk=3, dv=2, causal=True, norm=False, window=3),
    dict(B=1, H=2, Hkv=1, N=6, dqk=3, dv=4, causal=True, norm="group", window=0),
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_gradients_match_finite_differences_of_brute_force(case):
    cfg = CASES[case]
    rng = np.random.default_rng(100 + case)
    B, H, Hkv, N, dqk, dv = (cfg[k] for k in ("B", "H", "Hkv", "N", "dqk", "dv"))
    x = {"q1": rnd(rng, B, H, N, dqk), "q2": rnd(rng, B, H, N, dqk), "k1": rnd(rng, B, Hkv, N, dqk),
         "k2": rnd(rng, B, Hkv, N, dqk), "v": rnd(rng, B, Hkv, N, dv),
         "lam": rng.uniform(0.1, 0.9, H), "gamma": rng.uniform(0.5, 1.5, (H, dv))}
    dout = rnd(rng, B, H, N, dv)
    kw = dict(causal=cfg["causal"], norm=cfg["norm"], depth=5, window=cfg["window"])
    g = bw.prefill_backward(x["q1"], x["q2"], x["k1"], x["k2"], x["v"], x["lam"], dout,
                            gamma=x["gamma"], **kw)
    grads = {"q1": g["dq1"], "q2": g["dq2"], "k1": g["dk1"], "k2": g["dk2"], "v": g["dv"],
             "lam": g["dlambda"], "gamma": g["dgamma"]}
    eps = 1e-6
    for name in grads:
        if name == "gamma" and not cfg["norm"]:
            assert np.all(grads[name] == 0)
            continue
        d = rng.standard_normal(x[name].shape)
        xp = dict(x)
        xm = dict(x)
        xp[name] = x[name] + eps * d
        xm[name] = x[name] - eps * d
        fp = (_forward_brute(xp["q1"], xp["q2"], xp["k1"], xp["k2"], xp["v"], xp["lam"], xp["gamma"], **kw)
              * dout).sum()
        fm = (_forward_brute(xm["q1"], xm["q2"], xm["k1"], xm["k2"], xm["v"], xm["lam"], xm["gamma"], **kw)
              * dout).sum()
        fd = (fp - fm) / (2 * eps)
        an = float((grads[name] * d).sum())
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(fd)), (name, fd, an)


def test_saved_forward_statistics():
    # o1 - lambda o2 (normed) is the C oracle's output; exp(s - lse) sums to 1 per row
    rng = np.random.default_rng(7)
    B, H, Hkv, N, dqk, dv = 1, 2, 1, 9, 4, 5
    q1, q2 = rnd(rng, B, H, N, dqk), rnd(rng, B, H, N, dqk)
    k1, k2 = rnd(rng, B, Hkv, N, dqk), rnd(rng, B, Hkv, N, dqk)
    v = rnd(rng, B, Hkv, N, dv)
    lam = np.array([0.3, 0.7])
    gamma = rng.uniform(0.9, 1.1, (H, dv))
    g = bw.prefill_backward(q1, q2, k1, k2, v, lam, np.zeros((B, H, N, dv)), depth=3, causal=True,
                            norm=True, gamma=gamma)
    f32 = lambda a: a.astype(np.float32)
    ref = oracle.prefill(f32(q1), f32(q2), f32(k1), f32(k2), f32(v), lam, depth=3, causal=True, norm=True,
                         gamma=f32(gamma))
    # the C oracle saw fp32-rounded inputs: compare at that precision
    y = g["o1"] - lam[None, :, None, None] * g["o2"]
    r = 1.0 / np.sqrt((y * y).mean(axis=-1, keepdims=True) + 1e-5)
    z = y * r * gamma[None, :, None, :] * (1 - oracle.lambda_init(3))
    np.testing.assert_allclose(z, ref, rtol=0, atol=1e-5)
    s1 = np.einsum("bhnd,bmd->bhnm", q1, k1[:, 0]) / math.sqrt(dqk)
    mask = np.tril(np.ones((N, N), bool))
    tot = np.where(mask, np.exp(s1 - g["lse1"][..., None]), 0.0).sum(axis=-1)
    np.testing.assert_allclose(tot, 1.0, rtol=0, atol=1e-13)


def test_lambda_zero_leaves_branch_two_without_gradient():
    rng = np.random.default_rng(8)
    B, H, N, d = 1, 1, 6, 3
    args = [rnd(rng, B, H, N, d) for _ in range(4)] + [rnd(rng, B, H, N, 4)]
    g = bw.prefill_backward(*args, np.array([0.0]), rnd(rng, B, H, N, 4), depth=1, causal=True, norm=False)
    assert np.all(g["dq2"] == 0) and np.all(g["dk2"] == 0)


def test_gqa_key_gradient_sums_over_the_group():
    # two heads sharing one KV head: dK equals the sum of each head alone
    rng = np.random.default_rng(9)
    N, d, dv = 5, 3, 4
    q1, q2 = rnd(rng, 1, 2, N, d), rnd(rng, 1, 2, N, d)
    k1, k2, v = rnd(rng, 1, 1, N, d), rnd(rng, 1, 1, N, d), rnd(rng, 1, 1, N, dv)
    lam, dout = np.array([0.2, 0.6]), rnd(rng, 1, 2, N, dv)
    g = bw.prefill_backward(q1, q2, k1, k2, v, lam, dout, depth=2, causal=True, norm=False)
    parts = [bw.prefill_backward(q1[:, h:h + 1], q2[:, h:h + 1], k1, k2, v, lam[h:h + 1], dout[:, h:h + 1],
                                 depth=2, causal=True, norm=False) for h in range(2)]
    for name in ("dk1", "dk2", "dv"):
        np.testing.assert_allclose(g[name], parts[0][name] + parts[1][name], rtol=1e-13, atol=1e-13)


def test_lambda_vector_gradients_match_finite_differences():
    rng = np.random.default_rng(10)
    H, dl = 3, 5
    vec = [rnd(rng, H, dl, std=0.3) for _ in range(4)]
    dlam = rnd(rng, H)
    g = bw.lambda_backward(*vec, dlam)
    eps = 1e-6
    for i, name in enumerate(("dlq1", "dlk1", "dlq2", "dlk2")):
        d = rnd(rng, H, dl)
        vp = [x.copy() for x in vec]
        vm = [x.copy() for x in vec]
        vp[i] += eps * d
        vm[i] -= eps * d
        f = lambda vs: sum(dlam[h] * brute.lambda_value(*(x[h].tolist() for x in vs), 4) for h in range(H))
        fd = (f(vp) - f(vm)) / (2 * eps)
        assert abs(fd - float((g[name] * d).sum())) <= 1e-7 * max(1.0, abs(fd)), name
