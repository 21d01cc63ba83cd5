"""GPU parity of the backward pass (and of the statistics the forward stores
for it) against the fp64 gradient oracle (oracle/backward.py), through the C ABI.

Tolerance for gradients: each gradient tensor's relative Frobenius error
<= 5e-3 and max |error| <= 2e-2 of its largest magnitude. The path rounds the
output gradient after the norm and the score gradients to bf16 (8 significant
bits, a relative error of at most 2^-9 = 2.0e-3 per rounding, about 1.1e-3 on
average) before the products, as the forward rounds the probabilities;
accumulation is fp32. A gradient element sums many such rounded terms, so
its error is about one rounding's worth of its size (measured 2.4e-3
relative Frobenius at most); 5e-3 leaves room for the largest of the
workloads, and a dropped term or key moves the error far beyond it. The
stored log-sum-exp must match to 1e-4 of max(1, |lse|): the forward sums the
unrounded fp32 probabilities for it (the bf16-rounded sum that normalises the
output would be off by up to ln(1 + 2^-9) = 1.95e-3), so what is left is the
fp32 arithmetic of the scores and the sum; a key dropped from a row of N keys
moves it by about ln(1 + 1/N) (5e-3 at N 200). dgamma (a sum over all
rows): relative error <= 1e-2. dlambda = -sum(dy o_2) over every row and
channel of a head: products that cancel heavily (their absolute sum is
10^2-10^3 times the result, so a relative bound on the result does not fit
it). Each product carries the bf16 rounding of the probabilities in o_2,
directly and through dy (the norm's backward), about 2^-8 of its size, and
such errors add like a random walk: to about 2^-8 times the l2 norm of the
products (the rounding of the probabilities alone, emulated on the CPU,
moves dlambda by up to 5.2e-3 of that norm; measured on the GPU up to
4.9e-3). The bound is 2^-6 of that norm per head; dropping a block of rows
or a branch moves dlambda far beyond it. The lambda-vector gradients (fp32
only): 1e-5 relative."""
import numpy as np
import pytest

import oracle
import workloads as W
from gpu_util import PrefillCase, check, dev, say, to_dev
from oracle import backward as bw

pytestmark = pytest.mark.gpu

GRAD_REL_FRO = 5e-3
DLAMBDA_OF_TERMS = 2.0 ** -6
GRAD_MAX_REL = 2e-2
LSE_REL = 1e-4


@pytest.fixture(scope="module")
def torch():
    import torch as t
    assert t.cuda.is_available()
    return t


@pytest.fixture(scope="module")
def da():
    import differential_attention_amd as m
    m.load_library()
    return m


def _case(form, N, causal, B=1, seed=0, H=None):
    if form == "v1":
        return W.prefill_v1(seed=seed, B=B, H=H or 2, N=N, causal=causal)
    return W.prefill_v2(seed=seed, B=B, H=H or 4, H_kv=2, N=N, causal=causal)


def _grad_check(got, ref, what, zero_scale=None):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite"
    err = got - ref
    if zero_scale is not None:
        # a gradient that is zero by construction: bounded by rounding noise
        # relative to the scale of the inputs that would otherwise feed it
        mx = float(np.abs(got).max()) / zero_scale
        say(f"  {what}: zero by construction, max|got| / scale {mx:.3e}")
        assert mx <= 1e-3, (what, mx)
        return
    fro = float(np.linalg.norm(err) / max(np.linalg.norm(ref), 1e-30))
    mx = float(np.abs(err).max() / max(np.abs(ref).max(), 1e-30))
    say(f"  {what}: rel-fro {fro:.3e} max/max|ref| {mx:.3e}")
    assert fro <= GRAD_REL_FRO, (what, fro)
    assert mx <= GRAD_MAX_REL, (what, mx)


def _terms_l2(ref):
    """Per head: the l2 norm of the products dy o_2 that dlambda sums."""
    return np.sqrt(((ref["dy"] * ref["o2"]) ** 2).sum(axis=(0, 2, 3)))


def _dlambda_check(got, ref, terms_l2):
    err = np.abs(np.asarray(got, np.float64) - ref)
    say(f"  dlambda: max |error| / l2 of its terms {float((err / terms_l2).max()):.3e}")
    assert np.all(err <= DLAMBDA_OF_TERMS * terms_l2 + 1e-6), (got, ref, terms_l2)


def _run(torch, da, p, window=0, seed=0):
    c = PrefillCase(p)
    stats = da.prefill_stats(c.q1, c.v)
    c.run(window=window, stats=stats)
    rng = np.random.default_rng(seed + 1000)
    dout_bits = W.f32_to_bf16(rng.standard_normal((p.B, p.H, p.N, p.d_v)).astype(np.float32))
    dout = to_dev(dout_bits, "bf16")
    g = da.backward(c.q1, c.q2, c.k1, c.k2, c.v, c.lam, stats, dout, depth=p.depth, causal=p.causal,
                    norm=p.norm, gamma=c.gamma, eps=p.eps, window=window)
    k1 = p.f32("k1")
    k2 = k1 if p.shared_k else p.f32("k2")
    ref = bw.prefill_backward(p.f32("q1"), p.f32("q2"), k1, k2, p.f32("v"), c.lam64, W.bf16_to_f32(dout_bits),
                              depth=p.depth, causal=p.causal, norm=p.norm, gamma=p.gamma, eps=p.eps,
                              window=window)
    return c, stats, g, ref


@pytest.mark.parametrize("form", ["v1", "v2"])
# (384, False) and (640, True, 300): whole tiles in the key blocks' unmasked
# middle stretch as well as masked ones at its ends (a window reaching over
# several tiles); the others: ragged ends, short windows and one-key windows
@pytest.mark.parametrize("N,causal,window", [(64, True, 0), (200, True, 0), (333, True, 0), (100, False, 0),
                                             (257, True, 40), (200, True, 1), (384, False, 0), (640, True, 300)])
def test_backward_parity(torch, da, form, N, causal, window):
    p = _case(form, N, causal, seed=N + window)
    say(f"backward {form} N {N} causal {causal} window {window}")
    c, stats, g, ref = _run(torch, da, p, window=window, seed=N)
    # the statistics the forward stored
    check(stats[0].cpu().numpy(), ref["o1"], "bf16", "o1")
    check(stats[1].cpu().numpy(), ref["o2"], "bf16", "o2")
    for k in (2, 3):
        r = ref["lse1" if k == 2 else "lse2"]
        d = float((np.abs(stats[k].cpu().numpy() - r) / np.maximum(1.0, np.abs(r))).max())
        say(f"  lse{k - 1}: max relative error {d:.3e}")
        assert d <= LSE_REL, ("lse", d)
    # with a window of one key each softmax is the constant 1, so the score
    # gradients, and with them dQ and dK, vanish identically (o_k = v_i)
    zs = float(np.abs(ref["dv"]).max()) if window == 1 else None
    for name in ("dq1", "dq2", "dv"):
        _grad_check(g[name].cpu().numpy(), ref[name], name, zs if name != "dv" else None)
    if p.shared_k:
        _grad_check(g["dk1"].cpu().numpy(), ref["dk1"] + ref["dk2"], "dk (shared)", zs)
    else:
        _grad_check(g["dk1"].cpu().numpy(), ref["dk1"], "dk1", zs)
        _grad_check(g["dk2"].cpu().numpy(), ref["dk2"], "dk2", zs)
    _dlambda_check(g["dlambda"].cpu().numpy(), ref["dlambda"], _terms_l2(ref))
    if p.norm:
        dg = g["dgamma"].cpu().numpy()
        assert np.linalg.norm(dg - ref["dgamma"]) <= 1e-2 * np.linalg.norm(ref["dgamma"])


@pytest.mark.parametrize("N,window", [(200, 0), (333, 100)])
def test_backward_d128_separate_keys(torch, da, N, window):
    # d_qk 128 with two key tensors (the kernels' non-shared d 128 form: each
    # branch reads its own key and transposed-key fragments)
    p = W.prefill_v2(seed=40 + N, B=1, H=4, H_kv=2, N=N, causal=True)
    rng = np.random.default_rng(41 + N)
    p.k2 = W.f32_to_bf16(rng.standard_normal(p.k1.shape).astype(np.float32))
    p.shared_k = False
    say(f"backward V2 shape, separate K1 and K2, N {N} window {window}")
    _, _, g, ref = _run(torch, da, p, window=window, seed=N)
    for name in ("dq1", "dq2", "dk1", "dk2", "dv"):
        _grad_check(g[name].cpu().numpy(), ref[name], name)
    _dlambda_check(g["dlambda"].cpu().numpy(), ref["dlambda"], _terms_l2(ref))


def test_backward_gqa_groups(torch, da):
    # 8 heads over 2 KV heads (4 heads per KV head accumulate into one dK, dV)
    p = W.prefill_v2(seed=5, B=2, H=8, H_kv=2, N=150)
    say("backward V2 8/2 heads, B 2, N 150")
    _, _, g, ref = _run(torch, da, p, seed=5)
    _grad_check(g["dk1"].cpu().numpy(), ref["dk1"] + ref["dk2"], "dk (shared, GQA)")
    _grad_check(g["dv"].cpu().numpy(), ref["dv"], "dv (GQA)")
    _grad_check(g["dq2"].cpu().numpy(), ref["dq2"], "dq2 (GQA)")


def test_backward_is_deterministic(torch, da):
    p = _case("v1", 300, True, seed=9)
    c = PrefillCase(p)
    stats = da.prefill_stats(c.q1, c.v)
    c.run(stats=stats)
    dout = to_dev(W.f32_to_bf16(np.ones((p.B, p.H, p.N, p.d_v), np.float32)), "bf16")
    g1 = da.backward(c.q1, c.q2, c.k1, c.k2, c.v, c.lam, stats, dout, depth=p.depth, norm=True, gamma=c.gamma)
    g2 = da.backward(c.q1, c.q2, c.k1, c.k2, c.v, c.lam, stats, dout, depth=p.depth, norm=True, gamma=c.gamma)
    for k in g1:
        if g1[k] is not None:
            assert torch.equal(g1[k], g2[k]), k


def test_backward_general_copy_paths_are_bitwise_equal(torch, da):
    # Both backward kernels copy whole tiles with buffer loads when the two
    # query (or key) tensors share their strides; otherwise every tile goes
    # through per-lane addresses. Same bytes in LDS: bitwise-equal gradients.
    p = _case("v1", 300, True, seed=23)
    c = PrefillCase(p)
    stats = da.prefill_stats(c.q1, c.v)
    c.run(stats=stats)
    rng = np.random.default_rng(23)
    dout = to_dev(W.f32_to_bf16(rng.standard_normal((p.B, p.H, p.N, p.d_v)).astype(np.float32)), "bf16")
    kw = dict(depth=p.depth, causal=True, norm=True, gamma=c.gamma, eps=p.eps)
    g1 = da.backward(c.q1, c.q2, c.k1, c.k2, c.v, c.lam, stats, dout, **kw)
    g1 = {k: (x.clone() if x is not None else None) for k, x in g1.items()}

    def wide(x, extra=64):
        w = torch.zeros(x.shape[:3] + (x.shape[3] + extra,), dtype=x.dtype, device=x.device)
        w[..., :x.shape[3]] = x
        return w[..., :x.shape[3]]

    say("backward V1, N 300: Q2 and K2 rows 64 elements longer than Q1's and K1's")
    g2 = da.backward(c.q1, wide(c.q2), c.k1, wide(c.k2), c.v, c.lam, stats, dout, **kw)
    for k in g1:
        if g1[k] is not None:
            assert torch.equal(g1[k], g2[k]), k


def test_lambda_backward(torch, da):
    rng = np.random.default_rng(3)
    H, dl = 5, 64
    vec = [(rng.standard_normal((H, dl)) * 0.1).astype(np.float32) for _ in range(4)]
    dlam = rng.standard_normal(H).astype(np.float32)
    got = da.lambda_backward(*(torch.from_numpy(x).to(dev()) for x in vec), torch.from_numpy(dlam).to(dev()))
    ref = bw.lambda_backward(*vec, dlam)
    for k in ref:
        np.testing.assert_allclose(got[k].cpu().numpy(), ref[k], rtol=1e-5, atol=1e-7)


def test_backward_prefill_v1_shape_sampled_heads(torch, da):
    # the prefill_v1 shape (B 2, H 16, N 4096, V1, RMS): gradients of two heads
    # compared in full (the oracle materialises their 4096 x 4096 maps)
    p = W.prefill_v1()
    c = PrefillCase(p)
    stats = da.prefill_stats(c.q1, c.v)
    c.run(stats=stats)
    rng = np.random.default_rng(77)
    dout_bits = W.f32_to_bf16(rng.standard_normal((p.B, p.H, p.N, p.d_v)).astype(np.float32))
    g = da.backward(c.q1, c.q2, c.k1, c.k2, c.v, c.lam, stats, to_dev(dout_bits, "bf16"), depth=p.depth,
                    norm=True, gamma=c.gamma, eps=p.eps)
    for b, h in ((0, 3), (1, 14)):
        say(f"backward prefill_v1 shape, head (b {b}, h {h})")
        sl = lambda x: x[b:b + 1, h:h + 1]
        ref = bw.prefill_backward(sl(p.f32("q1")), sl(p.f32("q2")), sl(p.f32("k1")), sl(p.f32("k2")),
                                  sl(p.f32("v")), c.lam64[h:h + 1], sl(W.bf16_to_f32(dout_bits)), depth=p.depth,
                                  causal=True, norm=True, gamma=p.gamma[h:h + 1], eps=p.eps)
        for name in ("dq1", "dq2", "dk1", "dk2", "dv"):
            _grad_check(sl(g[name].cpu().numpy()), ref[name], f"{name} (b {b}, h {h})")


@pytest.mark.parametrize("form", ["v1", "v2"])
def test_backward_group_norm(torch, da, form):
    p = _case(form, 200, True, seed=41)
    if not p.norm:
        p.gamma = np.random.default_rng(41).uniform(0.9, 1.1, (p.H, p.d_v)).astype(np.float32)
    p.norm = "group"
    say(f"backward {form} GroupNorm")
    _, _, g, ref = _run(torch, da, p, seed=41)
    for name in ("dq1", "dq2", "dv"):
        _grad_check(g[name].cpu().numpy(), ref[name], name)
    dg = g["dgamma"].cpu().numpy()
    assert np.linalg.norm(dg - ref["dgamma"]) <= 1e-2 * np.linalg.norm(ref["dgamma"])
    _dlambda_check(g["dlambda"].cpu().numpy(), ref["dlambda"], _terms_l2(ref))


# ---------------------------------------------------------------- full-size gradients


def _scalar_check(got, ref, what, tol=1e-2):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    err = float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30))
    say(f"  {what}: relative error {err:.3e}")
    assert err <= tol, (what, err)


def test_backward_prefill_v1_all_heads(torch, da):
    # every head of the prefill_v1 shape, and dlambda / dgamma, which sum over
    # all rows of all batches
    p = W.prefill_v1()
    c = PrefillCase(p)
    stats = da.prefill_stats(c.q1, c.v)
    c.run(stats=stats)
    rng = np.random.default_rng(78)
    dout_bits = W.f32_to_bf16(rng.standard_normal((p.B, p.H, p.N, p.d_v)).astype(np.float32))
    g = da.backward(c.q1, c.q2, c.k1, c.k2, c.v, c.lam, stats, to_dev(dout_bits, "bf16"), depth=p.depth,
                    norm=True, gamma=c.gamma, eps=p.eps)
    got = {k: g[k].cpu().numpy() for k in ("dq1", "dq2", "dk1", "dk2", "dv", "dlambda", "dgamma")}
    f = {k: p.f32(k) for k in ("q1", "q2", "k1", "k2", "v")}
    dout = W.bf16_to_f32(dout_bits)
    ref = {k: np.zeros_like(got[k], np.float64) for k in got}
    t2 = np.zeros(p.H)
    for b in range(p.B):
        for h in range(p.H):
            sl = lambda x: x[b:b + 1, h:h + 1]
            r = bw.prefill_backward(sl(f["q1"]), sl(f["q2"]), sl(f["k1"]), sl(f["k2"]), sl(f["v"]),
                                    c.lam64[h:h + 1], sl(dout), depth=p.depth, causal=True, norm=True,
                                    gamma=p.gamma[h:h + 1], eps=p.eps)
            for k in ("dq1", "dq2", "dk1", "dk2", "dv"):
                ref[k][b, h] = r[k][0, 0]
            ref["dlambda"][h] += r["dlambda"][0]
            t2[h] += _terms_l2(r)[0] ** 2
            ref["dgamma"][h] += r["dgamma"][0]
            say(f"  oracle head (b {b}, h {h}) done", live=True)
    for k in ("dq1", "dq2", "dk1", "dk2", "dv"):
        _grad_check(got[k], ref[k], f"{k} all heads")
    _dlambda_check(got["dlambda"], ref["dlambda"], np.sqrt(t2))
    _scalar_check(got["dgamma"], ref["dgamma"], "dgamma")


def test_backward_prefill_v2_sampled_heads(torch, da):
    # the prefill_v2 shape (GQA, N 16384): dQ of two heads, and dK, dV of one KV
    # head (the oracle sums its 4 output heads' contributions)
    p = W.prefill_v2()
    c = PrefillCase(p)
    stats = da.prefill_stats(c.q1, c.v)
    c.run(stats=stats)
    rng = np.random.default_rng(79)
    dout_bits = W.f32_to_bf16(rng.standard_normal((p.B, p.H, p.N, p.d_v)).astype(np.float32))
    g = da.backward(c.q1, c.q2, c.k1, c.k2, c.v, c.lam, stats, to_dev(dout_bits, "bf16"), depth=p.depth,
                    norm=False)
    q1, q2, k, v = p.f32("q1"), p.f32("q2"), p.f32("k1"), p.f32("v")
    dout = W.bf16_to_f32(dout_bits)
    grp = p.H // p.H_kv
    kvh = 5
    heads = list(range(kvh * grp, (kvh + 1) * grp))
    dk = np.zeros((p.N, p.d_qk))
    dv = np.zeros((p.N, p.d_v))
    for h in heads:
        r = bw.prefill_backward(q1[:, h:h + 1], q2[:, h:h + 1], k[:, kvh:kvh + 1], k[:, kvh:kvh + 1],
                                v[:, kvh:kvh + 1], c.lam64[h:h + 1], dout[:, h:h + 1], depth=p.depth,
                                causal=True, norm=False)
        dk += r["dk1"][0, 0] + r["dk2"][0, 0]
        dv += r["dv"][0, 0]
        if h in (heads[0], heads[-1]):
            _grad_check(g["dq1"][:, h:h + 1].cpu().numpy(), r["dq1"], f"dq1 head {h}")
            _grad_check(g["dq2"][:, h:h + 1].cpu().numpy(), r["dq2"], f"dq2 head {h}")
        say(f"  oracle head {h} done", live=True)
    # shared keys: the library returns the summed key gradient in dk1
    _grad_check(g["dk1"][0, kvh].cpu().numpy(), dk, f"dk KV head {kvh}")
    _grad_check(g["dv"][0, kvh].cpu().numpy(), dv, f"dv KV head {kvh}")
