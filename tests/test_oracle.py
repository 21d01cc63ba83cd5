"""Pins for the CPU oracle (no GPU).

Each test ties the fp64 oracle to something other than itself: a closed form,
an exact special case, a library routine (torch's scaled-dot-product attention
in fp64), an independent stdlib brute force, an invariant the mathematics
fixes, or the mask figure printed on the lesson "Attention Variants".
They are chosen so that a dropped term, a wrong sign, a swapped branch, a
transposed operand or a wrong head/page index fails at least one of them.
"""
import math
import os

import numpy as np
import pytest

import oracle
from oracle import brute

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rnd(rng, *shape, std=1.0):
    return (rng.standard_normal(shape) * std).astype(np.float32)


def _prefill(q1, q2, k1, k2, v, lam, **kw):
    kw.setdefault("depth", 1)
    return oracle.prefill(q1, q2, k1, k2, v, np.asarray(lam, np.float64), **kw)


# --------------------------------------------------------------------------
# lambda_init and lambda (lesson "Differential Attention (V2)", section
# "Concept"; depth schedule from the integrator skill page)
# --------------------------------------------------------------------------


def test_lambda_init_depth_one_is_0p2():
    # exp(-0.3 * 0) = 1 exactly, so lambda_init(1) = 0.8 - 0.6 = 0.2
    assert abs(oracle.lambda_init(1) - 0.2) <= 1e-15


def test_lambda_init_limit_and_monotone():
    vals = [oracle.lambda_init(d) for d in range(1, 60)]
    assert all(b > a for a, b in zip(vals, vals[1:]))
    assert all(0.2 - 1e-15 <= x < 0.8 for x in vals)
    assert all(oracle.lambda_init(d) <= 0.8 for d in range(60, 500))
    # the schedule settles at 0.8, "a small positive number like 0.8"
    assert abs(oracle.lambda_init(100000) - 0.8) <= 1e-15
    # halfway point 0.5: exp(-0.3 (d-1)) = 1/2 at d - 1 = ln 2 / 0.3 = 2.31
    assert oracle.lambda_init(3) < 0.5 < oracle.lambda_init(4)


def test_lambda_exact_exponents():
    H, dl = 4, 8
    lq1 = np.zeros((H, dl), np.float32)
    lk1 = np.zeros((H, dl), np.float32)
    lq2 = np.zeros((H, dl), np.float32)
    lk2 = np.zeros((H, dl), np.float32)
    # head 0: all zero -> exp(0) - exp(0) + init = init exactly
    # head 1: lq1.lk1 = 0.5*2 + 0.25*(-4) + 1*1 = 1 -> e - 1 + init
    lq1[1, :3] = [0.5, 0.25, 1.0]
    lk1[1, :3] = [2.0, -4.0, 1.0]
    # head 2: second exponent ln-free: lq2.lk2 = 2 -> 1 - e^2 + init (negative)
    lq2[2, 0], lk2[2, 0] = 4.0, 0.5
    # head 3: the pairing matters: lq1 with lk1 (=0) and lq2 with lk2 (=0),
    # but lq1.lq2 = 3 and lk1.lk2 = 3, so a mixed-up pairing would not give init
    lq1[3, 0], lq2[3, 0] = 1.0, 3.0
    lk1[3, 1], lk2[3, 1] = 1.0, 3.0
    for depth in (1, 12, 20):
        init = oracle.lambda_init(depth)
        lam = oracle.lambda_(lq1, lk1, lq2, lk2, depth)
        assert lam[0] == init
        assert abs(lam[1] - (math.e - 1.0 + init)) <= 1e-15
        assert abs(lam[2] - (1.0 - math.e ** 2 + init)) <= 1e-14
        assert lam[2] < 0  # lambda can be negative
        assert lam[3] == init


def test_lambda_matches_brute():
    rng = np.random.default_rng(11)
    vec = [rnd(rng, 5, 16, std=0.3) for _ in range(4)]
    lam = oracle.lambda_(*vec, 7)
    for h in range(5):
        ref = brute.lambda_value(*(v[h].astype(np.float64).tolist() for v in vec), 7)
        assert abs(lam[h] - ref) <= 1e-14


# --------------------------------------------------------------------------
# prefill
# --------------------------------------------------------------------------


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("norm", [False, True])
@pytest.mark.parametrize("N,dqk,dv,H,Hkv", [(1, 3, 2, 2, 2), (5, 4, 3, 2, 1), (13, 8, 5, 4, 2)])
def test_prefill_matches_brute(causal, norm, N, dqk, dv, H, Hkv):
    rng = np.random.default_rng(100 + N + dqk + int(causal) + 2 * int(norm))
    B = 2
    q1, q2 = rnd(rng, B, H, N, dqk), rnd(rng, B, H, N, dqk)
    k1, k2 = rnd(rng, B, Hkv, N, dqk), rnd(rng, B, Hkv, N, dqk)
    v = rnd(rng, B, Hkv, N, dv)
    lams = np.array([-0.5, 0.0, 0.2, 0.8, 1.0, 1.5][:H], np.float64)
    if H > len(lams):
        lams = np.resize(lams, H)
    gamma = rng.uniform(0.9, 1.1, (H, dv)).astype(np.float32)
    depth = 5
    out = _prefill(q1, q2, k1, k2, v, lams, depth=depth, causal=causal, norm=norm, gamma=gamma)
    init = brute.lambda_init(depth)
    grp = H // Hkv
    for b in range(B):
        for h in range(H):
            g = h // grp
            ref = brute.diff_attention(
                q1[b, h].astype(np.float64).tolist(), k1[b, g].astype(np.float64).tolist(),
                q2[b, h].astype(np.float64).tolist(), k2[b, g].astype(np.float64).tolist(),
                v[b, g].astype(np.float64).tolist(), float(lams[h]), causal=causal, norm=norm,
                gamma=gamma[h].astype(np.float64).tolist(), lambda_init=init)
            np.testing.assert_allclose(out[b, h], np.array(ref), rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal", [True, False])
def test_lambda_zero_is_standard_attention(causal):
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(5)
    B, H, Hkv, N, d, dv = 2, 4, 2, 37, 16, 24
    q1, q2 = rnd(rng, B, H, N, d), rnd(rng, B, H, N, d)
    k1, k2 = rnd(rng, B, Hkv, N, d), rnd(rng, B, Hkv, N, d)
    v = rnd(rng, B, Hkv, N, dv)
    out = _prefill(q1, q2, k1, k2, v, np.zeros(H), causal=causal, norm=False)
    rep = H // Hkv
    tq = torch.from_numpy(q1).double()
    tk = torch.from_numpy(k1).double().repeat_interleave(rep, dim=1)
    tv = torch.from_numpy(v).double().repeat_interleave(rep, dim=1)
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal).numpy()
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-13)
    # and branch 2 is irrelevant at lambda = 0
    out2 = _prefill(q1, rnd(rng, B, H, N, d), k1, rnd(rng, B, Hkv, N, d), v, np.zeros(H),
                    causal=causal, norm=False)
    np.testing.assert_array_equal(out, out2)


@pytest.mark.parametrize("causal", [True, False])
def test_rows_sum_to_one_minus_lambda(causal):
    rng = np.random.default_rng(6)
    B, H, N, d = 1, 3, 29, 8
    q1, q2, k1, k2 = (rnd(rng, B, H, N, d, std=2.0) for _ in range(4))
    v = np.ones((B, H, N, 4), np.float32)
    lam = np.array([0.2, -0.7, 1.3])
    out = _prefill(q1, q2, k1, k2, v, lam, causal=causal, norm=False)
    for h in range(H):
        np.testing.assert_allclose(out[0, h], 1.0 - lam[h], rtol=0, atol=1e-14)


@pytest.mark.parametrize("norm", [False, True])
def test_identical_branches_lambda_one_is_exactly_zero(norm):
    rng = np.random.default_rng(7)
    B, H, N, d, dv = 2, 2, 33, 8, 16
    q, k, v = rnd(rng, B, H, N, d), rnd(rng, B, H, N, d), rnd(rng, B, H, N, dv)
    gamma = np.ones((H, dv), np.float32)
    out = _prefill(q, q, k, k, v, np.ones(H), causal=True, norm=norm, gamma=gamma)
    assert np.all(out == 0.0)


def test_branch_swap_symmetry():
    # (A1 - l A2) V = -l (A2 - (1/l) A1) V
    rng = np.random.default_rng(8)
    B, H, N, d, dv = 1, 2, 21, 8, 6
    q1, q2, k1, k2 = (rnd(rng, B, H, N, d) for _ in range(4))
    v = rnd(rng, B, H, N, dv)
    lam = np.array([0.37, -1.6])
    a = _prefill(q1, q2, k1, k2, v, lam, causal=True, norm=False)
    b = _prefill(q2, q1, k2, k1, v, 1.0 / lam, causal=True, norm=False)
    np.testing.assert_allclose(a, -lam[None, :, None, None] * b, rtol=0, atol=1e-13)


def test_linear_in_v_and_causal_row_zero():
    rng = np.random.default_rng(9)
    B, H, N, d, dv = 1, 2, 17, 8, 5
    q1, q2, k1, k2 = (rnd(rng, B, H, N, d) for _ in range(4))
    # values on a 1/64 grid so that 2 va - 3 vb is exact in fp32
    va = np.round(rnd(rng, B, H, N, dv) * 64) / np.float32(64)
    vb = np.round(rnd(rng, B, H, N, dv) * 64) / np.float32(64)
    lam = np.array([0.8, 0.25])
    oa = _prefill(q1, q2, k1, k2, va, lam, causal=True, norm=False)
    ob = _prefill(q1, q2, k1, k2, vb, lam, causal=True, norm=False)
    vc = (2.0 * va.astype(np.float64) - 3.0 * vb.astype(np.float64)).astype(np.float32)
    oc = _prefill(q1, q2, k1, k2, vc, lam, causal=True, norm=False)
    np.testing.assert_allclose(oc, 2.0 * oa - 3.0 * ob, rtol=0, atol=1e-12)
    # causal row 0 sees key 0 only: y0 = (1 - lambda) v0
    for h in range(H):
        np.testing.assert_allclose(oa[0, h, 0], (1 - lam[h]) * va[0, h, 0], rtol=0, atol=1e-15)


def test_rmsnorm_closed_form_and_scale_invariance():
    rng = np.random.default_rng(10)
    B, H, N, d, dv = 1, 2, 19, 8, 32
    q1, q2, k1, k2 = (rnd(rng, B, H, N, d) for _ in range(4))
    v = rnd(rng, B, H, N, dv)
    lam = np.array([0.5, 0.1])
    depth, eps = 12, 1e-5
    init = oracle.lambda_init(depth)
    o = _prefill(q1, q2, k1, k2, v, lam, depth=depth, causal=True, norm=False)
    y = _prefill(q1, q2, k1, k2, v, lam, depth=depth, causal=True, norm=True,
                 gamma=np.ones((H, dv), np.float32), eps=eps)
    ms = np.mean(o * o, axis=-1)
    rms_y = np.sqrt(np.mean(y * y, axis=-1))
    np.testing.assert_allclose(rms_y, (1 - init) * np.sqrt(ms / (ms + eps)), rtol=1e-13, atol=0)
    # direction preserved: y is a positive multiple of o
    np.testing.assert_allclose(y / np.linalg.norm(y, axis=-1, keepdims=True),
                               o / np.linalg.norm(o, axis=-1, keepdims=True), atol=1e-13)
    # scaling V by 64 leaves the normalised output unchanged up to eps
    y64 = _prefill(q1, q2, k1, k2, v * np.float32(64.0), lam, depth=depth, causal=True, norm=True,
                   gamma=np.ones((H, dv), np.float32), eps=0.0)
    y1 = _prefill(q1, q2, k1, k2, v, lam, depth=depth, causal=True, norm=True,
                  gamma=np.ones((H, dv), np.float32), eps=0.0)
    np.testing.assert_allclose(y64, y1, rtol=0, atol=1e-12)


def test_gqa_equals_repeated_kv_heads():
    rng = np.random.default_rng(12)
    B, H, Hkv, N, d, dv = 2, 8, 2, 15, 8, 6
    q1, q2 = rnd(rng, B, H, N, d), rnd(rng, B, H, N, d)
    k, v = rnd(rng, B, Hkv, N, d), rnd(rng, B, Hkv, N, dv)
    lam = rng.uniform(-1, 1, H)
    gqa = _prefill(q1, q2, k, k, v, lam, causal=True, norm=False)
    kr, vr = np.repeat(k, H // Hkv, axis=1), np.repeat(v, H // Hkv, axis=1)
    mha = _prefill(q1, q2, kr, kr, vr, lam, causal=True, norm=False)
    np.testing.assert_array_equal(gqa, mha)


def test_two_key_closed_form():
    # d = 1, scale 1: branch-1 scores (2, 0) -> weights (s(2), s(-2)) with s the
    # logistic function; branch-2 scores (0, 0) -> (1/2, 1/2).
    q1 = np.array([[[[1.0], [1.0]]]], np.float32)
    k1 = np.array([[[[2.0], [0.0]]]], np.float32)
    q2 = np.array([[[[1.0], [1.0]]]], np.float32)
    k2 = np.array([[[[0.0], [0.0]]]], np.float32)
    v = np.array([[[[3.0, 1.0], [-1.0, 5.0]]]], np.float32)
    lam = 0.6
    out = _prefill(q1, q2, k1, k2, v, [lam], causal=False, norm=False, scale=1.0)
    sig = 1.0 / (1.0 + math.exp(-2.0))
    w = np.array([sig - lam * 0.5, (1.0 - sig) - lam * 0.5])
    ref = w @ v[0, 0].astype(np.float64)
    np.testing.assert_allclose(out[0, 0, 0], ref, rtol=0, atol=1e-15)
    np.testing.assert_allclose(out[0, 0, 1], ref, rtol=0, atol=1e-15)


def _read_mask(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            rows.append([c == "x" for c in line.split()])
    return np.array(rows)


def test_causal_mask_matches_printed_figure():
    fig = _read_mask("causal_mask_8.txt")
    N = fig.shape[0]
    rng = np.random.default_rng(13)
    q1, q2, k1, k2 = (rnd(rng, 1, 1, N, 4) for _ in range(4))
    v = rnd(rng, 1, 1, N, 3)
    base = _prefill(q1, q2, k1, k2, v, [0.3], causal=True, norm=False)
    seen = np.zeros((N, N), bool)
    for j in range(N):
        kk, vv = k1.copy(), v.copy()
        kk[0, 0, j] += 1.0
        vv[0, 0, j] += 1.0
        out = _prefill(q1, q2, kk, k2, vv, [0.3], causal=True, norm=False)
        seen[:, j] = np.any(out[0, 0] != base[0, 0], axis=-1)
    np.testing.assert_array_equal(seen, fig)


def test_invalid_arguments_raise():
    z = np.zeros((1, 3, 4, 2), np.float32)
    with pytest.raises(ValueError):   # H not a multiple of H_kv
        oracle.prefill(z, z, np.zeros((1, 2, 4, 2), np.float32), np.zeros((1, 2, 4, 2), np.float32),
                       np.zeros((1, 2, 4, 2), np.float32), np.zeros(3), depth=1, causal=True, norm=False)


# --------------------------------------------------------------------------
# decode
# --------------------------------------------------------------------------


def _paged(k, v, page, rng, extra_pages=3):
    """Scatter contiguous [B, Hkv, L, d] keys/values into a shuffled page pool."""
    B, Hkv, L, d = k.shape
    dv = v.shape[-1]
    npg = (L + page - 1) // page
    P = B * npg + extra_pages
    perm = rng.permutation(P)
    table = np.full((B, npg + 2), -1, np.int32)
    kc = rnd(rng, P, Hkv, page, d)      # garbage everywhere not overwritten
    vc = rnd(rng, P, Hkv, page, dv)
    for b in range(B):
        for p in range(npg):
            phys = int(perm[b * npg + p])
            table[b, p] = phys
            n = min(page, L - p * page)
            kc[phys, :, :n] = k[b, :, p * page:p * page + n]
            vc[phys, :, :n] = v[b, :, p * page:p * page + n]
    return kc, vc, table


@pytest.mark.parametrize("L,page", [(1, 4), (13, 4), (16, 4), (37, 8)])
def test_decode_equals_last_prefill_row(L, page):
    rng = np.random.default_rng(20 + L)
    B, H, Hkv, d, dv = 2, 4, 2, 8, 6
    q1, q2 = rnd(rng, B, H, L, d), rnd(rng, B, H, L, d)
    k1, k2 = rnd(rng, B, Hkv, L, d), rnd(rng, B, Hkv, L, d)
    v = rnd(rng, B, Hkv, L, dv)
    lam = rng.uniform(-0.5, 1.2, H)
    gamma = rng.uniform(0.9, 1.1, (H, dv)).astype(np.float32)
    for norm in (False, True):
        pre = _prefill(q1, q2, k1, k2, v, lam, depth=9, causal=True, norm=norm, gamma=gamma)
        kc1, vc, table = _paged(k1, v, page, np.random.default_rng(1))
        kc2, _, _ = _paged(k2, v, page, np.random.default_rng(1))
        dec = oracle.decode(q1[:, :, -1], q2[:, :, -1], kc1, kc2, vc, table,
                            np.full(B, L, np.int32), lam, depth=9, norm=norm, gamma=gamma)
        np.testing.assert_allclose(dec, pre[:, :, -1], rtol=0, atol=1e-14)


@pytest.mark.parametrize("L,page,window", [(13, 4, 1), (13, 4, 5), (16, 4, 8), (37, 8, 9), (37, 8, 37),
                                           (37, 8, 100)])
def test_decode_window_equals_last_windowed_prefill_row(L, page, window):
    # the decode query is the last row of its sequence: with a window it sees
    # tokens L-W..L-1, the last row of the windowed prefill
    rng = np.random.default_rng(40 + L + window)
    B, H, Hkv, d, dv = 2, 2, 1, 8, 6
    q1, q2 = rnd(rng, B, H, L, d), rnd(rng, B, H, L, d)
    k1, k2 = rnd(rng, B, Hkv, L, d), rnd(rng, B, Hkv, L, d)
    v = rnd(rng, B, Hkv, L, dv)
    lam = rng.uniform(-0.5, 1.2, H)
    gamma = rng.uniform(0.9, 1.1, (H, dv)).astype(np.float32)
    pre = _prefill(q1, q2, k1, k2, v, lam, depth=9, causal=True, norm=True, gamma=gamma, window=window)
    kc1, vc, table = _paged(k1, v, page, np.random.default_rng(2))
    kc2, _, _ = _paged(k2, v, page, np.random.default_rng(2))
    dec = oracle.decode(q1[:, :, -1], q2[:, :, -1], kc1, kc2, vc, table, np.full(B, L, np.int32), lam,
                        depth=9, norm=True, gamma=gamma, window=window)
    np.testing.assert_allclose(dec, pre[:, :, -1], rtol=0, atol=1e-14)
    if window >= L:  # no token outside the window: the plain decode, bit for bit
        full = oracle.decode(q1[:, :, -1], q2[:, :, -1], kc1, kc2, vc, table, np.full(B, L, np.int32),
                             lam, depth=9, norm=True, gamma=gamma)
        assert np.array_equal(dec, full)


def test_decode_page_permutation_invariance_and_brute():
    rng = np.random.default_rng(30)
    B, H, Hkv, d, dv, page = 3, 2, 1, 4, 3, 4
    lens = [5, 12, 9]
    L = max(lens)
    k1, k2 = rnd(rng, B, Hkv, L, d), rnd(rng, B, Hkv, L, d)
    v = rnd(rng, B, Hkv, L, dv)
    q1, q2 = rnd(rng, B, H, d), rnd(rng, B, H, d)
    lam = np.array([0.4, 1.1])
    ctx = np.array(lens, np.int32)
    outs = []
    for seed in (1, 2):
        kc1, vc, table = _paged(k1, v, page, np.random.default_rng(seed))
        kc2, _, _ = _paged(k2, v, page, np.random.default_rng(seed))
        outs.append(oracle.decode(q1, q2, kc1, kc2, vc, table, ctx, lam, depth=3, norm=False))
    np.testing.assert_array_equal(outs[0], outs[1])
    for b in range(B):
        n = lens[b]
        for h in range(H):
            ref = brute.diff_attention([q1[b, h].astype(np.float64).tolist()],
                                       k1[b, 0, :n].astype(np.float64).tolist(),
                                       [q2[b, h].astype(np.float64).tolist()],
                                       k2[b, 0, :n].astype(np.float64).tolist(),
                                       v[b, 0, :n].astype(np.float64).tolist(), float(lam[h]),
                                       causal=False)
            np.testing.assert_allclose(outs[0][b, h], ref[0], rtol=0, atol=1e-13)


def test_decode_rejects_bad_page_id():
    rng = np.random.default_rng(31)
    kc = rnd(rng, 2, 1, 4, 4)
    vc = rnd(rng, 2, 1, 4, 2)
    q = rnd(rng, 1, 1, 4)
    table = np.array([[0, 5]], np.int32)   # page 5 does not exist
    with pytest.raises(ValueError):
        oracle.decode(q, q, kc, kc, vc, table, np.array([6], np.int32), [0.5], depth=1, norm=False)


# --------------------------------------------------------------------------
# the lesson's signal-plus-noise toy ("Build it", step 4; exercise on the
# lambda sweep): shared noise cancels, the planted signal survives
# --------------------------------------------------------------------------


def _toy(seed=0, N=1024, d=64, s=337):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal(d)
    qh = q / np.linalg.norm(q)
    u = rng.standard_normal(d)
    u -= (u @ qh) * qh
    u /= np.linalg.norm(u)
    noise = rng.standard_normal((N, d))
    k1 = noise.copy()
    k2 = noise.copy()
    k1[s] = math.sqrt(d) * (0.9 * qh + math.sqrt(0.19) * u)   # cosine 0.9, norm sqrt(d)
    f = lambda a: a.astype(np.float32)
    return f(q), f(k1), f(k2), s


def _toy_weights(q, k1, k2, lam):
    """Weights of one query over the N keys, read out through V = identity."""
    N, d = k1.shape
    page = 64
    P = N // page
    kc1 = k1.reshape(P, 1, page, d)
    kc2 = k2.reshape(P, 1, page, d)
    vc = np.eye(N, dtype=np.float32).reshape(P, 1, page, N)
    table = np.arange(P, dtype=np.int32)[None, :]
    qq = q.reshape(1, 1, d)
    return oracle.decode(qq, qq, kc1, kc2, vc, table, np.array([N], np.int32), [lam],
                         depth=1, norm=False)[0, 0]


def test_toy_noise_cancels_signal_survives():
    q, k1, k2, s = _toy()
    a1 = _toy_weights(q, k1, k2, 0.0)              # lambda = 0: plain softmax of branch 1
    ones = np.ones(k1.shape[0], bool)
    ones[s] = False
    # the two branches differ only at s, so on every noise key A1/A2 = Z2/Z1
    # (Z_b the branch's softmax normaliser) and lambda* = Z2/Z1 removes the noise
    a2 = a1 - _toy_weights(q, k1, k2, 1.0)          # A2 = A1 - (A1 - A2)
    ratio = a1[ones] / a2[ones]
    assert np.ptp(ratio) <= 1e-12 * ratio.mean()
    lam_star = float(ratio.mean())
    w = _toy_weights(q, k1, k2, lam_star)
    noise_mass0 = np.abs(a1[ones]).sum()
    assert noise_mass0 > 0.3                          # softmax spreads a lot of mass on noise
    assert np.abs(w[ones]).sum() <= 1e-13             # ... which the difference cancels
    assert w[s] > 0.5 * a1[s] > 0                     # the planted signal survives

    def snr(wts):
        return wts[s] / np.mean(np.abs(wts[ones]))
    base = snr(a1)
    for lam in (0.0, 0.2, 0.5, 0.8, lam_star - 1e-3):
        wl = _toy_weights(q, k1, k2, lam)
        closed = (wl[s] / a1[s]) / abs(1.0 - lam / lam_star)
        assert abs(snr(wl) / base - closed) <= 1e-9 * closed
    # the lambda sweep over [0, 1] peaks at lambda*
    grid = np.linspace(0.0, 1.0, 41)
    snrs = [snr(_toy_weights(q, k1, k2, lam)) for lam in grid]
    assert abs(grid[int(np.argmax(snrs))] - lam_star) <= 0.5 * (grid[1] - grid[0]) + 1e-12


# --------------------------------------------------------------------------
# causal sliding window (lesson "Attention Variants", "Build it", step 2 and
# the sliding-window figure of its "Concept" section): row i sees keys
# i - W + 1 .. i
# --------------------------------------------------------------------------


def test_swa_mask_matches_printed_figure():
    fig = _read_mask("swa_mask_8_w4.txt")
    N = fig.shape[0]
    rng = np.random.default_rng(14)
    q1, q2, k1, k2 = (rnd(rng, 1, 1, N, 4) for _ in range(4))
    v = rnd(rng, 1, 1, N, 3)
    base = _prefill(q1, q2, k1, k2, v, [0.3], causal=True, norm=False, window=4)
    seen = np.zeros((N, N), bool)
    for j in range(N):
        kk, vv = k1.copy(), v.copy()
        kk[0, 0, j] += 1.0
        vv[0, 0, j] += 1.0
        out = _prefill(q1, q2, kk, k2, vv, [0.3], causal=True, norm=False, window=4)
        seen[:, j] = np.any(out[0, 0] != base[0, 0], axis=-1)
    np.testing.assert_array_equal(seen, fig)


def test_swa_window_at_least_n_is_full_causal_bitwise():
    rng = np.random.default_rng(15)
    N = 37
    q1, q2, k1, k2 = (rnd(rng, 2, 3, N, 8) for _ in range(4))
    v = rnd(rng, 2, 3, N, 5)
    lam = [0.1, 0.5, 0.9]
    g = rng.uniform(0.9, 1.1, (3, 5)).astype(np.float32)
    full = _prefill(q1, q2, k1, k2, v, lam, causal=True, norm=True, gamma=g)
    for w in (N, N + 1, 10 * N):
        got = _prefill(q1, q2, k1, k2, v, lam, causal=True, norm=True, gamma=g, window=w)
        assert np.array_equal(got, full)


def test_swa_window_one_sees_only_itself():
    # each row's only key is its own: both softmaxes are 1, y = (1 - lambda) v_i
    rng = np.random.default_rng(16)
    N = 20
    q1, q2, k1, k2 = (rnd(rng, 1, 2, N, 6) for _ in range(4))
    v = rnd(rng, 1, 2, N, 4)
    lam = np.array([0.25, -0.5])
    got = _prefill(q1, q2, k1, k2, v, lam, causal=True, norm=False, window=1)
    ref = (1.0 - lam)[None, :, None, None] * v.astype(np.float64)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-15)


@pytest.mark.parametrize("window", [1, 2, 3, 5, 9])
def test_swa_matches_brute(window):
    rng = np.random.default_rng(17 + window)
    N, dqk, dv = 11, 4, 3
    q1, q2, k1, k2 = (rnd(rng, 1, 1, N, dqk) for _ in range(4))
    v = rnd(rng, 1, 1, N, dv)
    got = _prefill(q1, q2, k1, k2, v, [0.7], causal=True, norm=False, window=window)
    ref = brute.diff_attention(*(x[0, 0].astype(np.float64).tolist() for x in (q1, k1, q2, k2, v)), 0.7,
                               causal=True, window=window)
    np.testing.assert_allclose(got[0, 0], np.array(ref), rtol=1e-12, atol=1e-13)


def test_swa_row_equals_causal_attention_over_its_window():
    # row i with window W is the last row of a plain causal attention over the
    # W keys i-W+1..i alone (a different construction: the sequence is cut)
    rng = np.random.default_rng(18)
    N, W = 40, 7
    q1, q2, k1, k2 = (rnd(rng, 1, 2, N, 8) for _ in range(4))
    v = rnd(rng, 1, 2, N, 6)
    lam = [0.3, 0.8]
    got = _prefill(q1, q2, k1, k2, v, lam, causal=True, norm=False, window=W)
    for i in (0, 3, W - 1, W, 25, N - 1):
        lo = max(0, i - W + 1)
        cut = lambda x: np.ascontiguousarray(x[:, :, lo:i + 1])
        sub = _prefill(cut(q1), cut(q2), cut(k1), cut(k2), cut(v), lam, causal=True, norm=False)
        np.testing.assert_allclose(got[0, :, i], sub[0, :, -1], rtol=1e-13, atol=1e-14)


def test_swa_needs_causal():
    rng = np.random.default_rng(19)
    x = rnd(rng, 1, 1, 4, 2)
    with pytest.raises(ValueError):
        _prefill(x, x, x, x, x, [0.1], causal=False, norm=False, window=2)


# --------------------------------------------------------------------------
# GroupNorm variant of the V1 norm (one group per head, mean subtracted;
# the community post on the DIFF Transformer)
# --------------------------------------------------------------------------


def test_group_norm_closed_form():
    rng = np.random.default_rng(60)
    B, H, N, d, dv = 1, 2, 9, 4, 8
    q1, q2, k1, k2 = (rnd(rng, B, H, N, d) for _ in range(4))
    v = rnd(rng, B, H, N, dv)
    lam = [0.4, 0.9]
    ones = np.ones((H, dv), np.float32)
    plain = _prefill(q1, q2, k1, k2, v, lam, causal=True, norm=False, depth=5)
    got = _prefill(q1, q2, k1, k2, v, lam, causal=True, norm="group", gamma=ones, depth=5, eps=1e-5)
    u = plain - plain.mean(axis=-1, keepdims=True)
    var = (u * u).mean(axis=-1, keepdims=True)
    ref = u / np.sqrt(var + 1e-5) * (1 - oracle.lambda_init(5))
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-13)
    assert np.all(np.abs(got.mean(axis=-1)) <= 1e-14)


def test_group_norm_ignores_a_constant_added_to_v_rms_does_not():
    # adding c to every value channel shifts y by (1 - lambda) c in every
    # channel (each row of A1 - lambda A2 sums to 1 - lambda): the mean
    # subtraction removes it exactly, the RMS norm does not
    rng = np.random.default_rng(61)
    B, H, N, d, dv = 1, 1, 12, 4, 6
    q1, q2, k1, k2 = (rnd(rng, B, H, N, d) for _ in range(4))
    v = np.round(rnd(rng, B, H, N, dv) * 64) / 64  # on a 1/64 grid, so v + 0.75 is exact in fp32
    g = rng.uniform(0.9, 1.1, (H, dv)).astype(np.float32)
    kw = dict(causal=True, gamma=g, depth=3)
    a = _prefill(q1, q2, k1, k2, v, [0.3], norm="group", **kw)
    b = _prefill(q1, q2, k1, k2, v + np.float32(0.75), [0.3], norm="group", **kw)
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-12)
    ra = _prefill(q1, q2, k1, k2, v, [0.3], norm=True, **kw)
    rb = _prefill(q1, q2, k1, k2, v + np.float32(0.75), [0.3], norm=True, **kw)
    assert np.abs(ra - rb).max() > 1e-2


def test_group_norm_matches_brute():
    rng = np.random.default_rng(62)
    N, d, dv = 7, 3, 5
    q1, q2, k1, k2 = (rnd(rng, 1, 1, N, d) for _ in range(4))
    v = rnd(rng, 1, 1, N, dv)
    g = rng.uniform(0.5, 1.5, (1, dv)).astype(np.float32)
    got = _prefill(q1, q2, k1, k2, v, [0.6], causal=True, norm="group", gamma=g, depth=4)
    L = lambda x: x[0, 0].astype(np.float64).tolist()
    ref = brute.diff_attention(L(q1), L(k1), L(q2), L(k2), L(v), 0.6, causal=True, norm="group",
                               gamma=g[0].astype(np.float64).tolist(), lambda_init=brute.lambda_init(4))
    np.testing.assert_allclose(got[0, 0], np.array(ref), rtol=1e-12, atol=1e-13)
