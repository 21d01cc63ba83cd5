"""GPU parity of lambda and prefill against the fp64 oracle, through the C ABI.

Tolerances: bf16 inputs with fp32 accumulation: max |error| <= 2e-2 and
relative Frobenius error <= 1e-2; the fp32 path: max |error| <= 1e-5."""
import numpy as np
import pytest

import oracle
import workloads as W
from gpu_util import (PrefillCase, check, check_all_rows_by_head, dev, gather_rows, sampled_rows, say, to_dev)

pytestmark = pytest.mark.gpu


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


# ---------------------------------------------------------------- lambda

@pytest.mark.parametrize("H,dl,depth", [(1, 64, 1), (16, 64, 12), (32, 128, 20), (8, 64, 12), (5, 1000, 3)])
def test_lambda_parity(torch, da, H, dl, depth):
    rng = np.random.default_rng(H * 1000 + dl)
    vecs = [(rng.standard_normal((H, dl)) * 0.1).astype(np.float32) for _ in range(4)]
    got = da.lambda_(*(torch.from_numpy(v).to(dev()) for v in vecs), depth).cpu().numpy()
    ref = oracle.lambda_(*vecs, depth)
    # fp32 evaluation of exp(a) - exp(b) + init: the terms are O(1), so a few
    # fp32 ulps of 1 bound the error (relative error is meaningless when they cancel)
    assert np.max(np.abs(got - ref)) <= 1e-6


# ---------------------------------------------------------------- fp32 path

def test_tiny_v1_fp32(torch, da):
    c = PrefillCase(W.tiny_v1())
    say("tiny_v1 fp32 (1 head, N 128, causal, RMS)")
    got = c.run().cpu().numpy()
    check(got, c.oracle(), "f32", "tiny_v1")


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("N,dqk,dv,H,Hkv,norm", [(1, 64, 128, 1, 1, True), (77, 48, 80, 4, 2, False),
                                                  (130, 128, 128, 2, 1, True), (65, 3, 5, 2, 2, False)])
def test_fp32_variants(torch, da, causal, N, dqk, dv, H, Hkv, norm):
    rng = np.random.default_rng(N + dqk)
    f = lambda *s: rng.standard_normal(s).astype(np.float32)
    p = W.Prefill("f32case", "f32", 2, H, Hkv, N, dqk, dv, f(2, H, N, dqk), f(2, H, N, dqk),
                  f(2, Hkv, N, dqk), f(2, Hkv, N, dqk), f(2, Hkv, N, dv),
                  *(0.1 * f(H, dqk) for _ in range(4)), depth=4, causal=causal, norm=norm,
                  gamma=rng.uniform(0.9, 1.1, (H, dv)).astype(np.float32) if norm else None)
    c = PrefillCase(p)
    say(f"f32 N {N} dqk {dqk} dv {dv} H {H}/{Hkv} causal {causal} norm {norm}")
    check(c.run().cpu().numpy(), c.oracle(), "f32", "f32 variant")


# ---------------------------------------------------------------- bf16 path, small shapes

def _bf16_case(form, N, causal, B=2, seed=0, shared=None, norm=None):
    if form == "v1":
        p = W.prefill_v1(seed=seed, B=B, H=3, N=N, causal=causal)
    else:
        p = W.prefill_v2(seed=seed, B=B, H=4, H_kv=2, N=N, causal=causal)
    if shared is not None and shared != p.shared_k:
        if shared:
            p.k2 = p.k1
        else:
            rng = np.random.default_rng(seed + 99)
            p.k2 = W.f32_to_bf16(rng.standard_normal(p.k1.shape).astype(np.float32))
        p.shared_k = shared
    if norm is not None and norm != p.norm:
        p.norm = norm
        p.gamma = np.random.default_rng(seed).uniform(0.9, 1.1, (p.H, p.d_v)).astype(np.float32) if norm else None
    return p


@pytest.mark.parametrize("form", ["v1", "v2"])
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("N", [1, 31, 64, 200, 333])
def test_bf16_small(torch, da, form, causal, N):
    p = _bf16_case(form, N, causal, seed=N)
    c = PrefillCase(p)
    say(f"bf16 {form} N {N} causal {causal}")
    check(c.run().float().cpu().numpy(), c.oracle(), "bf16", f"{form} N={N}")


@pytest.mark.parametrize("form,shared,norm", [("v1", True, True), ("v1", False, False), ("v1", True, False),
                                              ("v2", False, False), ("v2", True, True), ("v2", False, True)])
def test_bf16_all_kernel_variants(torch, da, form, shared, norm):
    p = _bf16_case(form, 257, True, B=1, seed=7, shared=shared, norm=norm)
    c = PrefillCase(p)
    say(f"bf16 variant {form} shared_k {shared} norm {norm}")
    check(c.run().float().cpu().numpy(), c.oracle(), "bf16", f"{form}/{shared}/{norm}")


def test_bf16_explicit_scale_and_strided_out(torch, da):
    p = _bf16_case("v2", 150, True, B=1, seed=3)
    c = PrefillCase(p)
    big = torch.zeros((1, p.N, p.H, 128), dtype=torch.bfloat16, device=dev())
    out = big.permute(0, 2, 1, 3)  # [B, H, N, d] view with the head stride 128
    c.run(scale=0.05, out=out)
    ref = oracle.prefill(p.f32("q1"), p.f32("q2"), p.f32("k1"), p.f32("k1"), p.f32("v"), c.lam64,
                         depth=p.depth, causal=True, norm=False, scale=0.05)
    check(out.float().cpu().numpy(), ref, "bf16", "scale 0.05, [B,N,H,d] output")


# ---------------------------------------------------------------- invariants (bitwise)

def _wide_rows(torch, x, extra):
    """The same values as x [B, H, N, d], in a view whose rows are `extra`
    elements longer (a different row stride)."""
    w = torch.zeros(x.shape[:3] + (x.shape[3] + extra,), dtype=x.dtype, device=x.device)
    w[..., :x.shape[3]] = x
    return w[..., :x.shape[3]]


def test_bf16_general_copy_path_is_bitwise_equal(torch, da):
    # Whole key/value tiles are copied with buffer loads when K1 and K2 share
    # their row stride and every (batch, KV head) slice spans less than 2^31
    # bytes; other layouts copy every tile through per-lane addresses. Both
    # must fill LDS with the same bytes, so the outputs agree bit for bit.
    c = PrefillCase(_bf16_case("v1", 700, True, B=1, seed=21))
    say("V1, N 700: K2 rows 64 elements longer than K1's")
    a = c.run().clone()
    c.k2 = _wide_rows(torch, c.k2, 64)
    assert torch.equal(a, c.run())
    # V2 with shared keys: a value row stride of 2^21 elements, so one slice
    # of V spans 2.5 GB (the storage is allocated, only 128 elements a row are set)
    p = W.prefill_v2(seed=22, B=1, H=2, H_kv=1, N=600)
    c = PrefillCase(p)
    say("V2, N 600: value rows 2^21 elements apart")
    a = c.run().clone()
    rs = 1 << 21
    store = torch.empty(p.N * rs, dtype=torch.bfloat16, device=dev())
    v = store.as_strided((1, 1, p.N, p.d_v), (p.N * rs, p.N * rs, rs, 1))
    v.copy_(c.v)
    c.v = v
    assert torch.equal(a, c.run())
    del store, v


def test_lambda_zero_ignores_branch_two(torch, da):
    c = PrefillCase(_bf16_case("v1", 190, True, B=1, seed=11))
    zero = torch.zeros(c.p.H, dtype=torch.float32, device=dev())
    a = c.run(lam=zero).clone()
    c.q2 = torch.randn_like(c.q2.float()).to(torch.bfloat16)
    c.k2 = torch.randn_like(c.k2.float()).to(torch.bfloat16)
    b = c.run(lam=zero)
    assert torch.equal(a, b)


def test_identical_branches_lambda_one_is_zero(torch, da):
    for form in ("v1", "v2"):
        c = PrefillCase(_bf16_case(form, 130, True, B=1, seed=12))
        c.q2, c.k2 = c.q1, c.k1
        one = torch.ones(c.p.H, dtype=torch.float32, device=dev())
        out = c.run(lam=one)
        assert torch.count_nonzero(out).item() == 0


def test_causality_and_determinism(torch, da):
    c = PrefillCase(_bf16_case("v2", 300, True, B=1, seed=13))
    a = c.run().clone()
    assert torch.equal(a, c.run())  # run to run
    r = 150
    k1 = c.k1.clone()
    v = c.v.clone()
    k1[:, :, r + 1:] = torch.randn_like(k1[:, :, r + 1:].float()).to(torch.bfloat16)
    v[:, :, r + 1:] = torch.randn_like(v[:, :, r + 1:].float()).to(torch.bfloat16)
    c.k1 = c.k2 = k1
    c.v = v
    b = c.run()
    assert torch.equal(a[:, :, :r + 1], b[:, :, :r + 1])
    assert not torch.equal(a[:, :, r + 1:], b[:, :, r + 1:])


# ---------------------------------------------------------------- full-size workloads

def test_prefill_v1_full(torch, da):
    # every row of every head (the oracle needs a few seconds for all 131072)
    p = W.prefill_v1()
    c = PrefillCase(p)
    say("prefill_v1 full: B 2, H 16, N 4096, d_qk 64, d_v 128, causal, RMS; all rows")
    out = c.run().float().cpu().numpy()
    check(out, c.oracle(), "bf16", "prefill_v1 all rows")


def test_prefill_v2_full(torch, da):
    # every row of every head: 524288 rows (the oracle over all of them takes
    # a minute or two on the host's cores, one head at a time)
    p = W.prefill_v2()
    c = PrefillCase(p)
    say("prefill_v2 full: 64 query heads / 8 KV heads, N 16384, d 128, causal; all rows")
    out = c.run().float().cpu().numpy()
    check_all_rows_by_head(c, out, "prefill_v2 all rows")


def test_longctx_v1_full(torch, da):
    # every row of every head (524288 rows, the planted keys' probe rows among
    # them); the probe rows are also checked on their own
    p = W.longctx_v1()
    c = PrefillCase(p)
    say("longctx_v1 full: H 8, N 65536, planted keys, causal, RMS; all rows")
    out_d = c.run()
    torch.cuda.synchronize()
    probe = np.unique(np.concatenate([(b * p.H + h) * p.N + p.probes[b, h, :, 1]
                                      for b in range(p.B) for h in range(p.H)]))
    check(gather_rows(out_d, probe, p.H, p.N), c.oracle(rows=probe), "bf16", "longctx_v1 probe rows")
    check_all_rows_by_head(c, out_d.float().cpu().numpy(), "longctx_v1 all rows")


# ---------------------------------------------------------------- causal sliding window

@pytest.mark.parametrize("form", ["v1", "v2"])
@pytest.mark.parametrize("N,window", [(200, 1), (200, 17), (333, 32), (333, 33), (513, 64), (513, 100),
                                      (513, 129), (700, 300)])
def test_bf16_sliding_window(torch, da, form, N, window):
    p = _bf16_case(form, N, True, seed=N + window)
    c = PrefillCase(p)
    say(f"bf16 {form} N {N} window {window}")
    check(c.run(window=window).float().cpu().numpy(), c.oracle(window=window), "bf16",
          f"{form} N={N} W={window}")


@pytest.mark.parametrize("form", ["v1", "v2"])
def test_bf16_window_at_least_n_is_full_causal_bitwise(torch, da, form):
    p = _bf16_case(form, 333, True, seed=5)
    c = PrefillCase(p)
    full = c.run().clone()
    for w in (333, 334, 5000):
        assert torch.equal(c.run(window=w), full), w


@pytest.mark.parametrize("N,window", [(1, 1), (77, 5), (130, 64), (130, 200)])
def test_fp32_sliding_window(torch, da, N, window):
    p = W.tiny_v1(seed=N, N=N, H=2)
    c = PrefillCase(p)
    say(f"f32 N {N} window {window}")
    check(c.run(window=window).cpu().numpy(), c.oracle(window=window), "f32", f"f32 W={window}")


def test_window_needs_causal(torch, da):
    p = _bf16_case("v1", 64, False, B=1, seed=1)
    c = PrefillCase(p)
    with pytest.raises(RuntimeError):
        c.run(window=8)


def test_bf16_long_sequence_small_window_sampled(torch, da):
    # V2 GQA at N 16384 with a 1024-key window (the 5:1 local-layer setting the
    # lesson cites): key tiles outside the windows are skipped; rows sampled
    p = W.prefill_v2(seed=31, N=16384)
    c = PrefillCase(p)
    say("prefill_v2 shape, window 1024, sampled rows")
    out = c.run(window=1024)
    rows = sampled_rows(p.B, p.H, p.N, seed=31, n_rand=24, edge=8)
    check(gather_rows(out, rows, p.H, p.N), c.oracle(rows=rows, window=1024), "bf16", "v2 W=1024")


# ---------------------------------------------------------------- GroupNorm variant of the V1 norm

@pytest.mark.parametrize("form,shared,N", [("v1", False, 200), ("v1", True, 333), ("v2", True, 150)])
def test_bf16_group_norm(torch, da, form, shared, N):
    p = _bf16_case(form, N, True, seed=N, shared=shared, norm=True)
    p.norm = "group"
    c = PrefillCase(p)
    say(f"bf16 {form} shared_k {shared} N {N} GroupNorm")
    check(c.run().float().cpu().numpy(), c.oracle(), "bf16", f"{form} GroupNorm")


def test_fp32_group_norm(torch, da):
    p = W.tiny_v1(seed=4, N=100, H=2)
    p.norm = "group"
    c = PrefillCase(p)
    check(c.run().cpu().numpy(), c.oracle(), "f32", "f32 GroupNorm")


# ---------------------------------------------------------------- score range: exact sweep after the fast one
# The bf16 kernels first sweep with probabilities 2^s against a fixed
# reference (no running max); a work-group whose rows leave the range where
# that is exact sweeps again with the running max. These inputs put scores
# far above (2^s would overflow to inf) or far below (2^s would underflow to
# 0) that range, so a missing or wrong second sweep gives non-finite rows.

@pytest.mark.parametrize("form", ["v1", "v2"])
@pytest.mark.parametrize("scale", [2.0, 16.0])
def test_bf16_large_scores(torch, da, form, scale):
    p = _bf16_case(form, 333, True, B=1, seed=41)
    c = PrefillCase(p)
    say(f"bf16 {form} N 333 scale {scale} (scores up to ~{scale * 9:.0f} nats)")
    got = c.run(scale=scale).float().cpu().numpy()
    k1 = p.f32("k1")
    ref = oracle.prefill(p.f32("q1"), p.f32("q2"), k1, k1 if p.shared_k else p.f32("k2"), p.f32("v"), c.lam64,
                         depth=p.depth, causal=True, norm=p.norm, gamma=p.gamma, eps=p.eps, scale=scale)
    check(got, ref, "bf16", f"{form} scale {scale}")


@pytest.mark.parametrize("form", ["v1", "v2"])
def test_bf16_all_scores_far_below_zero(torch, da, form):
    # every key carries +10 u and every query -10 u (u a unit vector), so all
    # scores sit near -100 * scale nats; the softmax depends only on the rest
    p = _bf16_case(form, 300, True, B=1, seed=43)
    u = np.zeros(p.d_qk, np.float32)
    u[3] = 1.0
    shift = lambda x, s: W.f32_to_bf16(W.bf16_to_f32(x) + s * u)
    if p.q_full is not None:
        p.q_full = shift(p.q_full, -10.0)
        p.q1, p.q2 = p.q_full[:, 0::2], p.q_full[:, 1::2]
    else:
        p.q1, p.q2 = shift(p.q1, -10.0), shift(p.q2, -10.0)
    p.k1 = shift(p.k1, 10.0)
    p.k2 = p.k1 if p.shared_k else shift(p.k2, 10.0)
    c = PrefillCase(p)
    say(f"bf16 {form} N 300, scores near -100 * scale")
    got = c.run(scale=2.0).float().cpu().numpy()
    k1 = p.f32("k1")
    ref = oracle.prefill(p.f32("q1"), p.f32("q2"), k1, k1 if p.shared_k else p.f32("k2"), p.f32("v"), c.lam64,
                         depth=p.depth, causal=True, norm=p.norm, gamma=p.gamma, eps=p.eps, scale=2.0)
    check(got, ref, "bf16", f"{form} negative scores")
