"""The seeded input generators (no GPU): bf16 rounding, determinism, structure."""
import numpy as np
import pytest

import workloads as W


def test_bf16_round_to_nearest_even_matches_torch():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 3,
                        np.array([0.0, -0.0, 1.0, 1.00390625, 1.01171875, 65504.0, 1e-30, -2.5],
                                 np.float32)])
    ours = W.f32_to_bf16(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)
    back = W.bf16_to_f32(ours)
    np.testing.assert_array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_generators_are_deterministic_and_shaped():
    a = W.prefill_v1(N=64, B=1, H=2)
    b = W.prefill_v1(N=64, B=1, H=2)
    np.testing.assert_array_equal(a.q1, b.q1)
    assert a.q1.shape == (1, 2, 64, 64) and a.v.shape == (1, 2, 64, 128)
    assert a.gamma.min() >= 0.9 and a.gamma.max() <= 1.1
    c = W.prefill_v2(N=32, H=4, H_kv=2)
    np.testing.assert_array_equal(c.q1, c.q_full[:, 0::2])
    np.testing.assert_array_equal(c.q2, c.q_full[:, 1::2])
    assert c.k1 is c.k2 and c.shared_k


def test_decode_page_table_structure():
    d = W.decode_v2(B=5, H=4, H_kv=2, max_pages=8, ctx_lo=1, ctx_hi=8 * 64)
    npg = (d.ctx_len + 63) // 64
    used = np.concatenate([d.page_table[b, :npg[b]] for b in range(d.B)])
    assert sorted(used.tolist()) == list(range(d.num_pages))   # a permutation of all pages
    for b in range(d.B):
        assert np.all(d.page_table[b, npg[b]:] == -1)
    assert d.k1_cache.shape == (d.num_pages, 2, 64, 128) and d.k1_cache is d.k2_cache


def test_longctx_planted_keys_have_cosine_0p9():
    p = W.longctx_v1(N=2048, H=2, n_planted=4)
    q1, k1 = p.f32("q1"), p.f32("k1")
    for h in range(2):
        for pos, t in p.probes[0, h]:
            q, k = q1[0, h, t].astype(np.float64), k1[0, h, pos].astype(np.float64)
            cos = q @ k / np.linalg.norm(q) / np.linalg.norm(k)
            assert abs(cos - 0.9) < 5e-3            # bf16 rounding of both vectors
            assert abs(np.linalg.norm(k) - 8.0) < 0.05
            assert pos < t
