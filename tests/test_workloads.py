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


def test_fp8_table_matches_format_and_torch():
    # e4m3 values from the format's definition (bias 7, subnormals m/8 * 2^-6,
    # S.1111.111 NaN, no infinities), checked on known codes and against torch
    import torch
    t = W.FP8_TABLE
    known = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 / 8 * 2.0 ** -6, 0x08: 2.0 ** -6, 0x38: 1.0,
             0x39: 1.125, 0x40: 2.0, 0x7e: 448.0, 0x80: -0.0, 0xb8: -1.0, 0xfe: -448.0}
    for c, v in known.items():
        assert t[c] == v and np.signbit(t[c]) == np.signbit(v), hex(c)
    assert np.isnan(t[0x7f]) and np.isnan(t[0xff]) and np.isfinite(np.delete(t, [0x7f, 0xff])).all()
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).float().numpy()
    assert np.array_equal(t, ref, equal_nan=True)


def test_fp8_encoder_rounds_to_nearest_even():
    vals = W.FP8_TABLE[np.isfinite(W.FP8_TABLE)]
    codes = W.f32_to_fp8(vals)
    assert np.array_equal(W.fp8_to_f32(codes), vals)          # representable values round-trip
    # midpoints between 1.0 (mantissa 0) and 1.125 (mantissa 1) go to the even one
    assert W.fp8_to_f32(W.f32_to_fp8(np.float32([1.0625, 1.1875, 1.06]))).tolist() == [1.0, 1.25, 1.0]
    x = np.random.default_rng(0).uniform(-448, 448, 4096).astype(np.float32)
    y = W.fp8_to_f32(W.f32_to_fp8(x))
    fin = np.sort(vals.astype(np.float64))
    # every result is a nearest representable value
    i = np.clip(np.searchsorted(fin, x), 1, len(fin) - 1)
    best = np.minimum(np.abs(fin[i] - x), np.abs(fin[i - 1] - x))
    assert np.all(np.abs(y - x) <= best + 0.0)


def test_fp8_decode_workloads():
    d = W.decode_v2_fp8(B=3, H=4, H_kv=2, max_pages=4, ctx_lo=1, ctx_hi=256)
    assert d.kv_dtype == "fp8" and d.k1_cache.dtype == np.uint8 and d.k1_cache is d.k2_cache
    b = W.decode_v2(B=3, H=4, H_kv=2, max_pages=4, ctx_lo=1, ctx_hi=256)
    np.testing.assert_array_equal(d.page_table, b.page_table)   # same draws, other storage
    np.testing.assert_array_equal(d.q_full, b.q_full)
    k8, k16 = d.f32("k1_cache"), b.f32("k1_cache")
    assert np.max(np.abs(k8 - k16)) <= 2 ** -4 * np.max(np.abs(k16)) + 1e-6  # 3 mantissa bits
    v1 = W.decode_v1(B=2, H=4, H_kv=2, max_pages=4, ctx_len=np.array([100, 200]), kv_dtype="fp8")
    assert v1.k1_cache.dtype == np.uint8 and v1.k2_cache is not v1.k1_cache
    assert abs(float(v1.f32("v_cache").std()) - 0.5) < 0.02
