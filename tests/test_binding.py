"""The Python binding rejects tensors of the wrong dtype, shape or layout
before any pointer reaches the library (CPU only: every case fails in the
checks, so nothing is launched)."""
import pytest
import torch

import differential_attention_amd as da


def _decode_inputs(**over):
    B, H, Hkv, P, page, mp = 3, 4, 2, 10, 64, 5
    t = dict(q1=torch.zeros(B, H, 128, dtype=torch.bfloat16), q2=torch.zeros(B, H, 128, dtype=torch.bfloat16),
             k_cache=torch.zeros(P, Hkv, page, 128, dtype=torch.bfloat16),
             v_cache=torch.zeros(P, Hkv, page, 128, dtype=torch.bfloat16),
             page_table=torch.zeros(B, mp, dtype=torch.int32), ctx_len=torch.ones(B, dtype=torch.int32),
             lam=torch.zeros(H, dtype=torch.float32))
    t.update(over)
    return t


def _decode(**over):
    t = _decode_inputs(**over)
    kw = {k: t.pop(k) for k in list(t) if k not in ("q1", "q2", "k_cache", "v_cache", "page_table",
                                                        "ctx_len", "lam")}
    return da.decode(t["q1"], t["q2"], t["k_cache"], t["v_cache"], t["page_table"], t["ctx_len"], t["lam"],
                     depth=3, **kw)


@pytest.mark.parametrize("over,exc,words", [
    (dict(page_table=torch.zeros(3, 5, dtype=torch.int64)), TypeError, "page_table"),   # torch's default ints
    (dict(ctx_len=torch.ones(3, dtype=torch.int64)), TypeError, "ctx_len"),
    (dict(ctx_len=torch.ones(4, dtype=torch.int32)), ValueError, "ctx_len"),
    (dict(page_table=torch.zeros(2, 5, dtype=torch.int32)), ValueError, "page_table"),
    (dict(page_table=torch.zeros(5, 3, dtype=torch.int32).t()), ValueError, "contiguous"),
    (dict(lam=torch.zeros(4, dtype=torch.float64)), TypeError, "lam"),
    (dict(lam=torch.zeros(5, dtype=torch.float32)), ValueError, "lam"),
    (dict(q2=torch.zeros(3, 4, 64, dtype=torch.bfloat16)), ValueError, "q2"),
    (dict(v_cache=torch.zeros(9, 2, 64, 128, dtype=torch.bfloat16)), ValueError, "v_cache"),   # fewer pages
    (dict(gamma=torch.ones(128, dtype=torch.float32), norm=True), ValueError, "gamma"),   # [d_v], not [H, d_v]
    (dict(gamma=torch.ones(4, 128, dtype=torch.bfloat16), norm=True), TypeError, "gamma"),
    (dict(gamma=None, norm=True), ValueError, "gamma"),
    (dict(k2_cache=torch.zeros(10, 2, 64, 64, dtype=torch.bfloat16)), ValueError, "k2_cache"),
    (dict(), ValueError, "device"),   # everything right but on the host
])
def test_decode_binding_rejects(over, exc, words):
    with pytest.raises(exc, match=words):
        _decode(**over)


def _prefill_inputs(**over):
    B, H, Hkv, N = 1, 4, 2, 16
    b = lambda *s: torch.zeros(*s, dtype=torch.bfloat16)
    t = dict(q1=b(B, H, N, 64), q2=b(B, H, N, 64), k1=b(B, Hkv, N, 64), k2=b(B, Hkv, N, 64), v=b(B, Hkv, N, 128),
             lam=torch.zeros(H, dtype=torch.float32))
    t.update(over)
    return t


@pytest.mark.parametrize("over,kw,exc,words", [
    (dict(k2=torch.zeros(1, 2, 8, 64, dtype=torch.bfloat16)), {}, ValueError, "k2"),     # fewer keys
    (dict(v=torch.zeros(1, 2, 16, 64, dtype=torch.bfloat16)), {}, ValueError, "v"),
    (dict(lam=torch.zeros(4, dtype=torch.float16)), {}, TypeError, "lam"),
    (dict(), dict(norm=True, gamma=torch.ones(128, dtype=torch.float32)), ValueError, "gamma"),
    (dict(), dict(norm=True, gamma=torch.ones(4, 128, dtype=torch.float32).t().contiguous().t()),
     ValueError, "gamma"),
    (dict(), dict(out=torch.zeros(1, 4, 16, 64, dtype=torch.bfloat16)), ValueError, "out"),
    (dict(), {}, ValueError, "device"),
])
def test_prefill_binding_rejects(over, kw, exc, words):
    t = _prefill_inputs(**over)
    with pytest.raises(exc, match=words):
        da.prefill(t["q1"], t["q2"], t["k1"], t["k2"], t["v"], t["lam"], depth=2, **kw)


def test_lambda_backward_binding_rejects():
    v = torch.zeros(4, 8, dtype=torch.float32)
    with pytest.raises(ValueError, match="lk1"):
        da.lambda_backward(v, torch.zeros(4, 9), v, v, torch.zeros(4))
    with pytest.raises(TypeError, match="dlambda"):
        da.lambda_backward(v, v, v, v, torch.zeros(4, dtype=torch.float64))
