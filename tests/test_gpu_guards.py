"""Guard margins around outputs and workspaces: every call below gets its
output (and, where it has one, its workspace) in the middle of a larger
buffer whose margins hold a byte pattern; after the call the margins must be
untouched, so a write past either end of a row, a head or the workspace shows
up even where the values inside are right. The values are checked against the
oracle as in the parity tests."""
import numpy as np
import pytest

import oracle
import workloads as W
from gpu_util import PrefillCase, check, dev, say, to_dev

pytestmark = pytest.mark.gpu

PAD = 1 << 16     # bytes of margin on each side (a multiple of 256, for alignment)
PATTERN = 0xA5


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


class Guarded:
    """A tensor of the given shape and dtype inside a byte buffer with PAD
    bytes of margin on each side, all filled with PATTERN."""

    def __init__(self, torch, shape, dtype):
        esize = torch.empty((), dtype=dtype).element_size()
        n = int(np.prod(shape)) * esize
        self.raw = torch.full((PAD + n + PAD,), PATTERN, dtype=torch.uint8, device=dev())
        self.n = n
        self.t = self.raw[PAD:PAD + n].view(dtype).view(shape)

    def intact(self) -> bool:
        lo, hi = self.raw[:PAD], self.raw[PAD + self.n:]
        return bool((lo == PATTERN).all().item() and (hi == PATTERN).all().item())


@pytest.mark.parametrize("form,N,window", [("v1", 333, 0), ("v2", 300, 0), ("v1", 300, 100), ("v2", 257, 64)])
def test_prefill_writes_nothing_outside_out(torch, da, form, N, window):
    p = W.prefill_v1(seed=N, B=2, H=3, N=N) if form == "v1" else W.prefill_v2(seed=N, B=2, H=4, H_kv=2, N=N)
    c = PrefillCase(p)
    g = Guarded(torch, (p.B, p.H, p.N, p.d_v), torch.bfloat16)
    say(f"guarded prefill {form} N {N} window {window}")
    c.run(out=g.t, window=window)
    torch.cuda.synchronize()
    assert g.intact(), "prefill wrote outside its output"
    check(g.t.float().cpu().numpy(), c.oracle(window=window), "bf16", f"{form} guarded")


def test_prefill_statistics_write_nothing_outside(torch, da):
    p = W.prefill_v1(seed=5, B=1, H=2, N=200)
    c = PrefillCase(p)
    gs = [Guarded(torch, (p.B, p.H, p.N, p.d_v), torch.float32) for _ in range(2)]
    gs += [Guarded(torch, (p.B, p.H, p.N), torch.float32) for _ in range(2)]
    g = Guarded(torch, (p.B, p.H, p.N, p.d_v), torch.bfloat16)
    c.run(out=g.t, stats=tuple(x.t for x in gs))
    torch.cuda.synchronize()
    assert g.intact() and all(x.intact() for x in gs), "prefill wrote outside its output or statistics"


@pytest.mark.parametrize("form", ["v2", "v1", "v2_fp8"])
def test_decode_writes_nothing_outside_out_or_workspace(torch, da, form):
    small = dict(B=5, H=8, H_kv=2, max_pages=12, ctx_lo=1, ctx_hi=12 * 64)
    d = {"v2": W.decode_v2, "v1": W.decode_v1, "v2_fp8": W.decode_v2_fp8}[form](**small)
    kv = "bf16" if d.kv_dtype == "bf16" else "u8"
    if d.q_full is not None:
        qd = to_dev(d.q_full, "bf16")
        q1, q2 = qd[:, 0::2], qd[:, 1::2]
    else:
        q1, q2 = to_dev(d.q1, "bf16"), to_dev(d.q2, "bf16")
    kc, vc = to_dev(d.k1_cache, kv), to_dev(d.v_cache, kv)
    kc2 = None if d.shared_k else to_dev(d.k2_cache, kv)
    table, ctx = torch.from_numpy(d.page_table).to(dev()), torch.from_numpy(d.ctx_len).to(dev())
    lam = da.lambda_(*(torch.from_numpy(x).to(dev()) for x in (d.lam_q1, d.lam_k1, d.lam_q2, d.lam_k2)), d.depth)
    gamma = torch.from_numpy(d.gamma).to(dev()) if d.norm else None
    kw = dict(depth=d.depth, norm=d.norm, gamma=gamma, eps=d.eps, k2_cache=kc2, k_scale=d.k_scale,
              v_scale=d.v_scale)
    need = da.decode_workspace_bytes(q1, q2, kc, vc, table, ctx, lam, **kw)
    ws = Guarded(torch, (need,), torch.uint8)
    out = Guarded(torch, (d.B, d.H, d.d_v), torch.bfloat16)
    say(f"guarded decode {form}: workspace {need} bytes")
    da.decode(q1, q2, kc, vc, table, ctx, lam, out=out.t, workspace=ws.t, **kw)
    torch.cuda.synchronize()
    assert out.intact(), "decode wrote outside its output"
    assert ws.intact(), "decode wrote outside its workspace"
    lam64 = oracle.lambda_(d.lam_q1, d.lam_k1, d.lam_q2, d.lam_k2, d.depth)
    ref = oracle.decode(d.f32("q1"), d.f32("q2"), d.f32("k1_cache"),
                        d.f32("k1_cache") if d.shared_k else d.f32("k2_cache"), d.f32("v_cache"), d.page_table,
                        d.ctx_len, lam64, depth=d.depth, norm=d.norm, gamma=d.gamma, eps=d.eps)
    check(out.t.float().cpu().numpy(), ref, "bf16", f"decode {form} guarded")


@pytest.mark.parametrize("form", ["v1", "v2"])
def test_backward_writes_nothing_outside_its_workspace(torch, da, form):
    p = W.prefill_v1(seed=3, B=1, H=2, N=257) if form == "v1" else W.prefill_v2(seed=3, B=1, H=4, H_kv=2, N=257)
    c = PrefillCase(p)
    stats = da.prefill_stats(c.q1, c.v)
    c.run(stats=stats)
    rng = np.random.default_rng(11)
    dout = to_dev(W.f32_to_bf16(rng.standard_normal((p.B, p.H, p.N, p.d_v)).astype(np.float32)), "bf16")
    probe = dict(depth=p.depth, causal=p.causal, norm=p.norm, gamma=c.gamma, eps=p.eps)
    g0 = da.backward(c.q1, c.q2, c.k1, c.k2, c.v, c.lam, stats, dout, **probe)  # unguarded reference
    need = da.backward_workspace_bytes(c.q1, c.q2, c.k1, c.k2, c.v, c.lam, stats, dout, **probe)
    ws = Guarded(torch, (need,), torch.uint8)
    g1 = da.backward(c.q1, c.q2, c.k1, c.k2, c.v, c.lam, stats, dout, workspace=ws.t, **probe)
    torch.cuda.synchronize()
    assert ws.intact(), "backward wrote outside its workspace"
    for k in g0:
        if g0[k] is not None:
            assert torch.equal(g0[k], g1[k]), k

