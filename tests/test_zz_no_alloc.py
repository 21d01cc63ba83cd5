"""The allocation-free paged decode (diffattn_decode_noalloc) against the
workspace form (diffattn_decode), through the C ABI.

Both forms run the same kernels with the same split, so their outputs agree
bit for bit; the oracle bounds the smaller case as in the decode parity tests.
Two calls in a row, the second smaller, so the second runs over scratch the
first left full of its own partial results."""
import numpy as np
import pytest

import workloads as W
from gpu_util import check, say

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


def _case(torch, da, d):
    from test_gpu_decode import DecodeCase
    return DecodeCase(d, torch, da)


def _noalloc(c, torch, **kw):
    """decode_noalloc into a preallocated output; checks torch allocated nothing."""
    d = c.d
    out = torch.full((d.B, c.q1.shape[1], c.vc.shape[3]), float("nan"), dtype=c.q1.dtype, device=c.q1.device)
    torch.cuda.synchronize()
    before = torch.cuda.memory_stats()["allocation.all.allocated"]
    c.da.decode_noalloc(c.q1, c.q2, c.kc, c.vc, c.table, c.ctx, c.lam, depth=d.depth, norm=d.norm,
                        gamma=c.gamma, eps=d.eps, k2_cache=c.kc2, k_scale=d.k_scale, v_scale=d.v_scale,
                        out=out, **kw)
    torch.cuda.synchronize()
    assert torch.cuda.memory_stats()["allocation.all.allocated"] == before
    return out


@pytest.mark.parametrize("split_pages", [0, 3])
def test_noalloc_matches_workspace_form_twice(torch, da, split_pages):
    big = _case(torch, da, W.decode_v2())
    say(f"noalloc call 1: decode_v2, 64 sequences, {big.d.num_pages} pages, split_pages {split_pages}")
    a1 = _noalloc(big, torch, split_pages=split_pages)
    r1 = big.run(split_pages=split_pages)
    assert torch.equal(a1, r1)

    small = _case(torch, da, W.decode_v2(seed=3, B=5, H=8, H_kv=2, max_pages=16,
                                         ctx_len=np.array([1, 64, 65, 700, 1024])))
    say(f"noalloc call 2: 5 sequences, H 8, H_kv 2, split_pages {split_pages}")
    a2 = _noalloc(small, torch, split_pages=split_pages)
    r2 = small.run(split_pages=split_pages)
    assert torch.equal(a2, r2)
    check(a2.float().cpu().numpy(), small.oracle(), "bf16", "decode_noalloc small case")


def test_noalloc_v1_fp8(torch, da):
    d = W.decode_v2(seed=5, B=4, H=8, H_kv=2, max_pages=16, ctx_len=np.array([3, 129, 640, 1000]))
    c = _case(torch, da, d)
    say("noalloc: V2 form, 4 sequences, then V1 form with fp8 caches")
    assert torch.equal(_noalloc(c, torch), c.run())
    from test_gpu_decode import small_fp8
    c8 = _case(torch, da, small_fp8([1, 65, 500], form="v1"))
    a = _noalloc(c8, torch)
    assert torch.equal(a, c8.run())
    check(a.float().cpu().numpy(), c8.oracle(), "bf16", "decode_noalloc V1 fp8")


def test_noalloc_rejects_too_much_scratch(torch, da):
    # 4096 sequences x 8 KV heads with 8 query pairs per KV head need more than
    # the 32 MiB scratch: rejected before any launch, output untouched
    B, H, H_kv = 4096, 64, 8
    q = torch.zeros((B, H, 128), dtype=torch.bfloat16, device="cuda")
    kc = torch.zeros((1, H_kv, 64, 128), dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros((1, H_kv, 64, 128), dtype=torch.bfloat16, device="cuda")
    table = torch.zeros((B, 1), dtype=torch.int32, device="cuda")
    ctx = torch.ones(B, dtype=torch.int32, device="cuda")
    lam = torch.zeros(H, dtype=torch.float32, device="cuda")
    out = torch.full((B, H, 128), 7.0, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(da.DiffAttnError, match="scratch"):
        da.decode_noalloc(q, q, kc, vc, table, ctx, lam, depth=1, out=out)
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())
