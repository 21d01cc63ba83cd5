"""GPU parity of the split-KV paged decode against the fp64 oracle, through the C ABI."""
import numpy as np
import pytest

import oracle
import workloads as W
from gpu_util import check, dev, say, to_dev

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


class DecodeCase:
    def __init__(self, d: W.Decode, torch, da):
        self.d, self.torch, self.da = d, torch, da
        if d.q_full is not None:
            qf = to_dev(d.q_full, "bf16")
            self.q1, self.q2 = qf[:, 0::2], qf[:, 1::2]
        else:
            self.q1, self.q2 = to_dev(d.q1, "bf16"), to_dev(d.q2, "bf16")
        kv = "bf16" if d.kv_dtype == "bf16" else "u8"  # fp8 caches go in as their uint8 codes
        self.kc = to_dev(d.k1_cache, kv)
        self.kc2 = None if d.shared_k else to_dev(d.k2_cache, kv)
        self.vc = to_dev(d.v_cache, kv)
        self.table = torch.from_numpy(d.page_table).to(dev())
        self.ctx = torch.from_numpy(d.ctx_len).to(dev())
        self.lam64 = oracle.lambda_(d.lam_q1, d.lam_k1, d.lam_q2, d.lam_k2, d.depth)
        vecs = [torch.from_numpy(x).to(dev()) for x in (d.lam_q1, d.lam_k1, d.lam_q2, d.lam_k2)]
        self.lam = da.lambda_(*vecs, d.depth)
        self.gamma = torch.from_numpy(d.gamma).to(dev()) if d.norm else None

    def run(self, **kw):
        d = self.d
        args = dict(depth=d.depth, norm=d.norm, gamma=self.gamma, eps=d.eps, k2_cache=self.kc2,
                    k_scale=d.k_scale, v_scale=d.v_scale)
        args.update(kw)
        return self.da.decode(self.q1, self.q2, self.kc, self.vc, self.table, self.ctx, self.lam, **args)

    def oracle(self, seqs=None, norm=None, gamma=None, window=0):
        """Oracle on all sequences, or on a subset with their pages compacted."""
        d = self.d
        norm = d.norm if norm is None else norm
        if gamma is None and norm:
            gamma = d.gamma
        if seqs is None:
            kc, kc2 = d.f32("k1_cache"), d.f32("k2_cache")
            return oracle.decode(d.f32("q1"), d.f32("q2"), kc, kc2, d.f32("v_cache"), d.page_table,
                                 d.ctx_len, self.lam64, depth=d.depth, norm=norm, gamma=gamma,
                                 window=window)
        seqs = np.asarray(seqs)
        npg = (d.ctx_len[seqs] + d.page - 1) // d.page
        used = np.concatenate([d.page_table[b, :n] for b, n in zip(seqs, npg)])
        remap = {int(p): i for i, p in enumerate(used)}
        table = np.full((len(seqs), d.max_pages), -1, np.int32)
        for r, (b, n) in enumerate(zip(seqs, npg)):
            table[r, :n] = [remap[int(p)] for p in d.page_table[b, :n]]
        kc = d.values("k1_cache", d.k1_cache[used])
        kc2 = d.values("k2_cache", d.k2_cache[used])
        vc = d.values("v_cache", d.v_cache[used])
        return oracle.decode(d.f32("q1")[seqs], d.f32("q2")[seqs], kc, kc2, vc, table, d.ctx_len[seqs],
                             self.lam64, depth=d.depth, norm=norm, gamma=gamma, window=window)


def small(B=6, lens=None, H=8, H_kv=2, seed=0, max_pages=16):
    if lens is None:
        return W.decode_v2(seed=seed, B=B, H=H, H_kv=H_kv, max_pages=max_pages, ctx_lo=1, ctx_hi=max_pages * 64)
    return W.decode_v2(seed=seed, B=len(lens), H=H, H_kv=H_kv, max_pages=max_pages, ctx_len=np.array(lens))


@pytest.mark.parametrize("lens", [[1, 63, 64, 65, 128, 1000], [1024, 777, 5, 129]])
@pytest.mark.parametrize("split_pages", [0, 1, 3, 7, 1 << 20])
def test_decode_ragged(torch, da, lens, split_pages):
    c = DecodeCase(small(lens=lens), torch, da)
    say(f"decode lens {lens} split_pages {split_pages}")
    check(c.run(split_pages=split_pages).float().cpu().numpy(), c.oracle(), "bf16", "decode")


@pytest.mark.parametrize("split_pages", [0, 50, 1 << 20])
def test_decode_long_ranges(torch, da, split_pages):
    # sequences of more than 64 pages: a work-group's range spans page-id
    # chunks and, with few work-groups, several whole sequences
    lens = [5000, 300, 9000, 4480]
    c = DecodeCase(small(lens=lens, H=4, H_kv=2, seed=11, max_pages=160), torch, da)
    say(f"decode long lens {lens} split_pages {split_pages}")
    check(c.run(split_pages=split_pages).float().cpu().numpy(), c.oracle(), "bf16", "decode long")


def test_decode_all_lengths_invalid(torch, da):
    d = small(lens=[64, 100], seed=12)
    d.ctx_len[:] = [0, 16 * 64 + 1]
    c = DecodeCase(d, torch, da)
    err = torch.zeros(1, dtype=torch.int32, device=dev())
    out = c.run(dev_err=err).float().cpu().numpy()
    assert err.item() == 2 and np.all(out == 0)


@pytest.mark.parametrize("H,H_kv", [(8, 8), (16, 2), (4, 4), (6, 2)])
def test_decode_groupings(torch, da, H, H_kv):
    c = DecodeCase(small(B=5, H=H, H_kv=H_kv, seed=H), torch, da)
    say(f"decode H {H} H_kv {H_kv}")
    check(c.run().float().cpu().numpy(), c.oracle(), "bf16", "decode grouping")


def test_decode_rms_norm(torch, da):
    c = DecodeCase(small(B=4, seed=5), torch, da)
    gamma = np.random.default_rng(5).uniform(0.9, 1.1, (c.d.H, 128)).astype(np.float32)
    got = c.run(norm=True, gamma=torch.from_numpy(gamma).to(dev())).float().cpu().numpy()
    check(got, c.oracle(norm=True, gamma=gamma), "bf16", "decode RMS norm")


def test_decode_page_permutation_is_bitwise_invariant(torch, da):
    d = small(B=4, seed=6)
    c = DecodeCase(d, torch, da)
    a = c.run().clone()
    perm = np.random.default_rng(1).permutation(d.num_pages)
    inv = np.argsort(perm)  # new physical page of old page p is inv[p]
    kc = np.empty_like(d.k1_cache)
    vc = np.empty_like(d.v_cache)
    kc[inv] = d.k1_cache
    vc[inv] = d.v_cache
    table = np.where(d.page_table >= 0, inv[np.maximum(d.page_table, 0)], -1).astype(np.int32)
    c.kc, c.vc = to_dev(kc, "bf16"), to_dev(vc, "bf16")
    c.table = torch.from_numpy(table).to(dev())
    assert torch.equal(a, c.run())


def test_decode_matches_prefill_last_row(torch, da):
    # one sequence of length L stored in pages in order equals the last row of
    # a causal V2 prefill over the same tokens
    L, H, H_kv = 300, 8, 2
    d = small(lens=[L], H=H, H_kv=H_kv, seed=8)
    c = DecodeCase(d, torch, da)
    dec = c.run().float()
    npg = (L + 63) // 64
    pages = d.page_table[0, :npg]
    k = d.k1_cache[pages].transpose(1, 0, 2, 3).reshape(H_kv, npg * 64, 128)[:, :L][None]
    v = d.v_cache[pages].transpose(1, 0, 2, 3).reshape(H_kv, npg * 64, 128)[:, :L][None]
    q = np.zeros((1, 2 * H, L, 128), np.uint16)
    q[0, :, L - 1] = d.q_full[0]
    qd = to_dev(q, "bf16")
    kd = to_dev(k, "bf16")
    pre = da.prefill(qd[:, 0::2], qd[:, 1::2], kd, kd, to_dev(v, "bf16"), c.lam, depth=d.depth,
                     causal=True)
    diff = (pre[0, :, L - 1].float() - dec[0]).abs().max().item()
    assert diff <= 1.6e-2, diff


def test_decode_reports_bad_page_and_length(torch, da):
    d = small(lens=[200, 130, 64], seed=9)
    table0 = d.page_table.copy()
    d.page_table[1, 2] = d.num_pages + 5   # out of range: its tokens (128, 129) are masked, bit 0
    d.ctx_len[2] = 0                        # invalid length: bit 1, zero output
    c = DecodeCase(d, torch, da)
    err = torch.zeros(1, dtype=torch.int32, device=dev())
    out = c.run(dev_err=err).float().cpu().numpy()
    assert err.item() == 3
    kc, vc = d.f32("k1_cache"), d.f32("v_cache")
    q1, q2 = d.f32("q1"), d.f32("q2")
    ref0 = oracle.decode(q1[:1], q2[:1], kc, kc, vc, table0[:1], np.array([200], np.int32), c.lam64,
                         depth=d.depth, norm=False)
    check(out[:1], ref0, "bf16", "decode seq 0 beside bad entries")
    # sequence 1 equals attention over its first two pages (the bad page is masked)
    table1 = table0[1:2].copy()
    table1[0, 2:] = -1
    ref1 = oracle.decode(q1[1:2], q2[1:2], kc, kc, vc, table1, np.array([128], np.int32), c.lam64,
                         depth=d.depth, norm=False)
    check(out[1:2], ref1, "bf16", "decode seq 1 with its bad page masked")
    assert np.all(out[2] == 0)


def test_decode_v2_full(torch, da):
    d = W.decode_v2()
    say(f"decode_v2 full: 64 sequences, {d.num_pages} pages, context {d.ctx_len.min()}..{d.ctx_len.max()}")
    c = DecodeCase(d, torch, da)
    out = c.run().float().cpu().numpy()
    check(out, c.oracle(), "bf16", "decode_v2 all sequences and heads")


# ---- V1 form: d_qk 64, separate K1 and K2 caches, value width 128, RMS norm


def small_v1(lens, H=8, H_kv=2, seed=0, max_pages=16):
    return W.decode_v1(seed=seed, B=len(lens), H=H, H_kv=H_kv, max_pages=max_pages,
                       ctx_len=np.array(lens))


@pytest.mark.parametrize("lens", [[1, 63, 64, 65, 128, 1000], [1024, 777, 5, 129]])
@pytest.mark.parametrize("split_pages", [0, 1, 3, 1 << 20])
def test_decode_v1_ragged(torch, da, lens, split_pages):
    c = DecodeCase(small_v1(lens, seed=21), torch, da)
    say(f"decode V1 lens {lens} split_pages {split_pages}")
    check(c.run(split_pages=split_pages).float().cpu().numpy(), c.oracle(), "bf16", "decode V1")


@pytest.mark.parametrize("H,H_kv", [(8, 8), (16, 2), (6, 2)])
def test_decode_v1_groupings(torch, da, H, H_kv):
    c = DecodeCase(small_v1([300, 64, 1, 700, 129], H=H, H_kv=H_kv, seed=22 + H), torch, da)
    say(f"decode V1 H {H} H_kv {H_kv}")
    check(c.run().float().cpu().numpy(), c.oracle(), "bf16", "decode V1 grouping")


def test_decode_v1_no_norm_and_swapped_caches(torch, da):
    # without the norm the V1 result is O1 - lambda O2; swapping (Q1, K1) with
    # (Q2, K2) must use each branch's own key cache, checked against the oracle
    d = small_v1([200, 500, 64], seed=23)
    c = DecodeCase(d, torch, da)
    check(c.run(norm=False).float().cpu().numpy(), c.oracle(norm=False), "bf16", "decode V1 no norm")
    c.q1, c.q2, c.kc, c.kc2 = c.q2, c.q1, c.kc2, c.kc
    d.q1, d.q2, d.k1_cache, d.k2_cache = d.q2, d.q1, d.k2_cache, d.k1_cache
    check(c.run(norm=False).float().cpu().numpy(), c.oracle(norm=False), "bf16", "decode V1 swapped")


def test_decode_v1_matches_prefill_last_row(torch, da):
    # one V1 sequence stored in pages in order equals the last row of a causal
    # V1 prefill (with the norm) over the same tokens
    L, H, H_kv = 333, 4, 4
    d = small_v1([L], H=H, H_kv=H_kv, seed=24)
    c = DecodeCase(d, torch, da)
    dec = c.run().float()
    npg = (L + 63) // 64
    pages = d.page_table[0, :npg]

    def gather(cache, width):
        return cache[pages].transpose(1, 0, 2, 3).reshape(H_kv, npg * 64, width)[:, :L][None]

    k1, k2, v = gather(d.k1_cache, 64), gather(d.k2_cache, 64), gather(d.v_cache, 128)
    q1 = np.zeros((1, H, L, 64), np.uint16)
    q2 = np.zeros((1, H, L, 64), np.uint16)
    q1[0, :, L - 1] = d.q1[0]
    q2[0, :, L - 1] = d.q2[0]
    pre = da.prefill(to_dev(q1, "bf16"), to_dev(q2, "bf16"), to_dev(k1, "bf16"), to_dev(k2, "bf16"),
                     to_dev(v, "bf16"), c.lam, depth=d.depth, causal=True, norm=True, gamma=c.gamma,
                     eps=d.eps)
    diff = (pre[0, :, L - 1].float() - dec[0]).abs().max().item()
    assert diff <= 1.6e-2, diff


def test_decode_v1_full(torch, da):
    d = W.decode_v1()
    say(f"decode_v1 full: 64 sequences, {d.num_pages} pages, context {d.ctx_len.min()}..{d.ctx_len.max()}")
    c = DecodeCase(d, torch, da)
    out = c.run().float().cpu().numpy()
    check(out, c.oracle(), "bf16", "decode_v1 all sequences and heads")


# ---- causal sliding window: the query sees its last W tokens


@pytest.mark.parametrize("form", ["v2", "v1"])
@pytest.mark.parametrize("window", [1, 15, 64, 65, 200, 1000])
@pytest.mark.parametrize("split_pages", [0, 2])
def test_decode_sliding_window(torch, da, form, window, split_pages):
    lens = [1, 63, 64, 65, 128, 1000, 333]
    d = small_v1(lens, seed=50 + window) if form == "v1" else small(lens=lens, seed=50 + window)
    c = DecodeCase(d, torch, da)
    say(f"decode {form} window {window} split_pages {split_pages}")
    check(c.run(window=window, split_pages=split_pages).float().cpu().numpy(), c.oracle(window=window),
          "bf16", f"decode {form} W={window}")


def test_decode_window_at_least_len_is_plain_bitwise(torch, da):
    d = small(lens=[300, 64, 1000, 5], seed=60)
    c = DecodeCase(d, torch, da)
    plain = c.run().clone()
    for w in (1000, 1024, 1 << 20):
        assert torch.equal(c.run(window=w), plain), w


def test_decode_v1_group_norm(torch, da):
    d = small_v1([300, 64, 1, 700, 129], seed=70)
    d.norm = "group"
    c = DecodeCase(d, torch, da)
    say("decode V1 GroupNorm")
    check(c.run().float().cpu().numpy(), c.oracle(), "bf16", "decode V1 GroupNorm")


# ---- fp8 (OCP e4m3) KV caches with per-tensor scales; the oracle reads the
# dequantised values (scale * code), exactly what the kernel contracts with


def small_fp8(lens, H=8, H_kv=2, seed=0, max_pages=16, form="v2"):
    mk = W.decode_v1 if form == "v1" else W.decode_v2
    return mk(seed=seed, B=len(lens), H=H, H_kv=H_kv, max_pages=max_pages, ctx_len=np.array(lens),
              kv_dtype="fp8")


@pytest.mark.parametrize("form", ["v2", "v1"])
@pytest.mark.parametrize("lens", [[1, 63, 64, 65, 128, 1000], [1024, 777, 5, 129]])
@pytest.mark.parametrize("split_pages", [0, 1, 3, 1 << 20])
def test_decode_fp8_ragged(torch, da, form, lens, split_pages):
    c = DecodeCase(small_fp8(lens, seed=80, form=form), torch, da)
    say(f"decode fp8 {form} lens {lens} split_pages {split_pages}")
    check(c.run(split_pages=split_pages).float().cpu().numpy(), c.oracle(), "bf16", f"decode fp8 {form}")


@pytest.mark.parametrize("form,H,H_kv", [("v2", 8, 8), ("v2", 16, 2), ("v2", 6, 2), ("v1", 16, 2), ("v1", 4, 4)])
def test_decode_fp8_groupings(torch, da, form, H, H_kv):
    c = DecodeCase(small_fp8([300, 64, 1, 700, 129], H=H, H_kv=H_kv, seed=81 + H, form=form), torch, da)
    say(f"decode fp8 {form} H {H} H_kv {H_kv}")
    check(c.run().float().cpu().numpy(), c.oracle(), "bf16", "decode fp8 grouping")


@pytest.mark.parametrize("form", ["v2", "v1"])
@pytest.mark.parametrize("window", [1, 65, 1000])
def test_decode_fp8_sliding_window(torch, da, form, window):
    c = DecodeCase(small_fp8([1, 63, 64, 65, 128, 1000, 333], seed=90 + window, form=form), torch, da)
    say(f"decode fp8 {form} window {window}")
    check(c.run(window=window).float().cpu().numpy(), c.oracle(window=window), "bf16",
          f"decode fp8 {form} W={window}")


def test_decode_fp8_group_norm(torch, da):
    d = small_fp8([300, 64, 1, 700, 129], seed=95, form="v1")
    d.norm = "group"
    c = DecodeCase(d, torch, da)
    check(c.run().float().cpu().numpy(), c.oracle(), "bf16", "decode fp8 V1 GroupNorm")


def test_decode_fp8_scales_and_nan_codes_past_the_end(torch, da):
    # other scales (k and v differ), and NaN codes (0x7f, 0xff) in the slots
    # past every sequence's end: those tokens are masked, so they cannot reach
    # the output
    d = small_fp8([100, 64, 1, 250], seed=96)
    d.k_scale, d.v_scale = 0.03125, 0.0125
    for b, L in enumerate(d.ctx_len):
        last = d.page_table[b, (L - 1) // 64]
        tail = L % 64
        if tail:
            d.k1_cache[last, :, tail:] = 0x7f
            d.v_cache[last, :, tail:] = 0xff
    c = DecodeCase(d, torch, da)
    got = c.run().float().cpu().numpy()
    assert np.all(np.isfinite(got))
    check(got, c.oracle(), "bf16", "decode fp8 scales / NaN tail")


def test_decode_fp8_page_permutation_is_bitwise_invariant(torch, da):
    d = small_fp8([200, 1000, 64, 5], seed=97)
    c = DecodeCase(d, torch, da)
    a = c.run().clone()
    perm = np.random.default_rng(2).permutation(d.num_pages)
    inv = np.argsort(perm)
    kc = np.empty_like(d.k1_cache)
    vc = np.empty_like(d.v_cache)
    kc[inv] = d.k1_cache
    vc[inv] = d.v_cache
    table = np.where(d.page_table >= 0, inv[np.maximum(d.page_table, 0)], -1).astype(np.int32)
    c.kc, c.vc = to_dev(kc, "u8"), to_dev(vc, "u8")
    c.table = torch.from_numpy(table).to(dev())
    assert torch.equal(a, c.run())


def test_decode_fp8_float8_tensor_input(torch, da):
    # torch.float8_e4m3fn caches are accepted as well as their uint8 codes
    d = small_fp8([300, 64, 129], seed=98)
    c = DecodeCase(d, torch, da)
    a = c.run().clone()
    c.kc, c.vc = c.kc.view(torch.float8_e4m3fn), c.vc.view(torch.float8_e4m3fn)
    assert torch.equal(a, c.run())


def test_decode_v2_fp8_full(torch, da):
    d = W.decode_v2_fp8()
    say(f"decode_v2_fp8 full: 64 sequences, {d.num_pages} pages")
    c = DecodeCase(d, torch, da)
    out = c.run().float().cpu().numpy()
    check(out, c.oracle(), "bf16", "decode_v2_fp8 all sequences and heads")
