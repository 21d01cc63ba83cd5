"""Helpers for the GPU parity tests: device copies of the seeded workloads,
calls through the C ABI (via the Python binding) and the tolerance check."""
from __future__ import annotations

import sys

import numpy as np

import oracle
import workloads as W

# tolerances: bf16 inputs with fp32 accumulation, and the fp32 path
BF16_MAX_ABS = 2e-2
BF16_REL_FRO = 1e-2
F32_MAX_ABS = 1e-5


_PYTEST_CONFIG = None  # set by conftest.py: lets say(..., live=True) bypass output capture


def say(msg: str, live: bool = False):
    """Print a progress line (kept with the test's captured output). live:
    also write it straight to the terminal while the test runs, so that a
    check lasting minutes shows its progress as it goes."""
    print(msg, flush=True)
    sys.stdout.flush()
    cm = _PYTEST_CONFIG.pluginmanager.getplugin("capturemanager") if live and _PYTEST_CONFIG else None
    if cm is not None:
        with cm.global_and_fixture_disabled():
            print(msg, flush=True)


def dev():
    import torch
    return torch.device("cuda:0")


def to_dev(x: np.ndarray, dtype: str):
    import torch
    x = np.ascontiguousarray(x)
    if dtype == "bf16":
        return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(dev())
    return torch.from_numpy(x).to(dev())


def check(got: np.ndarray, ref: np.ndarray, dtype: str, what: str = ""):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    d = np.abs(got - ref)
    mx = float(d.max()) if d.size else 0.0
    where = np.unravel_index(int(d.argmax()), d.shape) if d.size else ()
    if dtype == "bf16":
        fro = float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300))
        say(f"  {what}: max|d| {mx:.3e} at {tuple(int(x) for x in where)} rel-fro {fro:.3e} over {d.size} elements")
        assert mx <= BF16_MAX_ABS, f"{what}: max abs error {mx}"
        assert fro <= BF16_REL_FRO, f"{what}: relative Frobenius error {fro}"
    else:
        say(f"  {what}: max|d| {mx:.3e} over {d.size} elements")
        assert mx <= F32_MAX_ABS, f"{what}: max abs error {mx}"
    return mx


def check_all_rows_by_head(c, out, what: str):
    """bf16 check of every row of a prefill output [B, H, N, d_v] (numpy),
    the oracle evaluated one (batch, head) at a time with a progress line per
    head; max abs and relative Frobenius errors accumulate over all rows."""
    p = c.p
    mx, dd, rr = 0.0, 0.0, 0.0
    for b in range(p.B):
        for h in range(p.H):
            rows = (b * p.H + h) * p.N + np.arange(p.N, dtype=np.int64)
            ref = c.oracle(rows=rows)
            got = np.asarray(out[b, h], np.float64)
            assert np.all(np.isfinite(got)), f"{what}: non-finite output in head {h}"
            diff = got - ref
            mx = max(mx, float(np.abs(diff).max()))
            dd += float((diff * diff).sum())
            rr += float((ref * ref).sum())
            say(f"  {what}: batch {b} head {h} done, max|d| so far {mx:.3e}", live=True)
    fro = (dd / max(rr, 1e-300)) ** 0.5
    say(f"  {what}: max|d| {mx:.3e} rel-fro {fro:.3e} over {out.size} elements", live=True)
    assert mx <= BF16_MAX_ABS, f"{what}: max abs error {mx}"
    assert fro <= BF16_REL_FRO, f"{what}: relative Frobenius error {fro}"


class PrefillCase:
    """A workload on the device plus its oracle."""

    def __init__(self, p: W.Prefill):
        import torch
        import differential_attention_amd as da
        self.p = p
        self.da = da
        dt = p.dtype
        if p.q_full is not None:
            qf = to_dev(p.q_full, dt)
            self.q1, self.q2 = qf[:, 0::2], qf[:, 1::2]
        else:
            self.q1, self.q2 = to_dev(p.q1, dt), to_dev(p.q2, dt)
        self.k1 = to_dev(p.k1, dt)
        self.k2 = self.k1 if p.shared_k else to_dev(p.k2, dt)
        self.v = to_dev(p.v, dt)
        self.gamma = torch.from_numpy(p.gamma).to(dev()) if p.norm else None
        vecs = [torch.from_numpy(x).to(dev()) for x in (p.lam_q1, p.lam_k1, p.lam_q2, p.lam_k2)]
        self.lam = da.lambda_(*vecs, p.depth)
        self.lam64 = oracle.lambda_(p.lam_q1, p.lam_k1, p.lam_q2, p.lam_k2, p.depth)

    def run(self, lam=None, **kw):
        p = self.p
        args = dict(depth=p.depth, causal=p.causal, norm=p.norm, gamma=self.gamma, eps=p.eps)
        args.update(kw)
        return self.da.prefill(self.q1, self.q2, self.k1, self.k2, self.v,
                               self.lam if lam is None else lam, **args)

    def oracle(self, rows=None, lam64=None, window: int = 0):
        p = self.p
        k1 = p.f32("k1")
        k2 = k1 if p.shared_k else p.f32("k2")
        return oracle.prefill(p.f32("q1"), p.f32("q2"), k1, k2, p.f32("v"),
                              self.lam64 if lam64 is None else lam64, depth=p.depth,
                              causal=p.causal, norm=p.norm, gamma=p.gamma, eps=p.eps, rows=rows,
                              window=window)


def gather_rows(out, rows: np.ndarray, H: int, N: int) -> np.ndarray:
    """Rows (flat ids (b*H + h)*N + i) of a [B, H, N, d] device tensor, as fp64 numpy."""
    import torch
    flat = out.reshape(-1, out.shape[-1])
    idx = torch.from_numpy(rows).to(out.device)
    return flat.index_select(0, idx).float().cpu().numpy().astype(np.float64)


def sampled_rows(B: int, H: int, N: int, seed: int, n_rand: int = 64, edge: int = 32, extra=None):
    rng = np.random.default_rng(seed)
    out = []
    for b in range(B):
        for h in range(H):
            rs = W.sample_rows(N, rng, n_rand=n_rand, edge=edge)
            if extra is not None:
                rs = np.union1d(rs, extra(b, h))
            out.append((b * H + h) * N + rs)
    return np.concatenate(out)
