#!/usr/bin/env python3
"""Benchmark of the differential-attention hot path on one MI355X.

One step is one pass of the whole path over one batch of synthetic input:
  lambda   diffattn_lambda for the prefill heads
  prefill  diffattn_prefill on longctx_v1: V1 form, B 1, H 8, N 65536,
           d_qk 64, d_v 128, causal, bf16, RMSNorm epilogue, planted keys
           (the largest single-GPU prefill workload)
  lambda   diffattn_lambda for the decode heads
  decode   diffattn_decode on decode_v2: V2 form, 64 sequences, context
           U{8192..32768}, 8 KV heads, 64 query heads, d 128, page 64, bf16
Inputs are resident in HBM before the timed region. Each call is bracketed by
HIP events on the stream the library launches on (the prefill runs for
milliseconds, so the host stays ahead of the device and the events time the
kernels, not the launches). The two other prefill workloads, prefill_v2
(V2 GQA, N 16384) and prefill_v1 (V1, B 2, H 16, N 4096), are timed after the
steps, each as a batch of back-to-back calls between two events.

Output: one JSON line. ``value`` is the step's prefill throughput, FLOPs
counted as B*H*(N^2/2)*2*(2*d_qk + 2*d_v) (both branches, QK and PV, causal
pairs halved), over the mean time of the lambda + prefill part of a step; the
``decode`` object gives the decode part's algorithmic HBM bytes (every visible
token's K and V once, plus Q, output and page-table entries) per second;
``prefill_other`` the other two prefill workloads. ``roofline`` is the
step's prefill kernel against the bf16 dense MFMA peak, ``decode.roofline``
the decode call against HBM bandwidth. ``cpu_baseline`` times the fp64 CPU
oracle on a bounded random sample of the headline workload's rows, with one
entry per workload under ``per_workload``.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

BF16_PEAK_TFLOPS = 2516.6   # 256 CU x 4096 flop/clk x 2.4 GHz, dense
HBM_PEAK_GBS = 8000.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def prefill_flops(B, H, N, dqk, dv, window=0):
    """Both branches, QK and PV, per visible (query, key) pair; causal pairs
    counted as N^2/2, and with a causal window W < N as W^2/2 + (N - W) W."""
    pairs = N * N / 2.0 if not window or window >= N else window * window / 2.0 + (N - window) * window
    return B * H * pairs * 2.0 * (2 * dqk + 2 * dv)


def backward_flops(B, H, N, dqk, dv, window=0):
    """Algorithmic FLOPs of the prefill's backward per visible (query, key)
    pair: both branches' scores recomputed (2 x 2 d_qk), the output-gradient
    product dy V^T shared by the branches (2 d_v), dV from the combined weight
    (2 d_v), dQ and dK of both branches (4 x 2 d_qk): 12 d_qk + 4 d_v."""
    pairs = N * N / 2.0 if not window or window >= N else window * window / 2.0 + (N - window) * window
    return B * H * pairs * (12 * dqk + 4 * dv)


def decode_bytes(d):
    """Algorithmic HBM bytes of one decode call: every visible token's keys
    (one cache, or one per branch) and values once, the queries, the output,
    the page-table entries used and ctx_len (plus gamma for the V1 norm)."""
    return decode_bytes_of(d, d.ctx_len)


def decode_bytes_of(d, ctx_len):
    """decode_bytes for the sequences whose lengths are ctx_len."""
    L = np.asarray(ctx_len).astype(np.int64)
    B = L.size
    nk = 1 if d.shared_k else 2
    kv = int(L.sum()) * d.H_kv * (nk * d.d_qk + d.d_v) * d.kv_bytes  # bf16: 2 bytes, fp8: 1
    q = B * 2 * d.H * d.d_qk * 2
    out = B * d.H * d.d_v * 2
    table = int(((L + d.page - 1) // d.page).sum()) * 4 + B * 4
    gamma = d.H * d.d_v * 4 if d.norm else 0
    return kv + q + out + table + gamma


# sources of the kernels each workload runs (their hash keys the stored counters)
KERNEL_SOURCES = {
    "prefill_v1": ["prefill_bf16.hip", "tiles.hpp", "common.hpp"],
    "prefill_v2": ["prefill_bf16.hip", "tiles.hpp", "common.hpp"],
    "longctx_v1": ["prefill_bf16.hip", "tiles.hpp", "common.hpp"],
    "decode_v2": ["decode.hip", "common.hpp"],
    "decode_v1": ["decode.hip", "common.hpp"],
    "decode_v2_fp8": ["decode.hip", "common.hpp"],
    "backward_v1": ["backward.hip", "tiles.hpp", "common.hpp"],
    "backward_v2": ["backward.hip", "tiles.hpp", "common.hpp"],
}


def kernel_source_hash(name):
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "differential_attention_amd", "csrc")
    for fn in KERNEL_SOURCES.get(name, []):
        with open(os.path.join(csrc, fn), "rb") as f:
            h.update(fn.encode() + f.read())
    return h.hexdigest()[:16]


def load_traffic(name):
    """HBM bytes per launch (calibrated FETCH_SIZE + WRITE_SIZE) from the
    committed counter summary, or None if it was taken on other kernel sources."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if name not in KERNEL_SOURCES or not os.path.exists(path):
        return None
    try:
        with open(path) as f:
            e = json.load(f).get(name)
        if e and e.get("source_hash") == kernel_source_hash(name):
            return e.get("bytes_per_launch")
    except (OSError, ValueError):
        return None
    return None


def cpu_model() -> str:
    """The host CPU's model name, as /proc/cpuinfo gives it."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown CPU"


def cpu_baseline_prefill(p, budget_s, seed=1234):
    """Oracle FLOP/s on a random sample of prefill rows (same inputs): about
    budget_s seconds of oracle time, FLOPs counted per visible key as for the
    GPU (both branches, QK and PV)."""
    import oracle
    rng = np.random.default_rng(seed)
    lam64 = oracle.lambda_(p.lam_q1, p.lam_k1, p.lam_q2, p.lam_k2, p.depth)
    q1, q2, k1, v = (p.f32(n) for n in ("q1", "q2", "k1", "v"))
    k2 = k1 if p.shared_k else p.f32("k2")
    per_key = 2 * (2 * p.d_qk + 2 * p.d_v)
    total = p.B * p.H * p.N

    def run(nrows):
        rows = np.sort(rng.choice(total, size=nrows, replace=False)).astype(np.int64)
        visible = ((rows % p.N) + 1) if p.causal else np.full(rows.size, p.N)
        flops = float(visible.sum()) * per_key
        t0 = time.perf_counter()
        oracle.prefill(q1, q2, k1, k2, v, lam64, depth=p.depth, causal=p.causal, norm=p.norm,
                       gamma=p.gamma, eps=p.eps, rows=rows)
        return flops, time.perf_counter() - t0

    f0, t0 = run(min(total, 64))  # calibration
    n = int(min(total, max(64, 64 * budget_s / max(t0, 1e-3))))
    f, t = run(n)
    return {"value": f / t / 1e12, "unit": "TFLOP/s", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"{n} random query rows of {p.name} (of {total}), fp64, {t:.1f} s on {cpu_model()}, "
                      f"FLOPs counted per visible key as for the GPU"}


def cpu_baseline_decode(d, budget_s, seed=1234):
    """Oracle GB/s (algorithmic bytes, as for the GPU) on a random sample of
    the decode's sequences. The sampled sequences' pages are gathered into a
    small pool (the page table renumbered to it) before the timed call, so no
    more than their share of the cache is widened to fp32."""
    import oracle
    rng = np.random.default_rng(seed)
    lam64 = oracle.lambda_(d.lam_q1, d.lam_k1, d.lam_q2, d.lam_k2, d.depth)

    def run(nseq):
        bs = np.sort(rng.choice(d.B, size=nseq, replace=False))
        table, ctx = d.page_table[bs], d.ctx_len[bs]
        used = np.unique(table[table >= 0])
        remap = np.full(d.num_pages, -1, np.int32)
        remap[used] = np.arange(used.size, dtype=np.int32)
        sub_table = np.where(table >= 0, remap[np.maximum(table, 0)], -1).astype(np.int32)
        k1c = d.values("k1_cache", d.k1_cache[used])
        k2c = k1c if d.shared_k else d.values("k2_cache", d.k2_cache[used])
        vc = d.values("v_cache", d.v_cache[used])
        q1, q2 = d.f32("q1")[bs], d.f32("q2")[bs]
        t0 = time.perf_counter()
        oracle.decode(q1, q2, k1c, k2c, vc, sub_table, ctx, lam64, depth=d.depth, norm=d.norm, gamma=d.gamma,
                      eps=d.eps)
        return float(decode_bytes_of(d, ctx)), time.perf_counter() - t0

    b0, t0 = run(1)
    n = int(min(d.B, max(1, budget_s / max(t0, 1e-3))))
    b, t = run(n)
    return {"value": b / t / 1e9, "unit": "GB/s", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"{n} random sequences of {d.name} (of {d.B}), fp64, {t:.1f} s on {cpu_model()}, "
                      f"bytes counted as for the GPU"}


def single_workload(args, torch, da, W, dev):
    """Time one workload alone: one call per step, HIP events around each call."""
    stream = torch.cuda.current_stream()

    def to_dev(x, dtype="bf16"):
        x = np.ascontiguousarray(x)
        if dtype == "bf16":
            return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(x).to(dev)

    name = args.workload
    if name in ("gemm", "gemm_zeros"):
        # the practical bf16 matrix-core ceiling: a large library GEMM (torch.matmul,
        # hipBLASLt) on N(0,1) operands; gemm_zeros multiplies all-zero operands, whose
        # lower switching power lets the engine clock run higher
        n = args.gemm_n
        g = torch.Generator(device=dev).manual_seed(5)
        if name == "gemm":
            A = torch.randn((n, n), generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
            Bm = torch.randn((n, n), generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
        else:
            A = torch.zeros((n, n), device=dev, dtype=torch.bfloat16)
            Bm = torch.zeros((n, n), device=dev, dtype=torch.bfloat16)
        C = torch.empty((n, n), device=dev, dtype=torch.bfloat16)
        call = lambda: torch.matmul(A, Bm, out=C)
        work, unit, metric, bound = 2.0 * n ** 3, "TFLOP/s", "bf16 GEMM TFLOP/s (torch.matmul)", "mfma"
        desc = (f"torch.matmul bf16 {n} x {n} x {n}, "
                + ("N(0,1) operands" if name == "gemm" else "all-zero operands"))
    elif name == "copy":
        n = 1 << 31  # 2 Gi bf16 elements = 4 GiB read + 4 GiB written
        src = torch.empty(n, dtype=torch.bfloat16, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        call = lambda: dst.copy_(src)
        work, unit, metric, bound = 2.0 * n * 2, "GB/s", "device copy GB/s (read + write)", "hbm"
        desc = "torch copy_ of 2^31 bf16 elements (4 GiB read, 4 GiB written)"
    elif name in ("decode_v2", "decode_v1", "decode_v2_fp8"):
        d = getattr(W, name)()
        if d.q_full is not None:
            qd = to_dev(d.q_full)
            q1, q2 = qd[:, 0::2], qd[:, 1::2]
        else:
            q1, q2 = to_dev(d.q1), to_dev(d.q2)
        kv = "bf16" if d.kv_dtype == "bf16" else "u8"  # fp8 caches as their uint8 codes
        kc, vc = to_dev(d.k1_cache, kv), to_dev(d.v_cache, kv)
        kc2 = None if d.shared_k else to_dev(d.k2_cache, kv)
        table, ctx = torch.from_numpy(d.page_table).to(dev), torch.from_numpy(d.ctx_len).to(dev)
        lam = da.lambda_(*(torch.from_numpy(x).to(dev) for x in (d.lam_q1, d.lam_k1, d.lam_q2, d.lam_k2)), d.depth)
        gamma = torch.from_numpy(d.gamma).to(dev) if d.norm else None
        out = torch.empty((d.B, d.H, d.d_v), dtype=torch.bfloat16, device=dev)
        kw = dict(depth=d.depth, norm=d.norm, gamma=gamma, eps=d.eps, k2_cache=kc2, k_scale=d.k_scale,
                  v_scale=d.v_scale)
        ws = torch.empty(da.decode_workspace_bytes(q1, q2, kc, vc, table, ctx, lam, **kw),
                         dtype=torch.uint8, device=dev)
        call = lambda: da.decode(q1, q2, kc, vc, table, ctx, lam, out=out, workspace=ws, **kw)
        work, unit, metric, bound = decode_bytes(d), "GB/s", "decode GB/s (algorithmic HBM bytes)", "hbm"
        if name == "decode_v2":
            desc = "decode_v2: V2 paged decode, 64 seqs, ctx U{8192..32768}, 8 KV / 64 Q heads, d 128, page 64"
        elif name == "decode_v2_fp8":
            desc = ("decode_v2_fp8: decode_v2 with an fp8 e4m3 KV cache (per-tensor scales), bf16 queries "
                    "and output")
        else:
            desc = ("decode_v1: V1 paged decode, 64 seqs, ctx U{8192..32768}, 8 KV / 32 heads, d_qk 64 "
                    "(K1, K2 caches), d_v 128, page 64, RMS norm")
    elif name in ("backward_v1", "backward_v2"):
        p = W.prefill_v1() if name == "backward_v1" else W.prefill_v2()
        if p.q_full is not None:
            qf = to_dev(p.q_full)
            q1, q2 = qf[:, 0::2], qf[:, 1::2]
        else:
            q1, q2 = to_dev(p.q1), to_dev(p.q2)
        k1 = to_dev(p.k1)
        k2 = k1 if p.shared_k else to_dev(p.k2)
        v = to_dev(p.v)
        gamma = torch.from_numpy(p.gamma).to(dev) if p.norm else None
        lam = da.lambda_(*(torch.from_numpy(x).to(dev) for x in (p.lam_q1, p.lam_k1, p.lam_q2, p.lam_k2)), p.depth)
        stats = da.prefill_stats(q1, v)
        win = args.window
        da.prefill(q1, q2, k1, k2, v, lam, depth=p.depth, causal=p.causal, norm=p.norm, gamma=gamma, eps=p.eps,
                   window=win, stats=stats)
        dout = torch.randn((p.B, p.H, p.N, p.d_v), generator=torch.Generator().manual_seed(7)).to(
            dev, torch.bfloat16)
        kw = dict(depth=p.depth, causal=p.causal, norm=p.norm, gamma=gamma, eps=p.eps, window=win)
        # the gradient tensors and workspace come from torch's caching allocator
        # (no device allocation after the first call)
        call = lambda: da.backward(q1, q2, k1, k2, v, lam, stats, dout, **kw)
        work = backward_flops(p.B, p.H, p.N, p.d_qk, p.d_v, win)
        unit, metric, bound = "TFLOP/s", "prefill backward TFLOP/s (algorithmic)", "mfma"
        desc = (f"{name}: gradients of the {'prefill_v1' if name == 'backward_v1' else 'prefill_v2'} "
                f"prefill (B {p.B}, H {p.H}, H_kv {p.H_kv}, N {p.N}, d_qk {p.d_qk}, d_v {p.d_v}), fp32 gradients")
        if win:
            desc += f", causal window {win}"
    else:
        if name == "copy_lds":
            # every key/value byte read once, by one work-group, through the
            # LDS-DMA buffer loads: a non-causal V1 prefill with one 192-row
            # block per head (no sharing between work-groups, no fast-sweep
            # sample since rows see fewer than 256 keys), 256 heads
            p = W.prefill_v1(seed=31, B=4, H=64, N=192, causal=False)
        else:
            p = getattr(W, name)()
        dt = p.dtype
        if p.q_full is not None:
            qf = to_dev(p.q_full, dt)
            q1, q2 = qf[:, 0::2], qf[:, 1::2]
        else:
            q1, q2 = to_dev(p.q1, dt), to_dev(p.q2, dt)
        k1 = to_dev(p.k1, dt)
        k2 = k1 if p.shared_k else to_dev(p.k2, dt)
        v = to_dev(p.v, dt)
        gamma = torch.from_numpy(p.gamma).to(dev) if p.norm else None
        lam = da.lambda_(*(torch.from_numpy(x).to(dev) for x in (p.lam_q1, p.lam_k1, p.lam_q2, p.lam_k2)), p.depth)
        out = torch.empty((p.B, p.H, p.N, p.d_v), dtype=q1.dtype, device=dev)
        win = args.window
        call = lambda: da.prefill(q1, q2, k1, k2, v, lam, depth=p.depth, causal=p.causal, norm=p.norm,
                                  gamma=gamma, eps=p.eps, out=out, window=win)
        work = prefill_flops(p.B, p.H, p.N, p.d_qk, p.d_v, win)
        if not p.causal:
            work *= 2.0  # every (query, key) pair visible
        unit, metric, bound = "TFLOP/s", "prefill TFLOP/s", "mfma"
        desc = f"{name}: B {p.B}, H {p.H}, H_kv {p.H_kv}, N {p.N}, d_qk {p.d_qk}, d_v {p.d_v}, {p.dtype}"
        if win:
            desc += f", causal window {win}"
    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for a, b in evs:
        a.record(stream)
        call()
        b.record(stream)
    torch.cuda.synchronize()
    ms = float(np.mean([a.elapsed_time(b) for a, b in evs]))
    scale = 1e12 if unit == "TFLOP/s" else 1e9
    val = work / (ms * 1e-3) / scale
    peak = BF16_PEAK_TFLOPS if bound == "mfma" else HBM_PEAK_GBS
    dtype = "f32" if name == "tiny_v1" else "bf16"
    line = {"metric": metric, "value": val, "unit": unit, "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": dtype, "data": "synthetic", "config": {"workload": desc},
            "roofline": {"bound": bound, "achieved": val, "peak": peak, "unit": unit, "frac": val / peak,
                         "traffic": load_traffic(name)}}
    log(f"{name}: {ms * 1e3:.1f} us per call, {val:.1f} {unit} ({100 * val / peak:.1f}% of peak)")
    print(json.dumps(line), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--cpu-budget", type=float, default=15.0,
                    help="seconds of oracle time for the headline cpu_baseline (a third of it for each other workload)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--only", choices=["prefill", "decode"], default=None,
                    help="profiling aid: run only one part of the step")
    ap.add_argument("--workload", default="step",
                    choices=["step", "prefill_v1", "prefill_v2", "longctx_v1", "tiny_v1", "decode_v2",
                             "decode_v1", "decode_v2_fp8", "backward_v1", "backward_v2", "copy", "copy_lds", "gemm",
                             "gemm_zeros"],
                    help="step: the whole path (default); otherwise time one workload alone "
                         "(copy: a plain device copy of 4 GiB, and copy_lds: a prefill whose key/value bytes "
                         "are each read once through LDS-DMA loads, for calibrating HBM byte counters; gemm and "
                         "gemm_zeros: an n^3 bf16 library GEMM (n = --gemm-n) on N(0,1) or all-zero operands, the practical "
                         "matrix-core ceiling)")
    ap.add_argument("--gemm-n", type=int, default=8192, help="matrix size of the gemm workloads")
    ap.add_argument("--window", type=int, default=0,
                    help="causal sliding window for a single prefill workload (0 = none)")
    args = ap.parse_args()
    if args.window and args.workload in ("step", "copy", "gemm", "gemm_zeros", "decode_v2", "decode_v1", "decode_v2_fp8",
                                         "tiny_v1"):
        ap.error("--window applies to a single prefill workload")
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: this library has no multi-GPU path "
              "(sharding is by (batch, KV head) with no communication; see the design notes)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import differential_attention_amd as da
    import workloads as W

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if not os.path.exists(da.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    dev = torch.device("cuda:0")

    def to_dev(x):
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(dev)

    if args.workload != "step":
        single_workload(args, torch, da, W, dev)
        return

    t_gen = time.perf_counter()
    p = W.longctx_v1()
    d = W.decode_v2() if args.only != "prefill" else None
    others = [W.prefill_v2(), W.prefill_v1()] if args.only is None else []
    log(f"inputs generated in {time.perf_counter() - t_gen:.1f} s")

    def prefill_inputs(w):
        if w.q_full is not None:
            qf = to_dev(w.q_full)
            q1, q2 = qf[:, 0::2], qf[:, 1::2]
        else:
            q1, q2 = to_dev(w.q1), to_dev(w.q2)
        k1 = to_dev(w.k1)
        k2 = k1 if w.shared_k else to_dev(w.k2)
        return dict(q1=q1, q2=q2, k1=k1, k2=k2, v=to_dev(w.v),
                    lamv=[torch.from_numpy(x).to(dev) for x in (w.lam_q1, w.lam_k1, w.lam_q2, w.lam_k2)],
                    gamma=torch.from_numpy(w.gamma).to(dev) if w.norm else None,
                    out=torch.empty((w.B, w.H, w.N, w.d_v), dtype=torch.bfloat16, device=dev),
                    lam=torch.empty(w.H, dtype=torch.float32, device=dev))

    def describe(w):
        form = "V2 GQA" if w.shared_k else "V1"
        return (f"{w.name} ({form}, B {w.B}, H {w.H}, H_kv {w.H_kv}, N {w.N}, d_qk {w.d_qk}, d_v {w.d_v}, causal, "
                f"{'RMS' if w.norm else 'no norm'})")

    P = prefill_inputs(p)
    # decode tensors
    if d is not None:
        qd = to_dev(d.q_full)
        kc, vc = to_dev(d.k1_cache), to_dev(d.v_cache)
        table = torch.from_numpy(d.page_table).to(dev)
        ctx = torch.from_numpy(d.ctx_len).to(dev)
        lamv_d = [torch.from_numpy(x).to(dev) for x in (d.lam_q1, d.lam_k1, d.lam_q2, d.lam_k2)]
        lam_d = torch.empty(d.H, dtype=torch.float32, device=dev)
        out_d = torch.empty((d.B, d.H, d.d_v), dtype=torch.bfloat16, device=dev)
        ws_bytes = da.decode_workspace_bytes(qd[:, 0::2], qd[:, 1::2], kc, vc, table, ctx, lam_d,
                                             depth=d.depth)
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()

    def prefill_call(w, T):
        da.lambda_(*T["lamv"], w.depth, out=T["lam"])
        return lambda: da.prefill(T["q1"], T["q2"], T["k1"], T["k2"], T["v"], T["lam"], depth=w.depth,
                                  causal=w.causal, norm=w.norm, gamma=T["gamma"], eps=w.eps, out=T["out"])

    def step(ev):
        if args.only != "decode":
            ev[0].record(stream)
            da.lambda_(*P["lamv"], p.depth, out=P["lam"])
            ev[1].record(stream)
            da.prefill(P["q1"], P["q2"], P["k1"], P["k2"], P["v"], P["lam"], depth=p.depth, causal=True,
                       norm=True, gamma=P["gamma"], eps=p.eps, out=P["out"])
            ev[2].record(stream)
        if d is not None:
            ev[3].record(stream)
            da.lambda_(*lamv_d, d.depth, out=lam_d)
            ev[4].record(stream)
            da.decode(qd[:, 0::2], qd[:, 1::2], kc, vc, table, ctx, lam_d, depth=d.depth, out=out_d,
                      workspace=ws)
            ev[5].record(stream)

    mk = lambda: [torch.cuda.Event(enable_timing=True) for _ in range(6)]
    for _ in range(args.warmup):
        step(mk())
    torch.cuda.synchronize()
    evs = [mk() for _ in range(args.steps)]
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    t_start.record(stream)
    for e in evs:
        step(e)
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    total_ms = t_start.elapsed_time(t_end)

    def mean_ms(a, b):
        return float(np.mean([e[a].elapsed_time(e[b]) for e in evs]))

    res = {}
    F = prefill_flops(p.B, p.H, p.N, p.d_qk, p.d_v)
    if args.only != "decode":
        pre_part = mean_ms(0, 2)
        pre_kernel = mean_ms(1, 2)
        res["prefill_part_ms"] = pre_part
        res["prefill_kernel_ms"] = pre_kernel
        log(f"prefill ({p.name}): step part {pre_part * 1e3:.1f} us, kernel {pre_kernel * 1e3:.1f} us, "
            f"{F / pre_kernel / 1e9:.1f} TFLOP/s")
    if d is not None:
        dbytes = decode_bytes(d)
        dec_part = mean_ms(3, 5)
        dec_call = mean_ms(4, 5)
        res["decode_part_ms"] = dec_part
        res["decode_call_ms"] = dec_call
        log(f"decode: step part {dec_part * 1e3:.1f} us, call {dec_call * 1e3:.1f} us, "
            f"{dbytes / dec_call / 1e6:.1f} GB/s")

    # the other prefill workloads: batches of back-to-back calls between two
    # events (a short kernel timed call by call would include the launch)
    other = {}
    for w in others:
        T = prefill_inputs(w)
        call = prefill_call(w, T)
        n_calls = max(10, min(100, int(args.steps * 4 * p.N / w.N)))
        for _ in range(max(3, args.warmup // 4)):
            call()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(n_calls):
            call()
        b.record(stream)
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / n_calls
        Fw = prefill_flops(w.B, w.H, w.N, w.d_qk, w.d_v)
        ach = Fw / (ms * 1e-3) / 1e12
        kern = f"prefill_bf16_kernel<{w.d_qk}, {'true' if w.shared_k else 'false'}, {'true' if w.norm else 'false'}, false, false>"
        other[w.name] = {"value": ach, "unit": "TFLOP/s", "ms_per_call": ms, "calls": n_calls,
                         "workload": describe(w),
                         "roofline": {"bound": "mfma", "kernel": kern, "achieved": ach, "peak": BF16_PEAK_TFLOPS,
                                      "unit": "TFLOP/s", "frac": ach / BF16_PEAK_TFLOPS,
                                      "traffic": load_traffic(w.name)}}
        log(f"{w.name}: {ms * 1e3:.1f} us per call, {ach:.1f} TFLOP/s ({100 * ach / BF16_PEAK_TFLOPS:.1f}% of peak)")
        del T
        torch.cuda.empty_cache()

    workload = describe(p)
    if d is not None:
        workload += (" + decode_v2 (V2 paged, 64 seqs, ctx U{8192..32768}, 8 KV / 64 Q heads, d 128, page 64)")
    line = {
        "metric": "prefill TFLOP/s (% bf16 MFMA peak) + decode GB/s (% HBM peak), 1 MI355X",
        "value": None, "unit": "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": total_ms / args.steps,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": workload, "global_batch": p.B, "seq_len": p.N, "parallelism": "none (1 GPU)"},
        "wall_s": wall,
    }
    if args.only != "decode":
        line["value"] = F / (res["prefill_part_ms"] * 1e-3) / 1e12
        ach = F / (res["prefill_kernel_ms"] * 1e-3) / 1e12
        line["roofline"] = {"bound": "mfma", "kernel": "prefill_bf16_kernel<64, false, true, false, false>",
                            "achieved": ach, "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                            "frac": ach / BF16_PEAK_TFLOPS, "traffic": load_traffic(p.name)}
    if d is not None:
        gbs = dbytes / (res["decode_part_ms"] * 1e-3) / 1e9
        ach = dbytes / (res["decode_call_ms"] * 1e-3) / 1e9
        line["decode"] = {"value": gbs, "unit": "GB/s", "tokens_per_s": d.B / (res["decode_part_ms"] * 1e-3),
                          "bytes_per_step": dbytes,
                          "roofline": {"bound": "hbm", "kernel": "decode_split_kernel + decode_combine_kernel",
                                       "achieved": ach, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                       "frac": ach / HBM_PEAK_GBS, "traffic": load_traffic("decode_v2")}}
    if other:
        line["prefill_other"] = other
    if not args.no_cpu and args.only != "decode":
        log("timing the CPU oracle ...")
        per = {p.name: cpu_baseline_prefill(p, args.cpu_budget)}
        for w in others:
            per[w.name] = cpu_baseline_prefill(w, args.cpu_budget / 3)
        if d is not None:
            per[d.name] = cpu_baseline_decode(d, args.cpu_budget / 3)
        line["cpu_baseline"] = dict(per[p.name], per_workload=per)
    print(json.dumps(line), flush=True)

if __name__ == "__main__":
    main()
