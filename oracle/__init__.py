"""CPU oracle for differential attention (fp64). TEST INFRASTRUCTURE ONLY.

Only ``tests/``, the smoke check and the benchmark's CPU-baseline leg import
this package. It shares no code with the HIP path (``differential_attention_amd``)
and never imports it; the product never imports this.

``oracle.c`` holds the arithmetic (plain C, fp64, OpenMP over rows); this
module builds it with gcc and marshals numpy arrays. ``brute.py`` is a second,
stdlib-only Python implementation for tiny shapes that pins the C oracle.

Parity status of each function (pins live in ``tests/test_oracle.py``):
  lambda_init  pinned (closed form at depth 1, limit, monotonicity)
  lambda_      pinned (exact exponent values, zero vectors, sign)
  prefill      pinned (brute force, lambda=0 vs torch SDPA, row sums, zero
               output, swap symmetry, causal row 0, norm closed form, the
               printed causal-mask figure, the signal-plus-noise toy)
  decode       pinned (equals the last row of causal prefill; page-table
               permutation invariance; brute force)
  backward.prefill_backward, backward.lambda_backward (the gradients, fp64
               numpy): pinned by central finite differences of the brute-force
               forward and by invariants (tests/test_oracle_backward.py)
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
# ORACLE_LIB: load another build of oracle.c instead (the sanitizer test runs
# the pins against an AddressSanitizer / UBSan build this way)
_LIB_OVERRIDE = os.environ.get("ORACLE_LIB")
_lib = None


def build(force: bool = True) -> str:
    """Compile liboracle.so with gcc (-O3 with IEEE semantics: no fast-math,
    no contraction into fused multiply-adds; OpenMP)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O3", "-fno-fast-math", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared",
                               "-std=c11", "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if _LIB_OVERRIDE:
        lib = ctypes.CDLL(_LIB_OVERRIDE)
    else:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()  # missing, or older than its source (its signatures may have changed)
        lib = ctypes.CDLL(_LIB)
    P = ctypes.c_void_p
    i, d, i64 = ctypes.c_int, ctypes.c_double, ctypes.c_int64
    lib.oracle_lambda_init.argtypes = [i]
    lib.oracle_lambda_init.restype = d
    lib.oracle_lambda.argtypes = [P, P, P, P, i, i, i, P]
    lib.oracle_lambda.restype = None
    lib.oracle_prefill.argtypes = [P, P, P, P, P, i, i, i, i, i, i, P, i, i, i, d, i, P, d, P, i64, P]
    lib.oracle_prefill.restype = i
    lib.oracle_decode.argtypes = [P, P, P, P, P, i, i, i, i, i, i, i, i, P, P, P, i, i, d, i, P, d, P]
    lib.oracle_decode.restype = i
    lib.oracle_num_threads.argtypes = []
    lib.oracle_num_threads.restype = i
    _lib = lib
    return lib


def _f32(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float32)


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _norm_code(norm) -> int:
    """norm: False/None (V2), True or "rms" (V1 RMSNorm), "group" (GroupNorm per head)."""
    if norm in (False, None, 0):
        return 0
    if norm in (True, "rms", 1):
        return 1
    if norm in ("group", 2):
        return 2
    raise ValueError(f"unknown norm {norm!r}")


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def lambda_init(depth: int) -> float:
    """lambda_init(depth) = 0.8 - 0.6 exp(-0.3 (depth - 1))."""
    return float(_load().oracle_lambda_init(int(depth)))


def lambda_(lq1, lk1, lq2, lk2, depth: int) -> np.ndarray:
    """Per-head lambda [H] (fp64) from the four [H, d_l] vectors."""
    lq1, lk1, lq2, lk2 = (_f32(x) for x in (lq1, lk1, lq2, lk2))
    H, dl = lq1.shape
    out = np.empty(H, np.float64)
    _load().oracle_lambda(_ptr(lq1), _ptr(lk1), _ptr(lq2), _ptr(lk2), H, dl, int(depth), _ptr(out))
    return out


def prefill(q1, q2, k1, k2, v, lam, *, depth: int, causal: bool, norm: bool,
            gamma=None, eps: float = 1e-5, scale: Optional[float] = None,
            rows: Optional[np.ndarray] = None, window: int = 0) -> np.ndarray:
    """Differential attention over a full sequence.

    q1, q2 [B, H, N, d_qk]; k1, k2 [B, H_kv, N, d_qk]; v [B, H_kv, N, d_v];
    lam [H]; window: 0, or a causal sliding window W (keys i-W+1..i).
    Returns [B, H, N, d_v] fp64, or [len(rows), d_v] when ``rows``
    (flat ids (b*H + h)*N + i) is given."""
    q1, q2, k1, k2, v = (_f32(x) for x in (q1, q2, k1, k2, v))
    B, H, N, dqk = q1.shape
    Hkv = k1.shape[1]
    dv = v.shape[3]
    assert q2.shape == q1.shape and k1.shape == (B, Hkv, N, dqk) and k2.shape == k1.shape
    assert v.shape == (B, Hkv, N, dv)
    lam = np.ascontiguousarray(lam, dtype=np.float64).reshape(H)
    g = _f32(gamma).reshape(H, dv) if _norm_code(norm) else None
    if scale is None:
        scale = 1.0 / np.sqrt(dqk)
    if rows is None:
        out = np.empty((B, H, N, dv), np.float64)
        nrows = B * H * N
        rp = None
    else:
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        nrows = rows.size
        out = np.empty((nrows, dv), np.float64)
        rp = _ptr(rows)
    rc = _load().oracle_prefill(_ptr(q1), _ptr(q2), _ptr(k1), _ptr(k2), _ptr(v), B, H, Hkv, N, dqk, dv,
                                _ptr(lam), int(depth), int(bool(causal)), int(window), float(scale),
                                _norm_code(norm),
                                _ptr(g), float(eps), rp, nrows, _ptr(out))
    if rc != 0:
        raise ValueError("oracle_prefill: invalid argument")
    return out


def decode(q1, q2, k1_cache, k2_cache, v_cache, page_table, ctx_len, lam, *, depth: int,
           norm: bool, gamma=None, eps: float = 1e-5, scale: Optional[float] = None,
           window: int = 0) -> np.ndarray:
    """Paged decode: q1, q2 [B, H, d_qk]; caches [P, H_kv, page, d]; page_table
    [B, max_pages] int32; ctx_len [B] int32; lam [H]; window 0 or W (the
    query sees its last W tokens). Returns [B, H, d_v] fp64."""
    q1, q2, kc1, kc2, vc = (_f32(x) for x in (q1, q2, k1_cache, k2_cache, v_cache))
    B, H, dqk = q1.shape
    P, Hkv, page, _ = kc1.shape
    dv = vc.shape[3]
    table = np.ascontiguousarray(page_table, dtype=np.int32)
    ctx = np.ascontiguousarray(ctx_len, dtype=np.int32)
    max_pages = table.shape[1]
    lam = np.ascontiguousarray(lam, dtype=np.float64).reshape(H)
    g = _f32(gamma).reshape(H, dv) if _norm_code(norm) else None
    if scale is None:
        scale = 1.0 / np.sqrt(dqk)
    out = np.empty((B, H, dv), np.float64)
    rc = _load().oracle_decode(_ptr(q1), _ptr(q2), _ptr(kc1), _ptr(kc2), _ptr(vc), B, H, Hkv, dqk, dv,
                               page, max_pages, P, _ptr(table), _ptr(ctx), _ptr(lam), int(depth),
                               int(window), float(scale), _norm_code(norm), _ptr(g), float(eps), _ptr(out))
    if rc != 0:
        raise ValueError("oracle_decode: invalid argument or page id")
    return out
