"""Python binding of libdiffattn (differential attention on MI355X / gfx950).

A thin ctypes layer over the C ABI declared in ``include/diffattn.h``: it
turns torch tensors into pointers, sizes and element strides, passes torch's
current HIP stream, and raises on a non-zero status. Every step of the
computation runs in the library's HIP kernels; torch only owns device memory
and the stream. There is no fallback: if ``libdiffattn.so`` is missing, or no
GPU is visible, the calls raise.

Functions (same names as the C entry points, without the prefix):
  lambda_init(depth)                             -> float (host)
  lambda_(lq1, lk1, lq2, lk2, depth)             -> [H] fp32 device tensor
  prefill(q1, q2, k1, k2, v, lam, ...)           -> [B, H, N, d_v]
  decode_workspace_bytes(...)                    -> int
  decode(q1, q2, k_cache, v_cache, page_table, ctx_len, lam, ...) -> [B, H, d_v]
                                                 (bf16 or fp8 e4m3 KV caches)
  decode_noalloc(...)                            -> the same, no workspace
  prefill_stats(q1, v)                           -> fp32 buffers for the backward
  backward_workspace_bytes(...)                  -> int
  backward(q1, q2, k1, k2, v, lam, stats, dout, ...) -> dict of gradients
  lambda_backward(lq1, lk1, lq2, lk2, dlambda)   -> dict of gradients
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libdiffattn.so")

OK, EINVAL, EUNSUPPORTED, EWORKSPACE, EHIP = 0, -1, -2, -3, -4
BF16, F32, FP8_E4M3 = 0, 1, 2
NORM_NONE, NORM_RMS, NORM_GROUP = 0, 1, 2


def _norm_code(norm) -> int:
    """norm: False/None (V2, no norm), True or "rms" (V1 RMSNorm), "group"
    (V1 GroupNorm per head, mean subtracted)."""
    if norm in (False, None, 0):
        return NORM_NONE
    if norm in (True, "rms", 1):
        return NORM_RMS
    if norm in ("group", 2):
        return NORM_GROUP
    raise ValueError(f"unknown norm {norm!r}")

_c_int64_3 = ctypes.c_int64 * 3
_c_int64_2 = ctypes.c_int64 * 2


class PrefillArgs(ctypes.Structure):
    _fields_ = [
        ("dtype", ctypes.c_int),
        ("B", ctypes.c_int), ("H", ctypes.c_int), ("H_kv", ctypes.c_int), ("N", ctypes.c_int),
        ("d_qk", ctypes.c_int), ("d_v", ctypes.c_int),
        ("q1", ctypes.c_void_p), ("q2", ctypes.c_void_p),
        ("k1", ctypes.c_void_p), ("k2", ctypes.c_void_p),
        ("v", ctypes.c_void_p),
        ("sq1", _c_int64_3), ("sq2", _c_int64_3), ("sk1", _c_int64_3), ("sk2", _c_int64_3),
        ("sv", _c_int64_3),
        ("lambda_", ctypes.c_void_p),
        ("depth", ctypes.c_int),
        ("causal", ctypes.c_int),
        ("scale", ctypes.c_float),
        ("norm", ctypes.c_int),
        ("gamma", ctypes.c_void_p),
        ("eps", ctypes.c_float),
        ("out", ctypes.c_void_p),
        ("so", _c_int64_3),
        ("window", ctypes.c_int),
        ("o1", ctypes.c_void_p), ("o2", ctypes.c_void_p),
        ("lse1", ctypes.c_void_p), ("lse2", ctypes.c_void_p),
    ]


class BackwardArgs(ctypes.Structure):
    _fields_ = [
        ("dtype", ctypes.c_int),
        ("B", ctypes.c_int), ("H", ctypes.c_int), ("H_kv", ctypes.c_int), ("N", ctypes.c_int),
        ("d_qk", ctypes.c_int), ("d_v", ctypes.c_int),
        ("q1", ctypes.c_void_p), ("q2", ctypes.c_void_p),
        ("k1", ctypes.c_void_p), ("k2", ctypes.c_void_p),
        ("v", ctypes.c_void_p),
        ("sq1", _c_int64_3), ("sq2", _c_int64_3), ("sk1", _c_int64_3), ("sk2", _c_int64_3),
        ("sv", _c_int64_3),
        ("lambda_", ctypes.c_void_p),
        ("depth", ctypes.c_int),
        ("causal", ctypes.c_int),
        ("window", ctypes.c_int),
        ("scale", ctypes.c_float),
        ("norm", ctypes.c_int),
        ("gamma", ctypes.c_void_p),
        ("eps", ctypes.c_float),
        ("o1", ctypes.c_void_p), ("o2", ctypes.c_void_p),
        ("lse1", ctypes.c_void_p), ("lse2", ctypes.c_void_p),
        ("dout", ctypes.c_void_p),
        ("sdo", _c_int64_3),
        ("dq1", ctypes.c_void_p), ("dq2", ctypes.c_void_p),
        ("dk1", ctypes.c_void_p), ("dk2", ctypes.c_void_p),
        ("dv", ctypes.c_void_p),
        ("dlambda", ctypes.c_void_p),
        ("dgamma", ctypes.c_void_p),
    ]


class DecodeArgs(ctypes.Structure):
    _fields_ = [
        ("dtype", ctypes.c_int),
        ("B", ctypes.c_int), ("H", ctypes.c_int), ("H_kv", ctypes.c_int),
        ("d_qk", ctypes.c_int), ("d_v", ctypes.c_int), ("page_size", ctypes.c_int),
        ("max_pages", ctypes.c_int), ("num_pages", ctypes.c_int),
        ("q1", ctypes.c_void_p), ("q2", ctypes.c_void_p),
        ("sq1", _c_int64_2), ("sq2", _c_int64_2),
        ("k1_cache", ctypes.c_void_p), ("k2_cache", ctypes.c_void_p), ("v_cache", ctypes.c_void_p),
        ("page_table", ctypes.c_void_p),
        ("ctx_len", ctypes.c_void_p),
        ("lambda_", ctypes.c_void_p),
        ("depth", ctypes.c_int),
        ("scale", ctypes.c_float),
        ("norm", ctypes.c_int),
        ("gamma", ctypes.c_void_p),
        ("eps", ctypes.c_float),
        ("out", ctypes.c_void_p),
        ("so", _c_int64_2),
        ("split_pages", ctypes.c_int),
        ("dev_err", ctypes.c_void_p),
        ("window", ctypes.c_int),
        ("kv_dtype", ctypes.c_int),
        ("k_scale", ctypes.c_float), ("v_scale", ctypes.c_float),
    ]


class DiffAttnError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"libdiffattn error {code}: {msg}")
        self.code = code


_lib = None


def load_library(path: Optional[str] = None):
    """Load libdiffattn.so (raises if it has not been built)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"{p} is missing: build it with `python -m differential_attention_amd.build`")
    lib = ctypes.CDLL(p)
    V, I, F = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    lib.diffattn_lambda_init.argtypes = [I]
    lib.diffattn_lambda_init.restype = ctypes.c_double
    lib.diffattn_lambda.argtypes = [V, V, V, V, I, I, I, V, V]
    lib.diffattn_lambda.restype = I
    lib.diffattn_prefill.argtypes = [ctypes.POINTER(PrefillArgs), V]
    lib.diffattn_prefill.restype = I
    lib.diffattn_decode_workspace_bytes.argtypes = [ctypes.POINTER(DecodeArgs)]
    lib.diffattn_decode_workspace_bytes.restype = ctypes.c_size_t
    lib.diffattn_decode.argtypes = [ctypes.POINTER(DecodeArgs), V, ctypes.c_size_t, V]
    lib.diffattn_decode.restype = I
    lib.diffattn_decode_noalloc.argtypes = [ctypes.POINTER(DecodeArgs), V]
    lib.diffattn_decode_noalloc.restype = I
    lib.diffattn_backward_workspace_bytes.argtypes = [ctypes.POINTER(BackwardArgs)]
    lib.diffattn_backward_workspace_bytes.restype = ctypes.c_size_t
    lib.diffattn_backward.argtypes = [ctypes.POINTER(BackwardArgs), V, ctypes.c_size_t, V]
    lib.diffattn_backward.restype = I
    lib.diffattn_lambda_backward.argtypes = [V, V, V, V, I, I, V, V, V, V, V, V]
    lib.diffattn_lambda_backward.restype = I
    lib.diffattn_last_error.argtypes = []
    lib.diffattn_last_error.restype = ctypes.c_char_p
    if path is None:
        _lib = lib
    return lib


def _check(rc: int):
    if rc != OK:
        msg = load_library().diffattn_last_error().decode()
        raise DiffAttnError(rc, msg)


def _stream(stream=None) -> int:
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return int(s.cuda_stream)


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise TypeError(f"unsupported dtype {t.dtype} (bf16 or fp32)")


def _kv_dtype_code(*caches) -> int:
    """Storage of the KV caches: all bf16, or all fp8 e4m3 (torch.float8_e4m3fn,
    or uint8 tensors holding the codes)."""
    import torch
    kinds = {c.dtype for c in caches if c is not None}
    if kinds == {torch.bfloat16}:
        return BF16
    if kinds <= {torch.float8_e4m3fn, torch.uint8}:
        return FP8_E4M3
    raise TypeError(f"KV caches must all be bf16 or all fp8 e4m3, got {sorted(map(str, kinds))}")


def _ptr(t) -> Optional[int]:
    return None if t is None else int(t.data_ptr())


def _need(t, name: str, dtype=None, shape=None, contiguous: bool = False):
    """Check one tensor argument before its pointer reaches the library: the
    kernels read exactly the sizes the ABI is given, so a wrong dtype (an
    int64 table read as int32 pairs) or shape would be read silently wrong or
    out of bounds. Checks dtype, then shape, then layout (the device is
    checked for all arguments together by _on_device)."""
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _on_device(**tensors):
    """Every tensor argument (None allowed) must live in device memory."""
    for name, t in tensors.items():
        if t is not None and not t.is_cuda:
            raise ValueError(f"{name} must be a device tensor")


def lambda_init(depth: int) -> float:
    """lambda_init(depth) = 0.8 - 0.6 exp(-0.3 (depth - 1)) (host, fp64)."""
    return float(load_library().diffattn_lambda_init(int(depth)))


def lambda_(lq1, lk1, lq2, lk2, depth: int, out=None, stream=None):
    """Per-head lambda [H] (fp32, device) from four [H, d_lambda] fp32 device tensors."""
    import torch
    vecs = [x.contiguous() for x in (lq1, lk1, lq2, lk2)]
    H, dl = vecs[0].shape
    for x in vecs:
        if x.shape != (H, dl) or x.dtype != torch.float32 or not x.is_cuda:
            raise ValueError("lambda vectors must be [H, d_lambda] fp32 device tensors of one shape")
    if out is None:
        out = torch.empty(H, dtype=torch.float32, device=vecs[0].device)
    _need(out, "out", torch.float32, (H,), contiguous=True)
    rc = load_library().diffattn_lambda(*(_ptr(x) for x in vecs), H, dl, int(depth), _ptr(out),
                                        _stream(stream))
    _check(rc)
    return out


def _strides3(t):
    s = t.stride()
    if t.dim() != 4 or s[3] != 1:
        raise ValueError("expected a 4-d tensor with unit innermost stride")
    return (s[0], s[1], s[2])


def prefill(q1, q2, k1, k2, v, lam, *, depth: int, causal: bool = True, norm: bool = False,
            gamma=None, eps: float = 1e-5, scale: float = 0.0, out=None, stream=None, window: int = 0,
            stats=None):
    """Differential-attention prefill.

    q1, q2 [B, H, N, d_qk]; k1, k2 [B, H_kv, N, d_qk] (pass the same tensor
    for both in the V2 form); v [B, H_kv, N, d_v]; lam [H] fp32 device;
    gamma [H, d_v] fp32 device when norm (V1). Views with unit innermost
    stride are accepted as they are. window > 0 (causal only) limits row i to
    keys i-window+1 .. i. stats: None, or a tuple (o1, o2, lse1, lse2) of fp32
    tensors [B, H, N, d_v] x 2 and [B, H, N] x 2 that receive the statistics
    the backward pass needs (see prefill_stats). Returns out [B, H, N, d_v]."""
    import torch
    B, H, N, dqk = q1.shape
    Hkv, dv = k1.shape[1], v.shape[3]
    a = PrefillArgs()
    a.dtype = _dtype_code(q1)
    _need(q1, "q1")
    _need(q2, "q2", q1.dtype, q1.shape)
    _need(k1, "k1", q1.dtype, (B, Hkv, N, dqk))
    _need(k2, "k2", q1.dtype, (B, Hkv, N, dqk))
    _need(v, "v", q1.dtype, (B, Hkv, N, dv))
    _need(lam, "lam", torch.float32, (H,), contiguous=True)
    if norm:
        if gamma is None:
            raise ValueError("gamma [H, d_v] is required with a norm")
        _need(gamma, "gamma", torch.float32, (H, dv), contiguous=True)
    if out is not None:
        _need(out, "out", q1.dtype, (B, H, N, dv))
    _on_device(q1=q1, q2=q2, k1=k1, k2=k2, v=v, lam=lam, gamma=gamma if norm else None, out=out)
    if out is None:
        out = torch.empty((B, H, N, dv), dtype=q1.dtype, device=q1.device)
    a.B, a.H, a.H_kv, a.N, a.d_qk, a.d_v = B, H, Hkv, N, dqk, dv
    a.q1, a.q2, a.k1, a.k2, a.v = _ptr(q1), _ptr(q2), _ptr(k1), _ptr(k2), _ptr(v)
    a.sq1, a.sq2 = _c_int64_3(*_strides3(q1)), _c_int64_3(*_strides3(q2))
    a.sk1, a.sk2 = _c_int64_3(*_strides3(k1)), _c_int64_3(*_strides3(k2))
    a.sv, a.so = _c_int64_3(*_strides3(v)), _c_int64_3(*_strides3(out))
    a.lambda_ = _ptr(lam)
    a.depth = int(depth)
    a.causal = int(bool(causal))
    a.window = int(window)
    if stats is not None:
        for t, shape, nm in zip(stats, ((B, H, N, dv), (B, H, N, dv), (B, H, N), (B, H, N)),
                                ("o1", "o2", "lse1", "lse2")):
            _need(t, "stats " + nm, torch.float32, shape, contiguous=True)
        _on_device(o1=stats[0], o2=stats[1], lse1=stats[2], lse2=stats[3])
        a.o1, a.o2, a.lse1, a.lse2 = (_ptr(t) for t in stats)
    a.scale = float(scale)
    a.norm = _norm_code(norm)
    a.gamma = _ptr(gamma) if norm else None
    a.eps = float(eps)
    a.out = _ptr(out)
    _check(load_library().diffattn_prefill(ctypes.byref(a), _stream(stream)))
    return out


def prefill_stats(q1, v):
    """Fresh (o1, o2, lse1, lse2) tensors for prefill(..., stats=...)."""
    import torch
    B, H, N, _ = q1.shape
    dv = v.shape[3]
    f = lambda *s: torch.empty(s, dtype=torch.float32, device=q1.device)
    return f(B, H, N, dv), f(B, H, N, dv), f(B, H, N), f(B, H, N)


def _backward_args(q1, q2, k1, k2, v, lam, stats, dout, g, depth, causal, norm, gamma, eps, scale, window):
    import torch
    B, H, N, dqk = q1.shape
    Hkv, dv_ = k1.shape[1], v.shape[3]
    shared = k1.data_ptr() == k2.data_ptr() and k1.stride() == k2.stride()
    a = BackwardArgs()
    a.dtype = _dtype_code(q1)
    a.B, a.H, a.H_kv, a.N, a.d_qk, a.d_v = B, H, Hkv, N, dqk, dv_
    _need(q1, "q1")
    _need(q2, "q2", q1.dtype, q1.shape)
    _need(k1, "k1", q1.dtype, (B, Hkv, N, dqk))
    _need(k2, "k2", q1.dtype, (B, Hkv, N, dqk))
    _need(v, "v", q1.dtype, (B, Hkv, N, dv_))
    _need(dout, "dout", q1.dtype, (B, H, N, dv_))
    _need(lam, "lam", torch.float32, (H,), contiguous=True)
    if norm:
        if gamma is None:
            raise ValueError("gamma [H, d_v] is required with a norm")
        _need(gamma, "gamma", torch.float32, (H, dv_), contiguous=True)
    for t, shape, nm in zip(stats, ((B, H, N, dv_), (B, H, N, dv_), (B, H, N), (B, H, N)),
                            ("o1", "o2", "lse1", "lse2")):
        _need(t, "stats " + nm, torch.float32, shape, contiguous=True)
    _on_device(q1=q1, q2=q2, k1=k1, k2=k2, v=v, dout=dout, lam=lam, gamma=gamma if norm else None,
               o1=stats[0], o2=stats[1], lse1=stats[2], lse2=stats[3])
    a.q1, a.q2, a.k1, a.k2, a.v = (_ptr(t) for t in (q1, q2, k1, k2, v))
    a.sq1, a.sq2 = _c_int64_3(*_strides3(q1)), _c_int64_3(*_strides3(q2))
    a.sk1, a.sk2 = _c_int64_3(*_strides3(k1)), _c_int64_3(*_strides3(k2))
    a.sv = _c_int64_3(*_strides3(v))
    a.lambda_ = _ptr(lam)
    a.depth, a.causal, a.window, a.scale = int(depth), int(bool(causal)), int(window), float(scale)
    a.norm = _norm_code(norm)
    a.gamma = _ptr(gamma) if norm else None
    a.eps = float(eps)
    a.o1, a.o2, a.lse1, a.lse2 = (_ptr(t) for t in stats)
    a.dout = _ptr(dout)
    a.sdo = _c_int64_3(*_strides3(dout))
    if g is not None:
        a.dq1, a.dq2, a.dk1, a.dv, a.dlambda = (_ptr(g[k]) for k in ("dq1", "dq2", "dk1", "dv", "dlambda"))
        a.dk2 = None if shared else _ptr(g["dk2"])
        a.dgamma = _ptr(g["dgamma"]) if norm else None
    return a


def backward_workspace_bytes(q1, q2, k1, k2, v, lam, stats, dout, *, depth: int, causal: bool = True,
                             norm: bool = False, gamma=None, eps: float = 1e-5, scale: float = 0.0,
                             window: int = 0) -> int:
    """Bytes of device workspace backward(...) needs for these arguments."""
    a = _backward_args(q1, q2, k1, k2, v, lam, stats, dout, None, depth, causal, norm, gamma, eps, scale, window)
    return int(load_library().diffattn_backward_workspace_bytes(ctypes.byref(a)))


def backward(q1, q2, k1, k2, v, lam, stats, dout, *, depth: int, causal: bool = True, norm: bool = False,
             gamma=None, eps: float = 1e-5, scale: float = 0.0, window: int = 0, workspace=None, stream=None):
    """Gradients of prefill(q1, q2, k1, k2, v, lam, ...) given dout (bf16
    [B, H, N, d_v]) and the statistics (o1, o2, lse1, lse2) a prefill call with
    stats=... stored. Returns a dict of fp32 tensors dq1, dq2, dk1, dk2, dv,
    dlambda and (norm) dgamma; with k1 is k2 (one key tensor) dk1 is the whole
    key gradient and dk2 is the same tensor. workspace: None, or a device
    tensor of at least backward_workspace_bytes(...) bytes, 256-byte aligned."""
    import torch
    B, H, N, dqk = q1.shape
    Hkv, dv_ = k1.shape[1], v.shape[3]
    shared = k1.data_ptr() == k2.data_ptr() and k1.stride() == k2.stride()
    f = lambda *sh: torch.empty(sh, dtype=torch.float32, device=q1.device)
    g = {"dq1": f(B, H, N, dqk), "dq2": f(B, H, N, dqk), "dk1": f(B, Hkv, N, dqk), "dv": f(B, Hkv, N, dv_),
         "dlambda": f(H)}
    g["dk2"] = g["dk1"] if shared else f(B, Hkv, N, dqk)
    g["dgamma"] = f(H, dv_) if norm else None
    a = _backward_args(q1, q2, k1, k2, v, lam, stats, dout, g, depth, causal, norm, gamma, eps, scale, window)
    lib = load_library()
    need = int(lib.diffattn_backward_workspace_bytes(ctypes.byref(a)))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q1.device)
    _check(lib.diffattn_backward(ctypes.byref(a), _ptr(workspace), workspace.numel(), _stream(stream)))
    return g


def lambda_backward(lq1, lk1, lq2, lk2, dlambda, stream=None):
    """Gradients of the four [H, d_lambda] lambda vectors given dlambda [H]."""
    import torch
    H, dl = lq1.shape
    for t, nm in zip((lq1, lk1, lq2, lk2), ("lq1", "lk1", "lq2", "lk2")):
        _need(t, nm, torch.float32, (H, dl), contiguous=True)
    _need(dlambda, "dlambda", torch.float32, (H,), contiguous=True)
    _on_device(lq1=lq1, lk1=lk1, lq2=lq2, lk2=lk2, dlambda=dlambda)
    outs = [torch.empty_like(lq1) for _ in range(4)]
    _check(load_library().diffattn_lambda_backward(_ptr(lq1), _ptr(lk1), _ptr(lq2), _ptr(lk2), H, dl,
                                                   _ptr(dlambda), *(_ptr(t) for t in outs), _stream(stream)))
    return dict(zip(("dlq1", "dlk1", "dlq2", "dlk2"), outs))


def _decode_args(q1, q2, k_cache, v_cache, page_table, ctx_len, lam, depth, norm, gamma, eps,
                 scale, out, split_pages, dev_err, k2_cache=None, window=0, k_scale=1.0,
                 v_scale=1.0) -> DecodeArgs:
    import torch
    B, H, dqk = q1.shape
    P, Hkv, page, _ = k_cache.shape
    dv = v_cache.shape[3]
    _need(q1, "q1")
    _need(q2, "q2", q1.dtype, q1.shape)
    if k_cache.dtype not in (torch.bfloat16, torch.float8_e4m3fn, torch.uint8):
        raise TypeError(f"k_cache must be bf16 or fp8 e4m3 (float8_e4m3fn or uint8 codes), got {k_cache.dtype}")
    _need(k_cache, "k_cache", shape=(P, Hkv, page, dqk), contiguous=True)
    if k2_cache is not None:
        _need(k2_cache, "k2_cache", k_cache.dtype, (P, Hkv, page, dqk), contiguous=True)
    _need(v_cache, "v_cache", shape=(P, Hkv, page, dv), contiguous=True)
    if page_table.dim() != 2 or page_table.shape[0] != B:
        raise ValueError(f"page_table must have shape [B={B}, max_pages], got {tuple(page_table.shape)}")
    _need(page_table, "page_table", torch.int32, contiguous=True)
    _need(ctx_len, "ctx_len", torch.int32, (B,), contiguous=True)
    _need(lam, "lam", torch.float32, (H,), contiguous=True)
    if norm:
        if gamma is None:
            raise ValueError("gamma [H, d_v] is required with a norm")
        _need(gamma, "gamma", torch.float32, (H, dv), contiguous=True)
    if out is not None:
        _need(out, "out", q1.dtype, (B, H, dv))
    if dev_err is not None:
        _need(dev_err, "dev_err", torch.int32)
    _on_device(q1=q1, q2=q2, k_cache=k_cache, k2_cache=k2_cache, v_cache=v_cache, page_table=page_table,
               ctx_len=ctx_len, lam=lam, gamma=gamma if norm else None, out=out, dev_err=dev_err)
    a = DecodeArgs()
    a.dtype = _dtype_code(q1)
    a.B, a.H, a.H_kv, a.d_qk, a.d_v = B, H, Hkv, dqk, dv
    a.page_size, a.max_pages, a.num_pages = page, page_table.shape[1], P
    a.q1, a.q2 = _ptr(q1), _ptr(q2)
    if q1.stride(2) != 1 or q2.stride(2) != 1:
        raise ValueError("q1/q2 need unit innermost stride")
    a.sq1 = _c_int64_2(q1.stride(0), q1.stride(1))
    a.sq2 = _c_int64_2(q2.stride(0), q2.stride(1))
    a.k1_cache = _ptr(k_cache)
    a.k2_cache = _ptr(k2_cache if k2_cache is not None else k_cache)
    a.v_cache = _ptr(v_cache)
    a.page_table = _ptr(page_table)
    a.ctx_len = _ptr(ctx_len)
    a.lambda_ = _ptr(lam)
    a.depth = int(depth)
    a.scale = float(scale)
    a.norm = _norm_code(norm)
    a.gamma = _ptr(gamma) if norm else None
    a.eps = float(eps)
    a.out = _ptr(out) if out is not None else None
    a.so = _c_int64_2(out.stride(0), out.stride(1)) if out is not None else _c_int64_2(H * dv, dv)
    a.split_pages = int(split_pages)
    a.dev_err = _ptr(dev_err)
    a.window = int(window)
    a.kv_dtype = _kv_dtype_code(k_cache, k2_cache, v_cache)
    a.k_scale, a.v_scale = float(k_scale), float(v_scale)
    return a


def decode_workspace_bytes(q1, q2, k_cache, v_cache, page_table, ctx_len, lam, *, depth: int,
                           norm: bool = False, gamma=None, eps: float = 1e-5, scale: float = 0.0,
                           split_pages: int = 0, k2_cache=None, window: int = 0, k_scale: float = 1.0,
                           v_scale: float = 1.0) -> int:
    a = _decode_args(q1, q2, k_cache, v_cache, page_table, ctx_len, lam, depth, norm, gamma, eps,
                     scale, None, split_pages, None, k2_cache, window, k_scale, v_scale)
    return int(load_library().diffattn_decode_workspace_bytes(ctypes.byref(a)))


def decode(q1, q2, k_cache, v_cache, page_table, ctx_len, lam, *, depth: int, norm: bool = False,
           gamma=None, eps: float = 1e-5, scale: float = 0.0, out=None, workspace=None,
           split_pages: int = 0, dev_err=None, stream=None, k2_cache=None, window: int = 0,
           k_scale: float = 1.0, v_scale: float = 1.0):
    """Paged decode (one query token per sequence).

    q1, q2 [B, H, d_qk]; k_cache [num_pages, H_kv, page, d_qk] and v_cache
    [num_pages, H_kv, page, d_v] contiguous; k_cache serves both branches
    unless k2_cache (the branch-2 keys, V1 form with d_qk 64) is given;
    page_table [B, max_pages] int32; ctx_len [B] int32; lam [H] fp32;
    window > 0: the query sees its last window tokens. The caches are bf16, or
    fp8 e4m3 (float8_e4m3fn or uint8 codes) read as k_scale * code and
    v_scale * code. Returns out [B, H, d_v]."""
    import torch
    B, H, _ = q1.shape
    dv = v_cache.shape[3]
    if out is None:
        out = torch.empty((B, H, dv), dtype=q1.dtype, device=q1.device)
    a = _decode_args(q1, q2, k_cache, v_cache, page_table, ctx_len, lam, depth, norm, gamma, eps,
                     scale, out, split_pages, dev_err, k2_cache, window, k_scale, v_scale)
    lib = load_library()
    need = int(lib.diffattn_decode_workspace_bytes(ctypes.byref(a)))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q1.device)
    _check(lib.diffattn_decode(ctypes.byref(a), _ptr(workspace), workspace.numel(), _stream(stream)))
    return out


def decode_noalloc(q1, q2, k_cache, v_cache, page_table, ctx_len, lam, *, depth: int, norm: bool = False,
                   gamma=None, eps: float = 1e-5, scale: float = 0.0, out=None, split_pages: int = 0,
                   dev_err=None, stream=None, k2_cache=None, window: int = 0, k_scale: float = 1.0,
                   v_scale: float = 1.0):
    """decode(...) without a workspace: the library's static device scratch
    holds the partial results (diffattn_decode_noalloc). With out given, no
    device memory is allocated by this call."""
    import torch
    B, H, _ = q1.shape
    dv = v_cache.shape[3]
    if out is None:
        out = torch.empty((B, H, dv), dtype=q1.dtype, device=q1.device)
    a = _decode_args(q1, q2, k_cache, v_cache, page_table, ctx_len, lam, depth, norm, gamma, eps,
                     scale, out, split_pages, dev_err, k2_cache, window, k_scale, v_scale)
    _check(load_library().diffattn_decode_noalloc(ctypes.byref(a), _stream(stream)))
    return out
