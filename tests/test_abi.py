"""The C ABI on the CPU: the library loads, exports every function declared in
include/diffattn.h, and rejects bad arguments on the host before any launch.
No call here reaches a kernel (this container has no GPU)."""
import ctypes
import math
import os
import re
import subprocess

import pytest

import differential_attention_amd as da
import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(da.LIB_PATH):
        from differential_attention_amd import build
        build.build()
    return da.load_library()


def _declared_functions():
    names = set()
    inc = os.path.join(ROOT, "include")
    for fn in os.listdir(inc):
        if fn.endswith(".h"):
            text = open(os.path.join(inc, fn)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names.update(re.findall(r"\b(diffattn_[a-z0-9_]+)\s*\(", text))
    return sorted(names)


def test_exports_every_declared_symbol(lib):
    names = _declared_functions()
    assert {"diffattn_prefill", "diffattn_decode", "diffattn_lambda"} <= set(names)
    for n in names:
        assert hasattr(lib, n), f"{n} declared in include/ but not exported"


def test_struct_layout_matches_header(tmp_path):
    """ctypes mirrors of the argument structs have the C compiler's layout."""
    src = ["#include <stdio.h>", "#include <stddef.h>", '#include "diffattn.h"', "int main(void) {"]
    structs = (("diffattn_prefill_args", da.PrefillArgs), ("diffattn_decode_args", da.DecodeArgs),
               ("diffattn_backward_args", da.BackwardArgs))
    for cname, py in structs:
        src.append(f'printf("{cname} size %zu\\n", sizeof({cname}));')
        for fname, _ in py._fields_:
            cf = "lambda" if fname == "lambda_" else fname
            src.append(f'printf("{cname} {fname} %zu\\n", offsetof({cname}, {cf}));')
    src.append("return 0; }")
    c = tmp_path / "layout.c"
    c.write_text("\n".join(src))
    exe = tmp_path / "layout"
    subprocess.check_call(["gcc", "-std=c11", "-I", os.path.join(ROOT, "include"), str(c), "-o", str(exe)])
    out = subprocess.check_output([str(exe)], text=True).split("\n")
    pys = dict(structs)
    for line in filter(None, out):
        cname, field, value = line.split()
        py = pys[cname]
        got = ctypes.sizeof(py) if field == "size" else getattr(py, field).offset
        assert got == int(value), (cname, field)


def test_lambda_init_matches_oracle(lib):
    for d in (1, 2, 12, 20, 100):
        assert abs(da.lambda_init(d) - oracle.lambda_init(d)) <= 1e-15
    assert math.isnan(da.lambda_init(0))


FAKE = 0x7F0000000000  # a 256-aligned fake device address; never dereferenced


def _prefill_args(**kw):
    a = da.PrefillArgs()
    a.dtype = da.BF16
    a.B, a.H, a.H_kv, a.N, a.d_qk, a.d_v = 1, 4, 2, 128, 64, 128
    step = 1 << 24
    a.q1, a.q2, a.k1, a.k2, a.v = FAKE, FAKE + step, FAKE + 2 * step, FAKE + 3 * step, FAKE + 4 * step
    for f, d in (("sq1", 64), ("sq2", 64), ("sk1", 64), ("sk2", 64), ("sv", 128)):
        h = 4 if f.startswith("sq") else 2
        setattr(a, f, (ctypes.c_int64 * 3)(h * 128 * d, 128 * d, d))
    a.lambda_ = FAKE + 5 * step
    a.depth, a.causal, a.scale, a.norm = 1, 1, 0.0, da.NORM_RMS
    a.gamma = FAKE + 6 * step
    a.eps = 1e-5
    a.out = FAKE + 7 * step
    a.so = (ctypes.c_int64 * 3)(4 * 128 * 128, 128 * 128, 128)
    for k, v in kw.items():
        setattr(a, k, v)
    return a


def _rc(lib, a):
    return lib.diffattn_prefill(ctypes.byref(a), None)


@pytest.mark.parametrize("field,value,code", [
    ("H", 3, da.EINVAL),                 # H % H_kv != 0
    ("H_kv", 0, da.EINVAL),
    ("N", -1, da.EINVAL),
    ("depth", 0, da.EINVAL),
    ("causal", 2, da.EINVAL),
    ("norm", 7, da.EINVAL),
    ("dtype", 9, da.EINVAL),
    ("eps", 0.0, da.EINVAL),
    ("scale", -1.0, da.EINVAL),
    ("d_qk", 96, da.EUNSUPPORTED),       # no bf16 kernel for (96, 128)
    ("q1", None, da.EINVAL),
    ("gamma", None, da.EINVAL),          # RMS without gamma
    ("k1", FAKE + 2 * (1 << 24) + 2, da.EINVAL),   # misaligned bf16 pointer
    ("window", -1, da.EINVAL),
])
def test_prefill_rejects(lib, field, value, code):
    a = _prefill_args(**{field: value})
    assert _rc(lib, a) == code
    assert lib.diffattn_last_error().decode().startswith("diffattn_prefill")


def test_prefill_window_needs_causal(lib):
    a = _prefill_args(causal=0, window=16)
    assert _rc(lib, a) == da.EINVAL
    assert "window" in lib.diffattn_last_error().decode()


def test_prefill_rejects_bad_strides_and_alias(lib):
    a = _prefill_args(sq1=(ctypes.c_int64 * 3)(4 * 128 * 64, 128 * 64, 60))   # not a multiple of 8
    assert _rc(lib, a) == da.EINVAL
    a = _prefill_args(out=FAKE)  # out overlaps q1
    assert _rc(lib, a) == da.EINVAL
    assert "overlaps" in lib.diffattn_last_error().decode()
    a = _prefill_args(so=(ctypes.c_int64 * 3)(4 * 128 * 128, 128 * 128, 64))  # rows overlap
    assert _rc(lib, a) == da.EINVAL


def test_prefill_f32_size_limits(lib):
    a = _prefill_args(dtype=da.F32, d_qk=129)
    assert _rc(lib, a) == da.EUNSUPPORTED


def test_empty_prefill_is_a_no_op(lib):
    a = _prefill_args(N=0, q1=None, q2=None, k1=None, k2=None, v=None, out=None)
    assert _rc(lib, a) == da.OK


def _decode_args(**kw):
    a = da.DecodeArgs()
    a.dtype = da.BF16
    a.B, a.H, a.H_kv, a.d_qk, a.d_v = 64, 32, 8, 128, 128
    a.page_size, a.max_pages, a.num_pages = 64, 512, 20000
    step = 1 << 34
    a.q1, a.q2 = FAKE, FAKE + 256
    a.sq1 = (ctypes.c_int64 * 2)(64 * 128, 256)
    a.sq2 = (ctypes.c_int64 * 2)(64 * 128, 256)
    a.k1_cache = a.k2_cache = FAKE + step
    a.v_cache = FAKE + 2 * step
    a.page_table = FAKE + 3 * step
    a.ctx_len = FAKE + 3 * step + (1 << 20)
    a.lambda_ = FAKE + 3 * step + (2 << 20)
    a.depth, a.scale, a.norm, a.gamma, a.eps = 20, 0.0, da.NORM_NONE, None, 1e-5
    a.out = FAKE + 3 * step + (3 << 20)
    a.so = (ctypes.c_int64 * 2)(32 * 128, 128)
    a.split_pages = 0
    a.dev_err = None
    for k, v in kw.items():
        setattr(a, k, v)
    return a


def test_decode_workspace_and_plan(lib):
    # header: int32 page prefix [B + 1] rounded up to 256 bytes; records: one
    # per (work-group, unit) pair, fewer than work-groups + units, each
    # 2 * (H / H_kv) query rows x (128 + 2) floats
    header = -(-65 * 4 // 256) * 256
    record = 4 * 2 * 130 * 4  # H / H_kv = 4
    units = 64 * 8
    a = _decode_args()  # library's choice: at most 2048 work-groups
    assert lib.diffattn_decode_workspace_bytes(ctypes.byref(a)) == header + (2048 + units) * record
    a = _decode_args(split_pages=1024)  # 64 * 8 * 512 pages / 1024 = 256 work-groups
    assert lib.diffattn_decode_workspace_bytes(ctypes.byref(a)) == header + (256 + units) * record
    a = _decode_args(d_qk=64, k2_cache=FAKE + 5 * (1 << 34))  # V1 form: same records
    assert lib.diffattn_decode_workspace_bytes(ctypes.byref(a)) == header + (2048 + units) * record
    a = _decode_args(B=1, H=2, H_kv=1, max_pages=3)  # 3 pages: 1 work-group of at least 4 pages
    assert lib.diffattn_decode_workspace_bytes(ctypes.byref(a)) == 256 + (1 + 1) * 4 * 130 * 4


@pytest.mark.parametrize("field,value,code", [
    ("d_qk", 96, da.EUNSUPPORTED),
    ("page_size", 32, da.EUNSUPPORTED),
    ("dtype", da.F32, da.EUNSUPPORTED),
    ("H", 36, da.EINVAL),               # not a multiple of H_kv
    ("k2_cache", FAKE + 5 * (1 << 34), da.EUNSUPPORTED),
    ("page_table", None, da.EINVAL),
    ("split_pages", -1, da.EINVAL),
    ("split_pages", (1 << 24) + 1, da.EINVAL),
    ("window", -3, da.EINVAL),
    ("out", FAKE, da.EINVAL),           # overlaps q1
    ("kv_dtype", da.F32, da.EINVAL),    # caches: bf16 or fp8 e4m3 only
    ("kv_dtype", 3, da.EINVAL),
])
def test_decode_rejects(lib, field, value, code):
    a = _decode_args(**{field: value})
    assert lib.diffattn_decode(ctypes.byref(a), FAKE + 6 * (1 << 34), 1 << 40, None) == code


def test_decode_fp8_scales_and_extents(lib):
    ws = FAKE + 6 * (1 << 34)
    good = dict(kv_dtype=da.FP8_E4M3, k_scale=0.5, v_scale=0.25)
    a = _decode_args(**good)
    assert lib.diffattn_decode_workspace_bytes(ctypes.byref(a)) == \
        lib.diffattn_decode_workspace_bytes(ctypes.byref(_decode_args()))  # same records as bf16
    for bad in (dict(k_scale=0.0), dict(v_scale=-1.0), dict(k_scale=float("inf")), dict(v_scale=float("nan"))):
        a = _decode_args(**{**good, **bad})
        assert lib.diffattn_decode_workspace_bytes(ctypes.byref(a)) == 0, bad
        assert lib.diffattn_decode(ctypes.byref(a), ws, 1 << 40, None) == da.EINVAL, bad
        assert "scale" in lib.diffattn_last_error().decode()
    # bf16 caches ignore the scales
    a = _decode_args(k_scale=0.0, v_scale=0.0)
    assert lib.diffattn_decode_workspace_bytes(ctypes.byref(a)) > 0
    # the overlap check sizes the caches by their storage: one byte per fp8
    # element, two per bf16 element
    v_end8 = 20000 * 8 * 64 * 128
    for kw in (dict(good, out=FAKE + 2 * (1 << 34) + v_end8 - 256), dict(out=FAKE + 2 * (1 << 34) + v_end8)):
        a = _decode_args(**kw)
        assert lib.diffattn_decode(ctypes.byref(a), ws, 1 << 40, None) == da.EINVAL
        assert "overlaps" in lib.diffattn_last_error().decode()


def test_decode_rejects_small_workspace(lib):
    a = _decode_args()
    need = lib.diffattn_decode_workspace_bytes(ctypes.byref(a))
    assert lib.diffattn_decode(ctypes.byref(a), FAKE + 6 * (1 << 34), need - 1, None) == da.EWORKSPACE
    assert lib.diffattn_decode(ctypes.byref(a), None, need, None) == da.EWORKSPACE


def test_decode_noalloc_checks_before_any_launch(lib):
    # the argument checks are those of diffattn_decode; a request needing more
    # than the 32 MiB static scratch is refused before any device call
    a = _decode_args(B=0)
    assert lib.diffattn_decode_noalloc(ctypes.byref(a), None) == da.OK
    a = _decode_args(sq1=(ctypes.c_int64 * 2)(64 * 128, 7))
    assert lib.diffattn_decode_noalloc(ctypes.byref(a), None) == da.EINVAL
    a = _decode_args(B=4096, H=64, max_pages=1,
                     sq1=(ctypes.c_int64 * 2)(64 * 128, 128), sq2=(ctypes.c_int64 * 2)(64 * 128, 128),
                     so=(ctypes.c_int64 * 2)(64 * 128, 128))
    need = lib.diffattn_decode_workspace_bytes(ctypes.byref(a))
    assert need > 32 << 20
    assert lib.diffattn_decode_noalloc(ctypes.byref(a), None) == da.EWORKSPACE
    assert "scratch" in lib.diffattn_last_error().decode()


def test_lambda_rejects(lib):
    f = lib.diffattn_lambda
    assert f(FAKE, FAKE + 4096, FAKE + 8192, FAKE + 12288, 0, 8, 1, FAKE + 65536, None) == da.EINVAL
    assert f(FAKE, FAKE + 4096, FAKE + 8192, FAKE + 12288, 4, 8, 0, FAKE + 65536, None) == da.EINVAL
    assert f(FAKE, FAKE + 4096, FAKE + 8192, FAKE + 12288, 4, 8, 1, FAKE + 8, None) == da.EINVAL  # alias


def test_decode_workspace_needs_no_pointers(lib):
    a = _decode_args(q1=None, q2=None, k1_cache=None, k2_cache=None, v_cache=None, page_table=None,
                     ctx_len=None, lambda_=None, out=None)
    assert lib.diffattn_decode_workspace_bytes(ctypes.byref(a)) > 0
    a = _decode_args(H=36)   # invalid sizes still give 0
    assert lib.diffattn_decode_workspace_bytes(ctypes.byref(a)) == 0


def _backward_args(**kw):
    a = da.BackwardArgs()
    a.dtype = da.BF16
    a.B, a.H, a.H_kv, a.N, a.d_qk, a.d_v = 1, 4, 2, 128, 64, 128
    step = 1 << 24
    a.q1, a.q2, a.k1, a.k2, a.v = FAKE, FAKE + step, FAKE + 2 * step, FAKE + 3 * step, FAKE + 4 * step
    a.sq1 = a.sq2 = (ctypes.c_int64 * 3)(4 * 128 * 64, 128 * 64, 64)
    a.sk1 = a.sk2 = (ctypes.c_int64 * 3)(2 * 128 * 64, 128 * 64, 64)
    a.sv = (ctypes.c_int64 * 3)(2 * 128 * 128, 128 * 128, 128)
    a.lambda_ = FAKE + 5 * step
    a.depth, a.causal, a.window, a.scale, a.norm, a.eps = 3, 1, 0, 0.0, da.NORM_NONE, 1e-5
    a.o1, a.o2, a.lse1, a.lse2 = FAKE + 6 * step, FAKE + 7 * step, FAKE + 8 * step, FAKE + 9 * step
    a.dout = FAKE + 10 * step
    a.sdo = (ctypes.c_int64 * 3)(4 * 128 * 128, 128 * 128, 128)
    a.dq1, a.dq2, a.dk1, a.dk2, a.dv = (FAKE + (11 + i) * step for i in range(5))
    a.dlambda = FAKE + 16 * step
    a.dgamma = None
    for k, v in kw.items():
        setattr(a, k, v)
    return a


def test_backward_workspace_sizes(lib):
    a = _backward_args()
    rows = 1 * 4 * 128
    r256 = lambda x: -(-x // 256) * 256
    want = r256(rows * 128 * 2) + 4 * r256(rows * 4) + r256(1 * 4 * 2 * 129 * 4)  # blocks of 64 rows
    assert lib.diffattn_backward_workspace_bytes(ctypes.byref(a)) == want
    assert lib.diffattn_backward_workspace_bytes(ctypes.byref(_backward_args(dtype=da.F32))) == 0


@pytest.mark.parametrize("field,value,code", [
    ("dtype", da.F32, da.EUNSUPPORTED),
    ("d_qk", 96, da.EUNSUPPORTED),
    ("o1", None, da.EINVAL),
    ("dout", None, da.EINVAL),
    ("dq1", None, da.EINVAL),
    ("dk2", None, da.EINVAL),                 # two key tensors need two key gradients
    ("dq2", FAKE + 11 * (1 << 24), da.EINVAL),  # overlaps dq1
    ("dv", FAKE, da.EINVAL),                  # overlaps q1
    ("window", 4, None),                      # valid (checked below with causal = 0)
])
def test_backward_rejects(lib, field, value, code):
    a = _backward_args(**{field: value})
    if code is None:
        a.causal = 0
        code = da.EINVAL
    rc = lib.diffattn_backward(ctypes.byref(a), FAKE + 20 * (1 << 24), 1 << 30, None)
    assert rc == code
    assert lib.diffattn_last_error().decode().startswith("diffattn_backward")


def test_backward_rejects_small_workspace(lib):
    a = _backward_args()
    need = lib.diffattn_backward_workspace_bytes(ctypes.byref(a))
    assert lib.diffattn_backward(ctypes.byref(a), FAKE + 20 * (1 << 24), need - 1, None) == da.EWORKSPACE


def test_prefill_rejects_partial_statistics(lib):
    a = _prefill_args(o1=FAKE + 6 * (1 << 24))
    assert _rc(lib, a) == da.EINVAL


def test_lambda_backward_rejects(lib):
    f = lib.diffattn_lambda_backward
    H, dl = 4, 8
    vec = H * dl * 4
    ins = [FAKE + i * 4096 for i in range(4)]       # lq1, lk1, lq2, lk2
    dlam = FAKE + 4 * 4096
    outs = [FAKE + (8 + i) * 4096 for i in range(4)]  # dlq1, dlk1, dlq2, dlk2

    def rc(ins_, dlam_, outs_, H_=H, dl_=dl):
        return f(*ins_, H_, dl_, dlam_, *outs_, None)

    assert rc(ins, dlam, outs, H_=0) == da.EINVAL
    assert rc(ins, dlam, outs, dl_=0) == da.EINVAL
    assert rc(ins, dlam, outs, dl_=4097) == da.EINVAL
    assert rc(ins, None, outs) == da.EINVAL
    assert rc(ins, dlam, outs[:3] + [None]) == da.EINVAL
    assert rc(ins, dlam, [outs[0] + 2] + outs[1:]) == da.EINVAL            # misaligned output
    assert "misaligned" in lib.diffattn_last_error().decode()
    assert rc([ins[0] + 1] + ins[1:], dlam, outs) == da.EINVAL             # misaligned input
    assert rc(ins, dlam, [ins[0]] + outs[1:]) == da.EINVAL                 # in place: dlq1 == lq1
    assert "overlaps an input" in lib.diffattn_last_error().decode()
    assert rc(ins, dlam, outs[:3] + [ins[3] + vec - 4]) == da.EINVAL       # partial overlap with lk2
    assert rc(ins, dlam, outs[:3] + [dlam]) == da.EINVAL                  # overlaps dlambda
    assert rc(ins, dlam, [outs[0], outs[0] + vec - 4] + outs[2:]) == da.EINVAL  # outputs overlap
    assert "outputs overlap" in lib.diffattn_last_error().decode()
    assert lib.diffattn_last_error().decode().startswith("diffattn_lambda_backward")
