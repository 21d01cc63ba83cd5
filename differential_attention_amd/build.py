"""Build libdiffattn.so (gfx950) in-tree with hipcc.

    python -m differential_attention_amd.build [--resources]

--resources also prints the compiler's per-kernel resource report (registers,
spills, scratch, LDS, occupancy), which every build writes to
_build/kernel_resources.json.

Every HIP translation unit is compiled for gfx950 only. Packed-fp32 VALU ops
are disabled in device code (-packed-fp32-ops); hipcc's host pass warns that
it does not know that feature, which is harmless.
"""
from __future__ import annotations

import concurrent.futures as cf
import json
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libdiffattn.so")

HIP_SOURCES = ["lambda.hip", "prefill_f32.hip", "prefill_bf16.hip", "decode.hip", "backward.hip"]
HOST_SOURCES = ["api.cpp"]      # host code that calls the HIP runtime
PLAIN_SOURCES = ["plan.cpp"]    # host code with no HIP dependency

ARCH = "gfx950"
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
# per-source device flags:
#  * prefill_bf16.hip is compiled without NaN semantics, so fmaxf needs no
#    canonicalising v_max per operand in the row-max reductions (about 3 %
#    faster). Its arithmetic never produces a NaN from finite inputs: masked
#    scores are -inf, exp2(-inf) = 0, and the rescale never subtracts -inf
#    from -inf; infinities keep their IEEE meaning.
SOURCE_FLAGS = {
    "prefill_bf16.hip": ["-fno-honor-nans"],
}


def _hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (expected /opt/rocm/bin/hipcc)")


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l and l.strip())
    if r.returncode != 0:
        raise RuntimeError("command failed: " + " ".join(cmd) + "\n" + out)
    return out


# The compiler's per-kernel resource remarks (-Rpass-analysis=kernel-resource-usage),
# collected while the HIP sources compile: registers, spills, scratch, LDS and
# the occupancy they allow, written to _build/kernel_resources.json.
RESOURCES = os.path.join(BUILD, "kernel_resources.json")
_REMARK = "-Rpass-analysis=kernel-resource-usage"
_FIELDS = {
    "TotalSGPRs": "sgprs", "VGPRs": "vgprs", "AGPRs": "agprs", "ScratchSize [bytes/lane]": "scratch_bytes_per_lane",
    "Occupancy [waves/SIMD]": "occupancy_waves_per_simd", "SGPRs Spill": "sgpr_spill", "VGPRs Spill": "vgpr_spill",
    "LDS Size [bytes/block]": "lds_bytes",
}


def _demangle(names):
    try:
        r = subprocess.run(["c++filt"], input="\n".join(names), stdout=subprocess.PIPE, text=True, check=True)
        out = r.stdout.splitlines()
        if len(out) == len(names):
            return out
    except (OSError, subprocess.CalledProcessError):
        pass
    return list(names)


def parse_resources(text: str, source: str):
    """Kernels and their resource fields from the compiler's remarks."""
    kernels, cur = [], None
    for line in text.splitlines():
        if "remark:" not in line or "kernel-resource-usage" not in line:
            continue
        body = line.split("remark:", 1)[1].replace("[" + _REMARK + "]", "").strip()
        key, _, val = body.partition(": ")
        if key == "Function Name":
            cur = {"source": source, "mangled": val.strip()}
            kernels.append(cur)
        elif cur is not None and key in _FIELDS:
            v = val.strip()
            cur[_FIELDS[key]] = int(v) if v.lstrip("-").isdigit() else v
    names = _demangle([k["mangled"] for k in kernels])
    for k, n in zip(kernels, names):
        n = n.replace("da::(anonymous namespace)::", "").replace("da::", "")
        n = n[5:] if n.startswith("void ") else n
        k["kernel"] = n.split("(")[0] if "(" in n else n
    return kernels


def resources_table(kernels) -> str:
    """The report as a markdown table."""
    rows = ["| Source | Kernel | VGPRs | AGPRs | SGPRs | Scratch B/lane | VGPR spill | LDS B | Waves/SIMD |",
            "|---|---|---|---|---|---|---|---|---|"]
    for k in kernels:
        rows.append(f"| {k['source']} | `{k['kernel']}` | {k.get('vgprs')} | {k.get('agprs')} | {k.get('sgprs')} | "
                    f"{k.get('scratch_bytes_per_lane')} | {k.get('vgpr_spill')} | {k.get('lds_bytes')} | "
                    f"{k.get('occupancy_waves_per_simd')} |")
    return "\n".join(rows)


def build(verbose: bool = False, jobs: int = 4) -> str:
    """Compile every source and link libdiffattn.so. Always recompiles."""
    hipcc = _hipcc()
    os.makedirs(BUILD, exist_ok=True)
    common = ["-O3", "-fPIC", "-std=c++17", "-I", INCLUDE, "-I", CSRC, "-Wall"]
    cmds = []
    objs = []
    for s in HIP_SOURCES:
        o = os.path.join(BUILD, s + ".o")
        cmds.append([hipcc, "-x", "hip", f"--offload-arch={ARCH}", *DEVICE_FLAGS, *SOURCE_FLAGS.get(s, []),
                     *common, _REMARK, "-c", os.path.join(CSRC, s), "-o", o])
        objs.append(o)
    for s in HOST_SOURCES:
        o = os.path.join(BUILD, s + ".o")
        cmds.append([hipcc, *common, "-c", os.path.join(CSRC, s), "-o", o])
        objs.append(o)
    for s in PLAIN_SOURCES:
        o = os.path.join(BUILD, s + ".o")
        cmds.append(["g++", *common, "-c", os.path.join(CSRC, s), "-o", o])
        objs.append(o)
    kernels = []
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        for cmd, out in zip(cmds, ex.map(_run, cmds)):
            if _REMARK in cmd:
                kernels += parse_resources(out, os.path.basename(cmd[cmd.index("-c") + 1]))
                out = "\n".join(l for l in out.splitlines() if "kernel-resource-usage" not in l)
            if verbose and out:
                print(out)
    with open(RESOURCES, "w") as f:
        json.dump(kernels, f, indent=1)
    tmp = LIB + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
    if "--resources" in sys.argv:
        with open(RESOURCES) as f:
            print(resources_table(json.load(f)))
