"""Kernel resources as the compiler reports them (registers, spills, LDS,
occupancy), recorded by every build in _build/kernel_resources.json: the
limits each kernel's design relies on. CPU only (the report comes from the
gfx950 compile)."""
import json
import os

import pytest

from differential_attention_amd import build as B

LDS_PER_CU = 160 * 1024  # gfx950


@pytest.fixture(scope="module")
def kernels():
    if not os.path.exists(B.RESOURCES):
        B.build()
    with open(B.RESOURCES) as f:
        ks = json.load(f)
    return {k["kernel"]: k for k in ks}


def _of(kernels, prefix):
    found = [k for name, k in kernels.items() if name.startswith(prefix)]
    assert found, f"no {prefix} kernel in the report"
    return found


def test_every_source_and_kernel_is_reported(kernels):
    assert {k["source"] for k in kernels.values()} == set(B.HIP_SOURCES)
    for name in ("lambda_kernel", "prefill_f32_kernel", "decode_combine_kernel", "bwd_prep_kernel",
                 "bwd_finalize_kernel", "lambda_backward_kernel",
                 "prefill_bf16_kernel<64, false, true, false, false>",
                 "prefill_bf16_kernel<128, true, false, false, false>",
                 "decode_split_kernel<128, false>", "decode_split_kernel<64, true>",
                 "bwd_dq_kernel<128, true, false>", "bwd_dkdv_kernel<128, true, false>"):
        assert name in kernels, name
    for k in kernels.values():
        for f in ("vgprs", "agprs", "scratch_bytes_per_lane", "lds_bytes", "occupancy_waves_per_simd"):
            assert isinstance(k.get(f), int), (k["kernel"], f)


def test_every_kernel_fits_a_compute_unit(kernels):
    for k in kernels.values():
        assert k["vgprs"] + k["agprs"] <= 512, k["kernel"]
        assert k["lds_bytes"] <= LDS_PER_CU, k["kernel"]
        assert k["occupancy_waves_per_simd"] >= 1, k["kernel"]


def test_prefill_runs_two_waves_per_simd(kernels):
    # 8-wave work-groups, one per compute unit: two waves share each SIMD, and
    # the LDS (two key/value stages) leaves room for that one work-group
    for k in _of(kernels, "prefill_bf16_kernel<"):
        assert k["occupancy_waves_per_simd"] >= 2, k["kernel"]
        assert k["vgprs"] + k["agprs"] <= 256, k["kernel"]


def test_prefill_d128_kernels_do_not_spill(kernels):
    for k in _of(kernels, "prefill_bf16_kernel<128"):
        assert k["scratch_bytes_per_lane"] == 0, k["kernel"]


def test_prefill_d64_spills_stay_small(kernels):
    # the two-branch d_qk 64 kernels hold 256 registers a lane and spill a
    # few (the longctx_v1 kernel: stores in the prologue, reloads in the
    # general per-lane-address tile copy of the sequence's last tile)
    for k in _of(kernels, "prefill_bf16_kernel<64"):
        assert k["scratch_bytes_per_lane"] <= 128, k["kernel"]


def test_decode_split_is_spill_free_with_two_waves(kernels):
    for k in _of(kernels, "decode_split_kernel<"):
        assert k["scratch_bytes_per_lane"] == 0, k["kernel"]
        assert k["occupancy_waves_per_simd"] >= 2, k["kernel"]


def test_backward_dkdv_holds_one_wave_a_simd(kernels):
    # key-major: 4 waves of 32 keys, both branches' accumulators in one wave
    # (VGPRs and AGPRs together), so one wave per SIMD
    for k in _of(kernels, "bwd_dkdv_kernel<"):
        assert k["vgprs"] + k["agprs"] > 256, k["kernel"]
        assert k["occupancy_waves_per_simd"] == 1, k["kernel"]


def test_backward_dq_holds_both_branches_without_spills(kernels):
    # 4 waves of 32 rows, both branches per wave (VGPRs and AGPRs together):
    # one wave per SIMD and nothing spilled
    for k in _of(kernels, "bwd_dq_kernel<"):
        assert k["scratch_bytes_per_lane"] == 0, k["kernel"]
        assert k["occupancy_waves_per_simd"] == 1, k["kernel"]
