"""Register budget of the HIP kernels, checked at compile time (CPU only).

The decode kernel's speed rests on holding one step of K/V loads in flight
per wave at three waves per SIMD, and several tempting changes push it into
register spills instead.  This test compiles each kernel source for gfx950
with the library's flags and reads the compiler's resource-usage remarks:
no kernel may spill vector registers, and the kernels keep the occupancy
their design assumes.
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "paged_kv_cache_230_amd", "csrc")
SOURCES = ["pagedkv_kernels.hip", "prefill_kernel.hip", "swap_kernel.hip"]


def _hipcc():
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    return None


def _usage(src, tmp_path):
    """{mangled kernel name: {"vgpr_spill": n, "waves": n}} from the remarks."""
    out = tmp_path / (src + ".o")
    cmd = [_hipcc(), "--offload-arch=gfx950", "-O3", "-std=c++17", "-c", "--offload-device-only",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-Rpass-analysis=kernel-resource-usage", os.path.join(CSRC, src), "-o", str(out)]
    res = subprocess.run(cmd, capture_output=True, text=True, cwd=CSRC)
    assert res.returncode == 0, res.stderr[-2000:]
    kernels, name = {}, None
    for line in res.stderr.splitlines():
        m = re.search(r"remark: Function Name: (\S+)", line)
        if m:
            name = m.group(1)
            kernels[name] = {}
            continue
        if name is None:
            continue
        m = re.search(r"remark:\s+VGPRs Spill: (\d+)", line)
        if m:
            kernels[name]["vgpr_spill"] = int(m.group(1))
        m = re.search(r"remark:\s+Occupancy \[waves/SIMD\]: (\d+)", line)
        if m:
            kernels[name]["waves"] = int(m.group(1))
    return kernels


@pytest.mark.skipif(_hipcc() is None, reason="hipcc not available")
def test_no_vector_register_spills_and_design_occupancy(tmp_path):
    found = {}
    for src in SOURCES:
        found.update(_usage(src, tmp_path))
    assert found, "no kernel resource remarks parsed"
    for name, u in found.items():
        assert "vgpr_spill" in u and "waves" in u, f"incomplete remarks for {name}"
        assert u["vgpr_spill"] == 0, f"{name} spills {u['vgpr_spill']} vector registers"
    # bf16 decode at head_dim 128 (the 8B/70B-shaped layers), both cache
    # policies (streamed, shared blocks): three waves per SIMD
    for bs in (16, 32):
        for shared in (0, 1):
            key = f"_ZN12_GLOBAL__N_113decode_kernelILb1ELi128ELi{bs}ELb{shared}EEEvNS_10DecodeArgsE"
            assert key in found, f"missing {key}"
            assert found[key]["waves"] >= 3, f"{key}: {found[key]['waves']} waves per SIMD"
    # chunked prefill at head_dim 128: two waves per SIMD (8 waves, one workgroup per compute unit)
    for bs in (16, 32):
        key = f"_ZN12_GLOBAL__N_114prefill_kernelILi128ELi{bs}EEEvNS_11PrefillArgsE"
        assert key in found, f"missing {key}"
        assert found[key]["waves"] >= 2, f"{key}: {found[key]['waves']} waves per SIMD"
