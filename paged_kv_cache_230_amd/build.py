"""Build libpagedkv.so in-tree with hipcc for gfx950.

``python paged_kv_cache_230_amd/build.py`` (or ``build()``) compiles the HIP
kernels and the host block manager into one shared library next to this
file.  The build always recompiles; the output is replaced atomically.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_NAME = "libpagedkv.so"
# A/B library whose bf16 decode kernel runs the Q.K and P.V products on the
# vector ALUs instead of the matrix cores (same loads, split and merge); it
# exists to measure that choice and is loaded only through PKV_LIB_PATH.
VALU_AB_LIB_NAME = "libpagedkv_valu_ab.so"
SOURCES = ["csrc/pagedkv_kernels.hip", "csrc/prefill_kernel.hip", "csrc/swap_kernel.hip", "csrc/measure_kernel.hip",
           "csrc/block_manager.cpp", "csrc/radix.cpp"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libpagedkv)")


def command(out_path: str, defines: tuple[str, ...] = ()) -> list[str]:
    return [
        hipcc(),
        f"--offload-arch={ARCH}",
        "-O3",
        *[f"-D{d}" for d in defines],
        "-std=c++17",
        "-fPIC",
        "-shared",
        "-Wall",
        # keep the compiler from forming packed fp32 VALU ops
        "-Xclang",
        "-target-feature",
        "-Xclang",
        "-packed-fp32-ops",
        *[os.path.join(HERE, s) for s in SOURCES],
        "-o",
        out_path,
    ]


def build(verbose: bool = False, valu_ab: bool = False) -> str:
    out = os.path.join(HERE, VALU_AB_LIB_NAME if valu_ab else LIB_NAME)
    tmp = out + ".tmp"
    cmd = command(tmp, ("PKV_DECODE_VALU_DOT=1",) if valu_ab else ())
    res = subprocess.run(cmd, cwd=HERE, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    log = "\n".join(l for l in (res.stdout + res.stderr).splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{' '.join(cmd)}\n{log}")
    if verbose and log.strip():
        print(log, file=sys.stderr)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True, valu_ab="--valu-ab" in sys.argv[1:]))
