"""Host sanitizer pass over the C++ block manager and radix index (CPU only).

The bookkeeping code (free stack, reference counts, copy-on-write, prefix
registry, swap pool, radix tree) is pointer- and index-heavy host C++.  This
test builds it host-only with AddressSanitizer and UndefinedBehaviorSanitizer
(g++, no GPU code: every GPU entry point of the header is a stub that
returns PKV_ERR_DEVICE), then runs the random-operation and scripted native
tests, which compare it bit for bit with the oracle's model, against that
build in a subprocess with the ASan runtime preloaded.  Any sanitizer report
fails the test.
"""
import os
import re
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "paged_kv_cache_230_amd", "csrc")
HOST_SOURCES = ["block_manager.cpp", "radix.cpp"]
NATIVE_TESTS = ["test_block_manager_native.py", "test_prefix_cache_native.py", "test_radix_native.py",
                "test_swap_native.py"]


def _runtime(name):
    gxx = shutil.which("g++")
    if not gxx:
        return None
    path = subprocess.run([gxx, f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def _gpu_stub_source():
    """Stubs for every header function the host sources do not define."""
    sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
    from test_capi import declared_functions

    host = "".join(open(os.path.join(CSRC, f)).read() for f in HOST_SOURCES)
    defined = set(re.findall(r"^[A-Za-z_][\w\s\*]*?\b((?:pkv|paged)_[a-z0-9_]*)\s*\([^;]*?\)\s*\{", host, flags=re.M))
    lines = ["#include <string>", "namespace pkv {",
             "std::string& last_error_slot() { thread_local std::string m; return m; }",
             "int stage_device_ptr(const int*, const int**) { last_error_slot() = \"host-only build\"; return -4; }",
             "int launch_stage(const int*, int, int, int, int, int*, int*, int*, int*, void*) { return -4; }",
             "}", 'extern "C" {',
             "const char* pkv_last_error(void) { return pkv::last_error_slot().c_str(); }"]
    for name in declared_functions():
        if name not in defined and name != "pkv_last_error":
            lines.append(f"long {name}(void) {{ pkv::last_error_slot() = \"host-only build\"; return -4; }}")
    lines.append("}")
    return "\n".join(lines) + "\n"


@pytest.mark.skipif(shutil.which("g++") is None or _runtime("libasan.so") is None or _runtime("libubsan.so") is None,
                    reason="g++ with the ASan/UBSan runtimes is not available")
def test_block_manager_and_radix_under_asan_ubsan(tmp_path):
    stubs = tmp_path / "gpu_stubs.cpp"
    stubs.write_text(_gpu_stub_source())
    lib = tmp_path / "libpagedkv_hostsan.so"
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=undefined", "-shared", "-fPIC", "-Wall",
           *[os.path.join(CSRC, f) for f in HOST_SOURCES], str(stubs), "-o", str(lib)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-3000:]
    env = dict(os.environ)
    env.update(PKV_LIB_PATH=str(lib), LD_PRELOAD=_runtime("libasan.so"),
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", HIP_VISIBLE_DEVICES="", CUDA_VISIBLE_DEVICES="")
    # -s: a sanitizer report goes to the process's stderr, which pytest's own
    # capture would otherwise swallow when the runtime ends the process
    run = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-s", "-p", "no:cacheprovider", "-m", "not gpu",
                          *[os.path.join(ROOT, "tests", t) for t in NATIVE_TESTS]],
                         capture_output=True, text=True, env=env, cwd=ROOT, timeout=900)
    out = run.stdout + run.stderr
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert run.returncode == 0, out[-4000:]
    assert re.search(r"\d+ passed", out), out[-2000:]
