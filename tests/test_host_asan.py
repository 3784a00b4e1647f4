"""The host side of the C ABI under AddressSanitizer: every CPU test of
tests/test_abi.py (argument checks, the prefill plan, the validators, MSA_LOG)
run against a copy of libmsa.so whose host code is ASan-instrumented, in a child
process with the ASan runtime preloaded. Any heap or stack overrun in that code
ends the child with a report instead of passing. Device code is not instrumented
(there is no GPU sanitizer here) and no kernel is launched."""
import os
import subprocess
import sys

import pytest

from block_sparse_long_11_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

DRIVER = """
import ctypes, pathlib, sys
import pytest
import block_sparse_long_11_amd as msa
assert hasattr(ctypes.CDLL(None), "__asan_report_load16"), "ASan runtime not loaded"
msa._LIB_PATH = pathlib.Path(sys.argv[1])
sys.exit(pytest.main(["-q", "-x", "-m", "not gpu", "-p", "no:cacheprovider",
                      "tests/test_abi.py"]))
"""


def asan_runtime():
    clang = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "llvm", "bin", "clang")
    try:
        out = subprocess.run([clang, "-print-file-name=libclang_rt.asan-x86_64.so"],
                             capture_output=True, text=True, timeout=60).stdout.strip()
    except OSError:
        return None
    return out if os.path.isabs(out) and os.path.exists(out) else None


def test_abi_host_code_under_asan():
    rt = asan_runtime()
    if rt is None:
        pytest.skip("no ASan runtime in this toolchain")
    lib = build.build_host_asan()
    readelf = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "llvm", "bin",
                           "llvm-readelf")
    syms = subprocess.run([readelf, "--dyn-syms", str(lib)], capture_output=True, text=True,
                          timeout=60).stdout
    assert "__asan_report_load" in syms, "host code is not instrumented"
    env = dict(os.environ)
    env["LD_PRELOAD"] = rt + (":" + env["LD_PRELOAD"] if env.get("LD_PRELOAD") else "")
    # the interpreter and torch leak by design; only memory errors count here
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:verify_asan_link_order=0"
    env["HIP_VISIBLE_DEVICES"] = ""
    r = subprocess.run([sys.executable, "-c", DRIVER, str(lib)], cwd=ROOT, env=env,
                       capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in r.stdout, out[-2000:]
