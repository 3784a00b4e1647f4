"""Builds libmsa.so (the HIP kernels and the C-ABI of include/msa.h) for gfx950.

Each .hip source is compiled to an object in its own hipcc process (in parallel),
then the objects are linked into block_sparse_long_11_amd/libmsa.so.
"""
import concurrent.futures
import os
import pathlib
import subprocess
import sys

PKG = pathlib.Path(__file__).resolve().parent
ROOT = PKG.parent
CSRC = PKG / "csrc"
BUILD = ROOT / "_build"
LIB = PKG / "libmsa.so"
PROBE = CSRC / "probe"
PROBE_LIB = PKG / "libmsa_probe.so"      # peak-rate probes used by bench.py
ARCH = "gfx950"

CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    f"-I{ROOT / 'include'}", f"-I{CSRC}",
    # never emit packed fp32 VALU ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # NaN inputs are undefined behaviour of the API: let fmaxf/fminf skip the
    # canonicalisation of every operand (halves the max-pooling VALU work)
    "-fno-honor-nans",
    "-Wno-unused-command-line-argument",
]


def _hipcc():
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def _compile(src: pathlib.Path, extra, flags=CFLAGS, out_dir=BUILD):
    obj = out_dir / (src.stem + ".o")
    cmd = [_hipcc(), *flags, *extra, "-c", str(src), "-o", str(obj)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src.name}:\n{res.stderr}")
    return obj


def _link(objs, lib):
    tmp = lib.with_suffix(".so.tmp")
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", str(tmp),
           *map(str, objs)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stderr}")
    os.replace(tmp, lib)


def build(verbose=False, extra=()):
    """Compile every kernel source and link libmsa.so (and the peak-rate probes into
    libmsa_probe.so). Returns the library path."""
    BUILD.mkdir(exist_ok=True)
    srcs = sorted(CSRC.glob("*.hip"))
    probes = sorted(PROBE.glob("*.hip"))
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs) + len(probes))) as ex:
        objs = list(ex.map(lambda s: _compile(s, list(extra)), srcs + probes))
    _link(objs[:len(srcs)], LIB)
    if probes:
        _link(objs[len(srcs):], PROBE_LIB)
    if verbose:
        print(f"built {LIB}" + (f" and {PROBE_LIB.name}" if probes else ""))
    return LIB


def build_host_asan(verbose=False):
    """A copy of libmsa.so whose host code (argument checks, plan, validators,
    launch set-up) is built with AddressSanitizer, for the CPU tests of the C ABI:
    `_build/asan/libmsa.so`. Its device code is the same source at -O1 and is never
    launched from those tests. Loading it needs the ASan runtime preloaded."""
    out = BUILD / "asan"
    out.mkdir(parents=True, exist_ok=True)
    flags = [f if f != "-O3" else "-O1" for f in CFLAGS] + [
        "-g", "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]
    srcs = sorted(CSRC.glob("*.hip"))
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, [], flags, out), srcs))
    lib = out / "libmsa.so"
    _link(objs, lib)
    if verbose:
        print(f"built {lib}")
    return lib


if __name__ == "__main__":
    build(verbose=True, extra=sys.argv[1:])
