"""The host library and the oracle under AddressSanitizer and UndefinedBehavior-
Sanitizer, on the CPU.

libpa_decode.so is rebuilt with the sanitizers on its host code only (hipcc with
-Xarch_host before each sanitizer flag; the gfx950 device code is built as
usual), and the oracle's C with the same clang, into a temporary directory.  A
child Python process with the clang ASan runtime preloaded then runs the ABI
tests (every argument check of every entry point, none of which reaches a
launch) and the oracle pins against those builds.  Any sanitizer report fails
the test: both runtimes halt on the first error and write their reports to
files that must stay empty."""
import glob
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "split_kv_paged_pa_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANG = "/opt/rocm/llvm/bin/clang"


def _asan_runtime():
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


def _build(out):
    """The sanitized libraries in out/: libpa_decode_san.so and libpa_oracle_san.so."""
    flags = ["-x", "hip", "--offload-arch=gfx950", "-O1", "-g", "-fPIC", "-std=c++17",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-mllvm", "-amdgpu-mfma-vgpr-form"] + HOST_SAN
    objs = []
    # every source of libpa_decode.so, as build.py lists them
    sys.path.insert(0, ROOT)
    from split_kv_paged_pa_amd import build as pa_build
    for path, _ in pa_build.SOURCES:
        obj = os.path.join(out, os.path.basename(path) + ".o")
        subprocess.run([HIPCC, *flags, "-c", path, "-o", obj], check=True, capture_output=True)
        objs.append(obj)
    lib = os.path.join(out, "libpa_decode_san.so")
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", lib],
                   check=True, capture_output=True)
    olib = os.path.join(out, "libpa_oracle_san.so")
    subprocess.run([CLANG, "-O1", "-g", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
                    "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=undefined", os.path.join(ROOT, "oracle", "pa_oracle.c"),
                    "-o", olib, "-lm"], check=True, capture_output=True)
    return lib, olib


DRIVER = """
import sys
sys.path.insert(0, {root!r})
sys.path.insert(0, {tests!r})
import split_kv_paged_pa_amd.api as api
api.LIB_PATH = {lib!r}
import oracle
oracle._LIB_PATH = {olib!r}
import pytest
sys.exit(pytest.main([{abi!r}, {pins!r}, "-x", "-q", "-p", "no:cacheprovider"]))
"""


def test_abi_and_oracle_pins_under_asan_ubsan(tmp_path):
    rt = _asan_runtime()
    if rt is None or not os.path.exists(HIPCC) or not os.path.exists(CLANG):
        pytest.skip("the ROCm clang sanitizer runtime or compilers are not installed")
    lib, olib = _build(str(tmp_path))
    logs = tmp_path / "logs"
    logs.mkdir()
    env = dict(os.environ)
    env.update({
        "LD_PRELOAD": rt,
        "LD_LIBRARY_PATH": "/opt/rocm/llvm/lib:" + env.get("LD_LIBRARY_PATH", ""),
        # Python itself is not instrumented and keeps objects alive at exit: no leak check.
        "ASAN_OPTIONS": f"detect_leaks=0:halt_on_error=1:log_path={logs}/asan",
        "UBSAN_OPTIONS": f"halt_on_error=1:print_stacktrace=1:log_path={logs}/ubsan",
    })
    code = DRIVER.format(root=ROOT, tests=os.path.join(ROOT, "tests"), lib=lib, olib=olib,
                         abi=os.path.join(ROOT, "tests", "test_abi.py"),
                         pins=os.path.join(ROOT, "tests", "test_oracle_pins.py"))
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True,
                       timeout=600, cwd=str(tmp_path))
    reports = "".join(open(p).read() for p in glob.glob(str(logs / "*")))
    assert r.returncode == 0 and not reports, (
        f"rc {r.returncode}\n{r.stdout[-3000:]}\n{r.stderr[-3000:]}\n{reports[:6000]}")
    assert " passed" in r.stdout
    shutil.rmtree(tmp_path, ignore_errors=True)
