"""Build libpa_decode.so (the C-ABI library with the gfx950 kernels) in-tree.

    python split_kv_paged_pa_amd/build.py [-v]

hipcc flags: gfx950 only, -O3, and packed-FP32 instructions disabled
(-Xclang -target-feature -Xclang -packed-fp32-ops) so that the compiler never
emits v_pk_{add,mul,fma}_f32.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libpa_decode.so")
SOURCES = [os.path.join(CSRC, "pa_kernels.hip"), os.path.join(CSRC, "pa_api.cpp")]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-function", "-Wl,--no-undefined"]


def build(verbose: bool = False, extra=()) -> str:
    tmp = LIB + ".tmp"
    cmd = [HIPCC, *FLAGS, *extra, "-x", "hip", *SOURCES, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
