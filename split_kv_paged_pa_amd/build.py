"""Build libpa_decode.so (the C-ABI library with the gfx950 kernels) and the
bandwidth probe libpa_probe.so in-tree.

    python split_kv_paged_pa_amd/build.py [-v]

hipcc flags: gfx950 only, -O3, MFMA results kept in ordinary VGPRs (no
AGPR copies around the VALU softmax code), and packed-FP32 instructions disabled
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
PROBE_LIB = os.path.join(HERE, "libpa_probe.so")
PROBE_SOURCES = [os.path.join(CSRC, "pa_probe.hip")]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-mllvm", "-amdgpu-mfma-vgpr-form",
         "-Wall", "-Wno-unused-function", "-Wl,--no-undefined"]


def _link(sources, lib, verbose, extra):
    tmp = lib + ".tmp"
    cmd = [HIPCC, *FLAGS, *extra, "-x", "hip", *sources, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, lib)


def build(verbose: bool = False, extra=()) -> str:
    """libpa_decode.so (the attention ABI) and libpa_probe.so (bandwidth probe)."""
    _link(SOURCES, LIB, verbose, extra)
    _link(PROBE_SOURCES, PROBE_LIB, verbose, extra)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
