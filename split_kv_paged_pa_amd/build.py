"""Build libpa_decode.so (the C-ABI library with the gfx950 kernels) and the
bandwidth probe libpa_probe.so in-tree.

    python split_kv_paged_pa_amd/build.py [-v]

hipcc flags: gfx950 only, -O3, packed-FP32 instructions disabled
(-Xclang -target-feature -Xclang -packed-fp32-ops) so that the compiler never
emits v_pk_{add,mul,fma}_f32, MFMA results kept in ordinary VGPRs (no AGPR
copies around the VALU softmax code), and kernel arguments preloaded into SGPRs
(the first 14-16 dwords arrive with the wave instead of through a load from the
argument buffer; the compiler also emits the loads in a 256-byte prologue that
firmware without preloading runs instead).  Each source is compiled to its own
object with its own flags, then linked.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libpa_decode.so")
VGPR_FORM = ["-mllvm", "-amdgpu-mfma-vgpr-form"]
# Measured on MI355X, 100K-token step: -0.3 us (both kernels start one argument
# load earlier).
PRELOAD = ["-mllvm", "-amdgpu-kernarg-preload-count=16"]
# (source, flags of its own)
SOURCES = [(os.path.join(CSRC, "pa_kernels.hip"), VGPR_FORM + PRELOAD),
           (os.path.join(CSRC, "pa_prefill.hip"), VGPR_FORM + PRELOAD),
           (os.path.join(CSRC, "pa_repack.hip"), []),
           (os.path.join(CSRC, "pa_api.cpp"), [])]
# Diagnostic copy of the same kernels with per-workgroup timestamps
# (-DPA_TIMELINE, csrc/pa_timeline.h); read by bench.py --timeline only.
TIMELINE_LIB = os.path.join(HERE, "libpa_decode_timeline.so")
PROBE_LIB = os.path.join(HERE, "libpa_probe.so")
PROBE_SOURCES = [(os.path.join(CSRC, "pa_probe.hip"), VGPR_FORM),
                 (os.path.join(CSRC, "pa_rates.hip"), [])]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
OBJ_DIR = os.path.join(HERE, "_build")

FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-function"]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)


def _link(sources, lib, verbose, extra, tag=""):
    os.makedirs(OBJ_DIR, exist_ok=True)
    objs = []
    for src, own in sources:
        obj = os.path.join(OBJ_DIR, os.path.basename(src) + tag + ".o")
        _run([HIPCC, *FLAGS, *own, *extra, "-x", "hip", "-c", src, "-o", obj], verbose)
        objs.append(obj)
    tmp = lib + ".tmp"
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-Wl,--no-undefined", *objs,
          "-o", tmp], verbose)
    os.replace(tmp, lib)


def build(verbose: bool = False, extra=()) -> str:
    """libpa_decode.so (the attention ABI), libpa_probe.so (bandwidth probe) and
    libpa_decode_timeline.so (the same kernels with timestamps, diagnostic)."""
    _link(SOURCES, LIB, verbose, extra)
    _link(PROBE_SOURCES, PROBE_LIB, verbose, extra)
    _link(SOURCES, TIMELINE_LIB, verbose, (*extra, "-DPA_TIMELINE"), tag=".timeline")
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
