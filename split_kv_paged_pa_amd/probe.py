"""Binding of libpa_probe.so: an HBM read-bandwidth probe with the decode
kernels' access shape, an instruction-rate probe and an LDS read-pattern probe
(measurement only; not part of the attention ABI)."""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpa_probe.so")
_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: run `python split_kv_paged_pa_amd/build.py`")
        lib = ctypes.CDLL(LIB_PATH)
        P, I = ctypes.c_void_p, ctypes.c_int
        lib.pa_probe_read.argtypes = [P, P, I, I, I, I, I, P, P]
        lib.pa_probe_read.restype = I
        lib.pa_probe_rates.argtypes = [I, I, P, I, I, I, P]
        lib.pa_probe_rates.restype = I
        lib.pa_probe_lds_pattern.argtypes = [P, P, I, I, P]
        lib.pa_probe_lds_pattern.restype = I
        lib.pa_probe_read_xcd.argtypes = [P, P, I, I, I, I, P, P, P]
        lib.pa_probe_read_xcd.restype = I
        _lib = lib
    return _lib


def read_bandwidth(buf: torch.Tensor, chunk_ids, chunk_bytes=4096, waves_per_group=4,
                   num_groups=1024, reps=20, stream=None, shape=0):
    """GB/s of reading the chunks of `buf` (a GPU tensor) listed in chunk_ids
    (int32 GPU tensor, or None for all chunks in order), timed with HIP events
    over `reps` launches on `stream`.  shape 0: 1 KiB contiguous per load
    instruction; shape 1: the attention kernels' 16-rows-by-64-bytes shape."""
    nbytes = buf.numel() * buf.element_size()
    n = nbytes // chunk_bytes if chunk_ids is None else chunk_ids.numel()
    if chunk_ids is not None:
        assert chunk_ids.dtype == torch.int32 and chunk_ids.is_cuda
        hi = int(chunk_ids.max().item())
        lo = int(chunk_ids.min().item())
        assert lo >= 0 and (hi + 1) * chunk_bytes <= nbytes, "chunk ids out of range"
    sink = torch.empty(num_groups * waves_per_group * 64, dtype=torch.int32, device=buf.device)
    st = stream or torch.cuda.current_stream()
    args = (ctypes.c_void_p(buf.data_ptr()),
            ctypes.c_void_p(0 if chunk_ids is None else chunk_ids.data_ptr()), int(n),
            int(chunk_bytes), int(waves_per_group), int(num_groups), int(shape),
            ctypes.c_void_p(sink.data_ptr()), ctypes.c_void_p(st.cuda_stream))
    lib = _load()
    assert lib.pa_probe_read(*args) == 0
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(st)
    for _ in range(reps):
        assert lib.pa_probe_read(*args) == 0
    e1.record(st)
    torch.cuda.synchronize()
    sec = e0.elapsed_time(e1) * 1e-3 / reps
    return n * chunk_bytes / sec / 1e9


RATE_KINDS = {0: "v_exp_f32", 1: "v_fma_f32", 2: "v_mfma_f32_16x16x32_bf16",
              3: "mfma + 3 independent fma", 4: "ds_read_b128 (8 then wait)"}
_RATE_INSTRS = {0: 8, 1: 8, 2: 8, 3: 32, 4: 8}  # instructions per round


def issue_rates(iters=4000, blocks=256):
    """Cycles per instruction per wave for each instruction stream of
    pa_rates.hip: one wave per SIMD (256 threads, one workgroup per CU), two
    waves of the same stream, and two waves of different streams sharing each
    SIMD (waves w and w + 4 of 512 threads).  Returns a list of rows
    {"lo", "hi", "threads", "clock_ghz", "lo_cycles_per_instr", "hi_cycles_per_instr"}."""
    import numpy as np
    lib = _load()
    rows = []
    pairs = [(k, k, t) for k in range(5) for t in (256, 512)] + [(2, 1, 512), (2, 0, 512), (2, 4, 512)]
    for lo, hi, threads in pairs:
        waves = blocks * threads // 64
        out = torch.zeros(waves * 3, dtype=torch.int64, device="cuda")
        st = torch.cuda.current_stream()
        assert lib.pa_probe_rates(lo, hi, ctypes.c_void_p(out.data_ptr()), blocks, threads, iters,
                                  ctypes.c_void_p(st.cuda_stream)) == 0
        torch.cuda.synchronize()
        o = out.cpu().numpy().reshape(waves, 3).astype(np.float64)
        cyc, rt = o[:, 0], o[:, 1]
        per_wg = threads // 64
        idx = np.arange(waves) % per_wg
        row = {"lo": RATE_KINDS[lo], "hi": RATE_KINDS[hi], "threads": threads,
               "clock_ghz": round(float(np.median(cyc / rt)) * 0.1, 3),
               "lo_cycles_per_instr": round(float(np.median(cyc[(idx & 4) == 0])) / (iters * _RATE_INSTRS[lo]), 2)}
        if threads == 512:
            row["hi_cycles_per_instr"] = round(float(np.median(cyc[(idx & 4) != 0])) / (iters * _RATE_INSTRS[hi]), 2)
        rows.append(row)
    return rows


def _bits_pattern(bits):
    """Lane l reads 16-byte slot (lane bits `bits`, packed) of 256-byte line
    (the other two lane bits, packed): the 16 lanes of a group read 16 distinct
    slots exactly when the group's lanes vary in the bits `bits` and agree in
    the other two."""
    rest = [b for b in range(6) if b not in bits]
    offs = []
    for lane in range(64):
        slot = sum(((lane >> b) & 1) << i for i, b in enumerate(bits))
        line = sum(((lane >> b) & 1) << i for i, b in enumerate(rest))
        offs.append(256 * line + 16 * slot)
    return offs


def _prefill_pattern(kind):
    """The per-lane LDS offsets of the tiled prefill's operand reads at D = 128
    (lane = n + 16 q; regions 4096 + 128 bytes apart): key tile 0 and 1, values
    in slab order, and values under the earlier permutation (token-half bit
    flipped by bits 3 and 4 of the piece index)."""
    region = 4096 + 128
    offs = []
    for lane in range(64):
        n, q = lane & 15, lane >> 4
        kb = (n >> 2) & 1
        if kind == "k0":
            o = (n >> 3) * region + q * 256 + (12 * kb + (n & 3)) * 16
        elif kind == "k1":
            o = (n >> 3) * region + q * 256 + (8 * kb + 4 * (1 - kb) + (n & 3)) * 16
        else:
            x = 2 * n + (q & 1)
            if kind == "v_permuted":
                x ^= ((x >> 3) ^ (x >> 4)) & 1
            o = (q >> 1) * region + x * 16
        offs.append(o)
    return offs


def lds_patterns():
    """Named 64-lane offset patterns for `lds_pattern_rates`, in run order."""
    import itertools
    pats = {"linear": [16 * l for l in range(64)],
            "stride256": [256 * (l % 16) + 16 * (l // 16) for l in range(64)]}
    for bits in itertools.combinations(range(6), 4):
        pats["bits" + "".join(map(str, bits))] = _bits_pattern(bits)
    for kind in ("k0", "k1", "v", "v_permuted"):
        pats["prefill_" + kind] = _prefill_pattern(kind)
    for name, offs in pats.items():
        assert len(offs) == 64 and all(0 <= o <= 32768 - 7 * 1024 - 16 and o % 16 == 0 for o in offs), name
    return pats


def lds_pattern_rates(iters=2000, blocks=256):
    """Clocks per ds_read_b128 per wave for each pattern of lds_patterns(), one
    dispatch per pattern in that order (4 waves per CU, all reading the same
    lane pattern).  A conflict-free 128-bit read takes 4 clocks of the CU's LDS
    (16 per read per wave with 4 waves sharing it); each round of 8 reads also
    waits out the LDS latency once, so conflict-free patterns measure above 16."""
    import numpy as np
    lib = _load()
    rows = []
    st = torch.cuda.current_stream()
    for name, offs in lds_patterns().items():
        dev = torch.tensor(offs, dtype=torch.int32, device="cuda")
        out = torch.zeros(blocks * 4 * 2, dtype=torch.int64, device="cuda")
        assert lib.pa_probe_lds_pattern(ctypes.c_void_p(dev.data_ptr()), ctypes.c_void_p(out.data_ptr()),
                                        blocks, iters, ctypes.c_void_p(st.cuda_stream)) == 0
        torch.cuda.synchronize()
        cyc = out.cpu().numpy().reshape(-1, 2)[:, 0].astype(np.float64)
        rows.append({"pattern": name, "clocks_per_read": round(float(np.median(cyc)) / (iters * 8), 2)})
    return rows


def xcd_read_rates(gib=4, chunks=50_000, groups=256, waves=4, reps=12, seed=5):
    """Per-XCD read timing of the read probe: each launch reads `chunks` random
    4 KiB chunks of a `gib` GiB buffer (as many as the 100K-token decode step
    reads), a set disjoint from the previous launches' sets (so no cache holds
    them), split evenly over `groups` workgroups of `waves` waves (one per CU).
    Returns the launches' mean duration and, per XCC id, the mean time (us) from
    a launch's first workgroup start to its workgroups' ends, over all launches
    and for each launch."""
    import numpy as np
    lib = _load()
    nbytes = gib << 30
    nsets = (nbytes // 4096) // chunks
    assert nsets >= reps + 1, "the buffer holds too few disjoint chunk sets"
    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    perm = np.random.default_rng(seed).permutation(nbytes // 4096).astype(np.int32)
    sink = torch.empty(groups * waves * 64, dtype=torch.int32, device="cuda")
    times = torch.zeros(groups * 3, dtype=torch.int64, device="cuda")
    st = torch.cuda.current_stream()
    runs = []
    for r in range(reps + 1):
        ids = torch.from_numpy(perm[r * chunks:(r + 1) * chunks].copy()).cuda()
        assert lib.pa_probe_read_xcd(ctypes.c_void_p(buf.data_ptr()), ctypes.c_void_p(ids.data_ptr()),
                                     chunks, 4096, waves, groups, ctypes.c_void_p(sink.data_ptr()),
                                     ctypes.c_void_p(times.data_ptr()), ctypes.c_void_p(st.cuda_stream)) == 0
        torch.cuda.synchronize()
        if r == 0:
            continue  # warm-up launch
        t = times.cpu().numpy().reshape(groups, 3).astype(np.float64)
        t0 = t[:, 0].min()
        runs.append(((t[:, 1] - t0) / 100.0, t[:, 2].astype(int)))
    xccs = sorted(set(runs[0][1].tolist()))
    per_run = [{int(x): round(float(e[c == x].mean()), 2) for x in xccs} for e, c in runs]
    kernel_us = float(np.mean([e.max() for e, _ in runs]))
    return {"kernel_us": round(kernel_us, 2), "gb_per_s": round(chunks * 4096 / (kernel_us * 1e-6) / 1e9, 1),
            "end_us_mean_by_xcc": {int(x): round(float(np.mean([p[x] for p in per_run])), 2) for x in xccs},
            "end_us_by_xcc_per_launch": per_run}
