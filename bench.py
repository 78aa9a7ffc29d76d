"""Decode-attention benchmark: one long sequence, 100000 tokens, GQA 8.

A step is one full pass of the hot path over one decode batch: V2 Phase 1
(per-partition attention into the workspace) plus Phase 2 (log-sum-exp merge
into the output), launched through the C ABI on torch's current stream.

    python bench.py [--steps K] [--warmup W] [--partition-size P] [--variant v2|v1]

Workload long_100k_gqa8: 1 sequence x 100000 tokens, 32 query / 4 kv heads,
head_dim 128, bf16, 16-token blocks scattered over an 8192-block pool.  The
204.8 MB of keys and values would fit in MI355X's 256 MB Infinity Cache, so
the cache pool is replicated `--copies` times and step i reads copy i mod
copies: every step streams its keys and values from HBM.  Inputs are resident
in HBM before the timed region starts.

Prints one JSON line:
  - value / ms_per_step: the K timed steps of the headline form (V2 at
    --partition-size), bracketed by torch.cuda.synchronize(), wall clock or HIP
    events, whichever is longer;
  - step_us: median, p10 and p90 of the same form from one event pair per step;
  - variants: the same per-step statistics for V2 at P = 512, at the library's
    partition size (partition_size = 0), and for V1, each with the mean of the
    same number of steps run back to back (back_to_back_mean);
  - roofline: the dominant kernel -- Phase 1 exactly as the step runs it
    (pa_decode_v2_groups) -- timed with HIP events on the launch stream, its
    algorithmic bytes, and the HBM traffic measured by rocprofv3 counters when
    those were taken on the current kernel source (else null);
  - cpu_baseline: the fp64 CPU oracle on a bounded sample.
"""
import argparse
import glob
import hashlib
import json
import os
import re
import sys
import time

# Kernel arguments in device memory: a ROCm runtime setting, read when HIP
# starts (so before torch is imported).  With the default, host-memory
# arguments, the first instruction of every kernel waits on a read across the
# host link; here that is two launches per step (measured on MI355X: the
# 100K-token step 40.7 -> 38.6 us).  A value already in the environment is kept,
# so HIP_FORCE_DEV_KERNARG=0 measures the default.
os.environ.setdefault("HIP_FORCE_DEV_KERNARG", "1")

import numpy as np  # noqa: E402
import torch  # noqa: E402

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import split_kv_paged_pa_amd as pa  # noqa: E402
from split_kv_paged_pa_amd import workloads as wl  # noqa: E402

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0  # dense bf16 matrix peak of MI355X
METRIC = "KV GB/s read and % of HBM peak; decode-attn µs/step at 100K ctx, GQA 8"
# Sources of the decode kernels (the Phase-1 kernel whose traffic profiles/ records).
KERNEL_SRC = [os.path.join(ROOT, "split_kv_paged_pa_amd", "csrc", f)
              for f in ("pa_kernels.hip", "pa_device.h")]
# Sources of the tiled prefill kernel.
PREFILL_SRC = [os.path.join(ROOT, "split_kv_paged_pa_amd", "csrc", f)
               for f in ("pa_prefill.hip", "pa_device.h")]


def kernel_sha(paths=None):
    """Hash of the kernel sources (by default the decode kernels) with comments and
    whitespace removed: it changes with the code, not with its comments."""
    src = ""
    for path in KERNEL_SRC if paths is None else paths:
        with open(path) as f:
            src += f.read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    src = re.sub(r"//[^\n]*", "", src)
    return hashlib.sha256("".join(src.split()).encode()).hexdigest()[:16]


def phase1_bytes(spec, P, entry_tokens=None):
    """Algorithmic bytes of one Phase-1 launch: each K/V row of the actual tokens
    read once (Hkv*D*es*2 per token), the query, the block-table entries used,
    seq_lens, and the workspace entries written (D+2 floats per (seq, head,
    entry); an entry covers entry_tokens tokens, by default one partition)."""
    es = spec.elem_size
    lens = spec.seq_lens.astype(np.int64)
    entries = int(np.sum(-(-lens // (entry_tokens or P))))
    kv = int(lens.sum()) * spec.num_kv_heads * spec.head_dim * es * 2
    q = spec.num_seqs * spec.num_q_heads * spec.head_dim * es
    tables = int(np.sum(-(-lens // 16))) * 4 + spec.num_seqs * 4
    partials = entries * spec.num_q_heads * (spec.head_dim + 2) * 4
    return kv + q + tables + partials, kv


def step_stats(us):
    """Median, p10 and p90 of per-step microseconds."""
    return {"median": round(float(np.median(us)), 2), "p10": round(float(np.percentile(us, 10)), 2),
            "p90": round(float(np.percentile(us, 90)), 2), "n": len(us)}


def time_per_step(run, n, stream):
    """One event pair per step, n steps back to back: microseconds of each step
    (the pair's own overhead included)."""
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
    torch.cuda.synchronize()
    for i in range(n):
        ev[i].record(stream)
        run(i)
    ev[n].record(stream)
    torch.cuda.synchronize()
    return [ev[i].elapsed_time(ev[i + 1]) * 1e3 for i in range(n)]


def prefill_extra(dev, stream, dtype, kc, vc, bt, spec, S, Hq, D, q_len=2048, L=8192):
    """q_len query tokens per sequence over the first L tokens of the workload's
    cache through pa_decode_v1_q (which takes the tiled prefill kernel at this
    size): microseconds per call and MFMA throughput, 4 * D flops per visible
    (query token, head, cache token).

    The first calls after other work run slower: on MI355X this kernel took ~300 us
    per call over its first 50 calls after an idle spell and ~221 us per call from
    then on (sysfs showed the board power climbing from ~0.3 to ~1 kW meanwhile,
    under its 1.4 kW cap).  So `us` is the mean of 50 calls after 100 untimed ones;
    `us_after_3` keeps the mean of the 10 calls that follow the first 3."""
    qp = torch.randn(S, q_len, Hq, D, device=dev).to(dtype)
    op = torch.empty_like(qp)
    slp = torch.full((S,), L, dtype=torch.int32, device=dev)

    def run():
        pa.pa_decode_v1_q(op, qp, kc, vc, bt, slp, spec.scale, L)

    def timed(n):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(n):
            run()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / n
    for _ in range(3):
        run()
    us_short = timed(10)
    for _ in range(100 - 13):
        run()
    us = timed(50)
    pairs = S * Hq * sum(L - q_len + j + 1 for j in range(q_len))
    tflops = 4.0 * D * pairs / (us * 1e-6) / 1e12
    tiles = pa.pa_select_q_kernel(1, S, q_len, Hq, spec.num_kv_heads, dtype, L)
    return {"us": round(us, 1), "tflops": round(tflops, 1), "peak_tflops": MFMA_BF16_PEAK_TFLOPS,
            "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4), "us_after_3": round(us_short, 1),
            "calls": "100 untimed, then 50 timed",
            "kernel": f"prefill_kernel<128,{tiles},single pass>" if tiles else "attend_kernel",
            "kernel_sha": kernel_sha(PREFILL_SRC)}


def load_traffic(workload, P):
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}_p{P}.txt")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_sha") != kernel_sha():
        return None
    return t


def cpu_baseline(batch, budget_s):
    import oracle
    threads = len(os.sched_getaffinity(0))
    q, kc, vc, bt, sl = batch.numpy()
    spec = batch.spec
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.decode(q, kc, vc, bt, sl, spec.scale, dtype=spec.dtype, threads=threads)
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s or reps >= 2000:
            break
    return {"value": round(spec.kv_bytes * reps / el / 1e9, 3), "unit": "GB/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{reps} full step(s) of {spec.name} (all {spec.num_q_heads} heads, "
                      f"{int(spec.seq_lens.sum())} tokens) in fp64 C, {el:.1f} s"}


def device_info():
    """Name, ISA, compute units, and the current shader and memory clock levels
    from the amdgpu driver's sysfs files when they are readable (no child
    process is started from this GPU process)."""
    p = torch.cuda.get_device_properties(0)
    info = {"name": p.name, "arch": getattr(p, "gcnArchName", None),
            "compute_units": p.multi_processor_count, "clocks": None}
    clocks = {}
    for path in sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_[sm]clk")):
        try:
            with open(path) as f:
                cur = [ln.strip() for ln in f if ln.rstrip().endswith("*")]
        except OSError:
            continue
        if cur:
            card = path.split("/")[4]
            clocks[f"{card}.{os.path.basename(path)[7:]}"] = cur[0]
    info["clocks"] = clocks or None
    return info


def hbm_probe(dev):
    """Achievable HBM read bandwidth (GB/s) for streaming and for random 4 KiB chunks,
    measured with libpa_probe.so (16-byte non-temporal loads, no arithmetic): the
    ceiling Phase 1 can approach.  'random' reads 300000 chunks (1.2 GB) drawn from
    a 4 GiB buffer per launch, so the 256 MB Infinity Cache cannot hold them, with
    1 KiB contiguous per load instruction (the decode kernels' shape for keys);
    'rows16x64' reads the same chunks 64 bytes of each of 16 rows per instruction
    (a token-major block layout)."""
    from split_kv_paged_pa_amd import probe
    buf = torch.zeros(4 << 30, dtype=torch.uint8, device=dev)
    ids = torch.randperm((4 << 30) // 4096, generator=torch.Generator().manual_seed(0))
    ids = ids[:300000].to(torch.int32).to(dev)
    res = {"sequential_4GiB": round(probe.read_bandwidth(buf, None, 4096, 4, 1024, reps=5), 1)}
    for groups in (196, 392):
        res[f"random_4KiB_{groups}wg"] = round(
            probe.read_bandwidth(buf, ids, 4096, 4, groups, reps=5, shape=0), 1)
        res[f"random_4KiB_{groups}wg_rows16x64"] = round(
            probe.read_bandwidth(buf, ids, 4096, 4, groups, reps=5, shape=1), 1)
    del buf, ids
    torch.cuda.empty_cache()
    return {"unit": "GB/s", **res}


def timeline(dev, args):
    """Per-workgroup timeline of K back-to-back V2 steps from the diagnostic build
    libpa_decode_timeline.so (the same kernels with start / mid / end stamps on the
    100 MHz constant clock, csrc/pa_timeline.h).  Prints one JSON object: per launch
    (then the median over launches), in us from the first Phase-1 workgroup's
    start: the spread of Phase-1 starts, Phase-1 wave-0 streaming ends (median,
    p90, last), the close (end - streaming end, median), the last Phase-1 end,
    Phase 2's first start, its partials' arrival (median, last) and its last
    end, and the next step's first Phase-1 start; then the mean streaming end of
    the workgroups on each XCD and the spread of each workgroup's end from launch
    to launch.  The Phase-2 record's atomic adds one round trip to the end of
    Phase 2, so the last interval and the step time run longer than in the
    product library."""
    import ctypes
    from split_kv_paged_pa_amd import api
    path = os.path.join(ROOT, "split_kv_paged_pa_amd", "libpa_decode_timeline.so")
    if not os.path.exists(path):
        raise SystemExit(f"{path} is missing: python split_kv_paged_pa_amd/build.py")
    api._lib = None
    api.LIB_PATH = path
    lib = api.load_library()
    lib.pa_timeline_fetch.restype = ctypes.c_int
    lib.pa_timeline_fetch.argtypes = [ctypes.c_void_p, ctypes.c_int]
    spec = wl.config(args.workload)
    batch = wl.generate(spec)
    S, Hq, D, L = spec.num_seqs, spec.num_q_heads, spec.head_dim, spec.max_seq_len
    P = args.partition_size or pa.pa_select_partition_size(S, spec.num_kv_heads, L)
    q, bt, sl = batch.query.to(dev), batch.block_tables.to(dev), batch.seq_lens.to(dev)
    kcs, vcs = [batch.key_cache.to(dev)], [batch.value_cache.to(dev)]
    for _ in range(args.copies - 1):
        kcs.append(kcs[0].clone())
        vcs.append(vcs[0].clone())
    out, stream = torch.empty_like(q), torch.cuda.current_stream()
    ws = pa.new_workspace(S, Hq, D, L, P, device=dev)
    calls = [pa.bind_decode_v2(out, q, kcs[c], vcs[c], bt, sl, spec.scale, L, P, ws, stream)
             for c in range(len(kcs))]
    n_rec = 1 << 18
    buf = np.zeros((n_rec, 4), np.uint64)
    for i in range(10):
        calls[i % len(calls)]()
    assert lib.pa_timeline_fetch(None, 0) >= 0  # clear
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(args.timeline):
        calls[i % len(calls)]()
    e1.record(stream)
    torch.cuda.synchronize()
    n = lib.pa_timeline_fetch(buf.ctypes.data, n_rec)
    assert 0 <= n <= n_rec, f"timeline fetch failed or overflowed: {n}"
    r = buf[:n].astype(np.int64)
    r = r[(r[:, 0] & 15) != 0]  # holes: workgroups that had no work
    kind, xcc, lin = r[:, 0] & 15, (r[:, 0] >> 4) & 15, (r[:, 0] >> 8) & 0xffffff
    t = r[:, 1:4] / 100.0  # 10 ns ticks -> us
    runs, a = [], 0  # consecutive records of one kind: one launch
    for i in range(1, len(r) + 1):
        if i == len(r) or kind[i] != kind[a]:
            runs.append((int(kind[a]), a, i))
            a = i
    p1 = [x for x in runs if x[0] == 1]
    p2 = [x for x in runs if x[0] == 2]
    rows, ends = [], []
    for k in range(min(len(p1), len(p2)) - 1):
        _, a1, b1 = p1[k]
        _, a2, b2 = p2[k]
        T0 = t[a1:b1, 0].min()
        s1, s2 = t[a1:b1] - T0, t[a2:b2] - T0
        rows.append([s1[:, 0].max(), np.median(s1[:, 1]), np.percentile(s1[:, 1], 90), s1[:, 1].max(),
                     np.median(s1[:, 2] - s1[:, 1]), s1[:, 2].max(), s2[:, 0].min(),
                     np.median(s2[:, 1]), s2[:, 1].max(), s2[:, 2].max(),
                     t[p1[k + 1][1]:p1[k + 1][2], 0].min() - T0])
        o = np.argsort(lin[a1:b1])
        ends.append(((t[a1:b1, 1] - T0)[o], xcc[a1:b1][o]))
    names = ["p1_start_spread", "p1_stream_end_median", "p1_stream_end_p90", "p1_stream_end_last",
             "p1_close_median", "p1_end_last", "p2_first_start", "p2_partials_median",
             "p2_partials_last", "p2_end_last", "next_p1_start"]
    R = np.array(rows)
    res = {nm: round(float(np.median(R[:, j])), 2) for j, nm in enumerate(names)}
    same = len({len(e[0]) for e in ends}) == 1
    if same and ends:
        E = np.array([e[0] for e in ends])
        X = ends[0][1]
        res["stream_end_mean_by_xcc"] = {int(x): round(float(E[:, X == x].mean()), 2)
                                         for x in np.unique(X)}
        resid = E - np.median(E, 1, keepdims=True)
        res["workgroup_end_spread_std"] = round(float((resid - resid.mean(0)).std()), 2)
    print(json.dumps({"timeline": res, "workload": spec.name, "partition_size": P,
                      "launches": len(rows), "phase1_workgroups": int(p1[0][2] - p1[0][1]),
                      "phase2_workgroups": int(p2[0][2] - p2[0][1]) if p2 else 0,
                      "us_per_step_back_to_back": round(e0.elapsed_time(e1) * 1e3 / args.timeline, 2),
                      "note": "diagnostic build (libpa_decode_timeline.so); us from the first "
                              "Phase-1 workgroup's start, medians over launches"}), flush=True)


DISPATCH_GRID = [(1, 1), (1, 8), (4, 8), (16, 8), (64, 8), (256, 8)]
DISPATCH_LENS = [512, 1024, 2048, 4096, 8192, 16384]


def dispatch_sweep(dev):
    """V1 against V2 (P = 512, 1024, and the library's choice) and the two dispatch
    rules, over uniform-length bf16 batches (Hq = 8 Hkv, D = 128, random block
    tables, random values).  Prints one JSON object with a row per (S, Hkv, L):
    the measured us per call of each form, the partition size the library picks,
    and the us of the form pa_select_v2 (the pages' rule) and pa_select_v2_auto
    (the MI355X rule) pick."""
    G, D = 8, 128
    st = torch.cuda.current_stream()
    rows = []
    for S, Hkv in DISPATCH_GRID:
        for L in DISPATCH_LENS:
            nblk = -(-L // 16)
            NB = S * nblk
            Hq = Hkv * G
            gen = torch.Generator(device=dev).manual_seed(S * 100003 + L)
            q = torch.randn(S, Hq, D, device=dev, generator=gen).to(torch.bfloat16)
            kc = torch.randn(NB, Hkv, D // 8, 16, 8, device=dev, generator=gen).to(torch.bfloat16)
            vc = torch.randn(NB, Hkv, D, 16, device=dev, generator=gen).to(torch.bfloat16)
            bt = torch.randperm(NB, device=dev, generator=gen).to(torch.int32).view(S, nblk)
            sl = torch.full((S,), L, dtype=torch.int32, device=dev)
            out = torch.empty_like(q)
            p_auto = pa.pa_select_partition_size(S, Hkv, L)
            row = {"S": S, "Hkv": Hkv, "L": L, "auto_partition_size": p_auto}
            for name, P in (("v1", None), ("v2_p512", 512), ("v2_p1024", 1024), ("v2_auto", 0)):
                ws = None if P is None else pa.new_workspace(S, Hq, D, L, P or p_auto, device=dev)

                def run():
                    if P is None:
                        pa.pa_decode_v1(out, q, kc, vc, bt, sl, 0.088, L)
                    else:
                        pa.pa_decode_v2(out, q, kc, vc, bt, sl, 0.088, L, P, ws)
                for _ in range(3):
                    run()
                torch.cuda.synchronize()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(st)
                for _ in range(20):
                    run()
                e1.record(st)
                torch.cuda.synchronize()
                row[name] = round(e0.elapsed_time(e1) * 1e3 / 20, 2)
            row["pages_rule_us"] = row["v2_p1024"] if pa.pa_select_v2(L, S, Hkv, 1024) else row["v1"]
            row["auto_rule_us"] = row["v2_auto"] if pa.pa_select_v2_auto(L, S, Hkv, 0) else row["v1"]
            print(f"[sweep] {row}", file=sys.stderr, flush=True)
            rows.append(row)
            del q, kc, vc, bt, sl, out
            torch.cuda.empty_cache()
    print(json.dumps({"dispatch_sweep": rows, "device": torch.cuda.get_device_name(0),
                      "compute_units": torch.cuda.get_device_properties(0).multi_processor_count,
                      "note": "us per call from HIP events over 20 back-to-back calls; calls under "
                              "~15 us are bound by the Python launch path, not the GPU"}),
          flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="long_100k_gqa8")
    ap.add_argument("--partition-size", type=int, default=1024,
                    help="partition size of the headline form (0: the library's choice)")
    ap.add_argument("--variant", choices=["v2", "v1"], default="v2")
    ap.add_argument("--copies", type=int, default=6)
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-probe", action="store_true", help="skip the HBM read-ceiling probe")
    ap.add_argument("--rates", action="store_true",
                    help="print the instruction-rate probe (libpa_probe.so) as JSON and exit")
    ap.add_argument("--lds-banks", action="store_true",
                    help="print the LDS read-pattern probe (libpa_probe.so) as JSON and exit: "
                         "one dispatch per lane pattern, in the printed order")
    ap.add_argument("--xcd-probe", action="store_true",
                    help="print the per-XCD read timing of the HBM probe (libpa_probe.so) as JSON "
                         "and exit")
    ap.add_argument("--no-variants", action="store_true",
                    help="skip the other partition sizes and V1 (for short profiling passes)")
    ap.add_argument("--extras", action="store_true",
                    help="also time V2 in a single launch, V2 with several query tokens per "
                         "sequence, and the tiled prefill kernel (same cache)")
    ap.add_argument("--timeline", type=int, default=0, metavar="K",
                    help="instead of the step benchmark, run K steps on the diagnostic timeline "
                         "build and print the per-workgroup timeline summary")
    ap.add_argument("--dispatch-sweep", action="store_true",
                    help="instead of the step benchmark, time V1 / V2 over a grid of batch shapes "
                         "and compare the two dispatch rules")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (the op shards by "
              "sequence, kv head or context with no change to the kernels)",
              file=sys.stderr)
        sys.exit(2)
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.rates:
        from split_kv_paged_pa_amd import probe
        print(json.dumps({"instruction_rates": probe.issue_rates(),
                          "device": torch.cuda.get_device_name(dev)}))
        return
    if args.xcd_probe:
        from split_kv_paged_pa_amd import probe
        print(json.dumps({"xcd_read": probe.xcd_read_rates(),
                          "device": torch.cuda.get_device_name(dev)}))
        return
    if args.lds_banks:
        from split_kv_paged_pa_amd import probe
        print(json.dumps({"lds_pattern_clocks": probe.lds_pattern_rates(),
                          "device": torch.cuda.get_device_name(dev)}))
        return

    if args.dispatch_sweep:
        dispatch_sweep(dev)
        return
    if args.timeline:
        timeline(dev, args)
        return
    spec = wl.config(args.workload)
    batch = wl.generate(spec)
    S, Hq, Hkv, D = spec.num_seqs, spec.num_q_heads, spec.num_kv_heads, spec.head_dim
    L = spec.max_seq_len
    P_auto = pa.pa_select_partition_size(S, Hkv, L)
    P = args.partition_size or P_auto
    q = batch.query.to(dev)
    bt = batch.block_tables.to(dev)
    sl = batch.seq_lens.to(dev)
    kcs = [batch.key_cache.to(dev)]
    vcs = [batch.value_cache.to(dev)]
    for _ in range(args.copies - 1):
        kcs.append(kcs[0].clone())
        vcs.append(vcs[0].clone())
    out = torch.empty_like(q)
    stream = torch.cuda.current_stream()
    workspaces = {}

    def workspace(part):
        if part not in workspaces:
            workspaces[part] = pa.new_workspace(S, Hq, D, L, part or P_auto, device=dev)
        return workspaces[part]

    def v2_calls(part):
        """One pre-marshalled pa_decode_v2 per cache copy (partition_size part, 0 =
        the library's choice)."""
        return [pa.bind_decode_v2(out, q, kcs[c], vcs[c], bt, sl, spec.scale, L, part,
                                  workspace(part), stream) for c in range(len(kcs))]

    def v1_step(i):
        c = i % len(kcs)
        pa.pa_decode_v1(out, q, kcs[c], vcs[c], bt, sl, spec.scale, L)

    head = v2_calls(args.partition_size)

    def step(i):
        if args.variant == "v2":
            head[i % len(head)]()
        else:
            v1_step(i)

    # Parity of every timed form on sampled rows, before any timing.
    import oracle
    rows = np.array([(s, h) for s in range(S) for h in range(0, Hq, max(1, Hq // 8))], np.int32)
    ref = oracle.decode(*batch.numpy(), spec.scale, dtype=spec.dtype, rows=rows)
    forms = [("headline", step)]
    if not args.no_variants:
        forms += [("v2_p512", lambda i, c=v2_calls(512): c[i % len(c)]()),
                  ("v2_auto", lambda i, c=v2_calls(0): c[i % len(c)]()), ("v1", v1_step)]
    for name, run in forms:
        out.fill_(float("nan"))
        run(0)
        torch.cuda.synchronize()
        got = out.double().cpu().numpy()[rows[:, 0], rows[:, 1]]
        err = np.abs(got - ref)
        assert np.all(err <= 2e-2 + 1e-2 * np.abs(ref)), f"bench parity failed ({name}): {err.max()}"
        print(f"[bench] parity {name} on {len(rows)} rows: max abs err {err.max():.3e}",
              file=sys.stderr, flush=True)

    # Calibration copy for the HBM counters: a plain 768 MiB device-to-device copy
    # (a size no other copy here has, so its dispatches are easy to pick out).
    cal_src = torch.empty(768 << 20, dtype=torch.uint8, device=dev)
    cal_dst = torch.empty_like(cal_src)
    for _ in range(3):
        cal_dst.copy_(cal_src)
    del cal_src, cal_dst

    # Per-step statistics of the headline form, then of the other forms: untimed
    # for the headline, and run before it, so that the headline's warmup and timed
    # steps start on a GPU that has been streaming (clocks up) rather than idle
    # after the parity checks.
    n_steps = max(20, min(args.steps, 100))
    step_us = step_stats(time_per_step(step, n_steps, stream))

    def form_line(run, n):
        """Per-step statistics of one form (an event pair per step, so each step
        also carries the pair's own overhead), then the mean of n steps run back
        to back between one event pair, as the headline value is taken.  A V2 form
        first runs 100 untimed steps: after V1, which leaves most of the GPU idle,
        the step takes ~60 steps to come back to its steady time (measured on
        MI355X: 38.7 us per step over the first 20, 36.6-36.8 us from the 60th)."""
        for i in range(100 if n > 5 else 1):
            run(i)
        st = step_stats(time_per_step(run, n, stream))
        st["gb_per_s"] = round(spec.kv_bytes / (st["median"] * 1e-6) / 1e9, 1)
        st["hbm_peak_frac"] = round(st["gb_per_s"] / HBM_PEAK_GBS, 4)
        b0, b1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        b0.record(stream)
        for i in range(n):
            run(i)
        b1.record(stream)
        torch.cuda.synchronize()
        st["back_to_back_mean"] = round(b0.elapsed_time(b1) * 1e3 / n, 2)
        st["back_to_back_gb_per_s"] = round(spec.kv_bytes / (st["back_to_back_mean"] * 1e-6) / 1e9, 1)
        return st
    variants = {}
    if not args.no_variants:
        # V1 first: it keeps most of the GPU idle (one workgroup per kv head), and
        # the headline follows the V2 forms, not an idle stretch.
        variants["v1"] = form_line(v1_step, 5)
        variants["v2_p512"] = dict(form_line(forms[1][1], n_steps), partition_size=512)
        variants["v2_auto"] = dict(form_line(forms[2][1], n_steps), partition_size=P_auto)
        for k, v in variants.items():
            print(f"[bench] {k}: median {v['median']} us (p10 {v['p10']}, p90 {v['p90']}), "
                  f"back to back {v['back_to_back_mean']} us", file=sys.stderr, flush=True)

    # The timed region: K steps between synchronisations.
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for i in range(args.steps):
        step(args.warmup + i)
    ev1.record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_wall = (t1 - t0) * 1e3 / args.steps
    ms_event = ev0.elapsed_time(ev1) / args.steps
    ms_per_step = max(ms_wall, ms_event)
    value = spec.kv_bytes / (ms_per_step * 1e-3) / 1e9
    print(f"[bench] {args.variant} P={P}: {ms_per_step * 1e3:.2f} us/step "
          f"(wall {ms_wall * 1e3:.2f}, events {ms_event * 1e3:.2f}), {value:.1f} GB/s",
          file=sys.stderr, flush=True)

    # Dominant kernel alone: V2 Phase 1 exactly as the step runs it.  An event pair
    # around n1 back-to-back launches gives the mean duration; one pair per launch
    # gives the spread.
    wsh = workspace(args.partition_size)
    entry_tokens = P

    def phase1(i):
        nonlocal entry_tokens
        c = i % len(kcs)
        entry_tokens = pa.pa_decode_v2_groups(q, kcs[c], vcs[c], bt, sl, spec.scale, L, P, wsh)
    n1 = max(20, min(args.steps, 100))
    for i in range(5):
        phase1(i)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for i in range(n1):
        phase1(i)
    e1.record(stream)
    torch.cuda.synchronize()
    p1_us = e0.elapsed_time(e1) * 1e3 / n1
    durs = time_per_step(phase1, n1, stream)  # includes per-pair event overhead
    alg_bytes, kv_bytes = phase1_bytes(spec, P, entry_tokens)
    achieved = alg_bytes / (p1_us * 1e-6) / 1e9
    traffic = load_traffic(args.workload, P)
    mode = f"entries of {entry_tokens} tokens"
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": None if traffic is None else traffic["bytes_per_launch"],
                "kernel": f"attend_kernel<bf16,128,4,2> (V2 Phase 1 as pa_decode_v2 runs it, {mode})",
                "launch_us_mean": round(p1_us, 2),
                "launch_us_p10_p90_single": [round(float(np.percentile(durs, 10)), 2),
                                             round(float(np.percentile(durs, 90)), 2)],
                "algorithmic_bytes_per_launch": alg_bytes}

    extras = {}
    if args.extras and args.variant == "v2":
        ws1 = pa.new_workspace(S, Hq, D, L, P, device=dev)

        def single(i):
            c = i % len(kcs)
            pa.pa_decode_v2_single(out, q, kcs[c], vcs[c], bt, sl, spec.scale, L, P, ws1)
        try:
            extras[f"v2_single_launch_p{P}_us_per_step"] = form_line(single, 50)["median"]
        except pa.PagedAttentionError as e:
            extras[f"v2_single_launch_p{P}_us_per_step"] = f"not applicable: {e}"
        # Several query tokens per sequence (causal over the cache): as many as fit the
        # 16 tile columns with this GQA group.
        qlen = max(1, 16 // (Hq // Hkv))
        if qlen > 1:
            qm = torch.randn(S, qlen, Hq, D, device=dev).to(q.dtype)
            om = torch.empty_like(qm)
            wsq = pa.new_workspace(S, qlen * Hq, D, L, P, device=dev)

            def multi(i):
                c = i % len(kcs)
                pa.pa_decode_v2_q(om, qm, kcs[c], vcs[c], bt, sl, spec.scale, L, P, wsq)
            extras[f"v2_qlen{qlen}_p{P}_us_per_step"] = form_line(multi, 50)["median"]
        extras["prefill_q2048_L8192"] = prefill_extra(dev, stream, q.dtype, kcs[0], vcs[0], bt,
                                                      spec, S, Hq, D)

    probe = None if args.no_probe else hbm_probe(dev)

    cpu = None if args.no_cpu_baseline else cpu_baseline(batch, args.cpu_seconds)

    line = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
        "us_per_step": round(ms_per_step * 1e3, 2), "hbm_peak_frac": round(value / HBM_PEAK_GBS, 4),
        # The two clocks of the timed region (ms_per_step is the larger): the wall
        # clock carries a fixed ~16 us of first launch into an idle queue and
        # completion signalling per timed run, ~0.8 us per step at K = 20.
        "us_per_step_wall": round(ms_wall * 1e3, 2), "us_per_step_events": round(ms_event * 1e3, 2),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": spec.dtype,
        "data": f"synthetic (seeded N(0,1) {spec.dtype} keys/values/query, random block permutation)",
        "config": {"workload": spec.name, "num_seqs": S, "seq_len": int(spec.seq_lens.max()),
                   "total_tokens": int(spec.seq_lens.sum()),
                   "q_heads": Hq, "kv_heads": Hkv, "head_dim": D, "block_size": 16,
                   "partition_size": P, "variant": args.variant, "kv_copies": len(kcs),
                   "kv_bytes_per_step": spec.kv_bytes},
        "step_us": step_us,
        "variants": variants,
        # Phase 2 and the gap between the launches, as the step sees them.
        "phase2_us_in_step": round(ms_per_step * 1e3 - p1_us, 2),
        "roofline": roofline,
        "cpu_baseline": cpu,
        "hbm_probe": probe,
        "extras": extras,
        "device": torch.cuda.get_device_name(0),
        "device_info": device_info(),
        "runtime_env": {"HIP_FORCE_DEV_KERNARG": os.environ.get("HIP_FORCE_DEV_KERNARG")},
        "kernel_sha": kernel_sha(),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
