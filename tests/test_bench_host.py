"""Host-side checks of bench.py (no GPU): the one-GPU contract, the algorithmic
byte count behind the roofline figure, and the source hash that ties the
recorded traffic counters to the kernels they were taken on."""
import importlib.util
import os
import subprocess
import sys

from split_kv_paged_pa_amd import workloads as wl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_bench_refuses_more_than_one_gpu():
    env = {k: v for k, v in os.environ.items() if k not in ("WORLD_SIZE", "RANK", "LOCAL_RANK")}
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""  # no JSON line for a configuration it does not run


def test_phase1_bytes_by_hand():
    """100000 tokens x 4 kv heads x 128 x 2 bytes x (K, V); the bf16 query (32 x 128);
    6250 table entries and one seq_len (int32); the partials, 130 floats per (head,
    partition): 98 partitions at P = 1024, 196 at P = 512."""
    b = _bench()
    spec = wl.config("long_100k_gqa8")
    kv = 100000 * 4 * 128 * 2 * 2
    rest = 32 * 128 * 2 + 6250 * 4 + 4
    assert b.phase1_bytes(spec, 1024) == (kv + rest + 98 * 32 * 130 * 4, kv)
    assert b.phase1_bytes(spec, 512) == (kv + rest + 196 * 32 * 130 * 4, kv)
    assert kv == spec.kv_bytes == 204_800_000
    # Entries of 1568-token spans (Phase 1 in equal spans): 64 entries per row.
    assert b.phase1_bytes(spec, 1024, 1568) == (kv + rest + 64 * 32 * 130 * 4, kv)
    assert b.phase1_bytes(spec, 512, 2048) == (kv + rest + 49 * 32 * 130 * 4, kv)


def test_step_stats():
    b = _bench()
    st = b.step_stats([float(x) for x in range(1, 101)])
    assert st["median"] == 50.5 and st["n"] == 100
    assert abs(st["p10"] - 10.9) < 1e-9 and abs(st["p90"] - 90.1) < 1e-9


def test_bench_starts_no_child_process():
    """bench.py reads clock levels from sysfs files; it must not start a program from
    the GPU process (under a profiler that is an exec of a preloaded process)."""
    src = open(os.path.join(ROOT, "bench.py")).read()
    for word in ("subprocess", "os.system", "popen", "os.exec"):
        assert word not in src.lower(), word


def test_kernel_hash_follows_code_not_comments(tmp_path, monkeypatch):
    b = _bench()
    src = tmp_path / "k.hip"
    monkeypatch.setattr(b, "KERNEL_SRC", [str(src)])
    src.write_text("int f(int x) { return x + 1; }\n")
    h0 = b.kernel_sha()
    src.write_text("// a comment\nint f(int x) {  /* another */ return x + 1; }\n")
    assert b.kernel_sha() == h0
    src.write_text("int f(int x) { return x + 2; }\n")
    assert b.kernel_sha() != h0
