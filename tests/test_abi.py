"""The C-ABI library on the CPU: it loads, exports every function the header
declares, and rejects every invalid argument before any HIP call is made.
No call here gets past validation, so nothing touches a GPU."""
import ctypes
import math
import os
import re

import pytest

import split_kv_paged_pa_amd as pa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pa_decode.h")

OK, NULLP, SHAPE, UNSUP, WS, HIP, ARG = range(7)
FAKE = 0x10000  # never dereferenced: each case below fails validation first


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pa_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_function():
    lib = pa.load_library()
    names = declared_functions()
    assert {"pa_decode_v1", "pa_decode_v2", "pa_workspace_size"} <= set(names)
    for n in names:
        assert hasattr(lib, n), f"{n} declared in pa_decode.h but not exported"


def test_timeline_library_exports():
    """The diagnostic build exports everything pa_decode.h declares plus the
    timeline fetch of pa_timeline.h; the product library does not export it."""
    path = os.path.join(ROOT, "split_kv_paged_pa_amd", "libpa_decode_timeline.so")
    if not os.path.exists(path):
        pytest.skip("libpa_decode_timeline.so not built")
    lib = ctypes.CDLL(path)
    text = open(os.path.join(ROOT, "include", "pa_timeline.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    extra = sorted(set(re.findall(r"\b(pa_[a-z0-9_]+)\s*\(", text)))
    assert extra == ["pa_timeline_fetch"]
    for n in declared_functions() + extra:
        assert hasattr(lib, n), f"{n} not exported by libpa_decode_timeline.so"
    assert not hasattr(pa.load_library(), "pa_timeline_fetch")


def test_status_strings():
    for st in range(7):
        assert pa.pa_status_string(st).startswith("PA_")


def test_workspace_size_arithmetic():
    # 100000 tokens, 32 query heads, D 128: 196 partitions of 512, 98 of 1024.
    # Layout: the 16 KiB counter header, then tmp_output, exp_sums, max_logits,
    # each rounded up to 256 bytes.
    def expect(S, Hq, D, L, P):
        n = -(-L // P)
        a = lambda x: -(-x // 256) * 256
        rows = S * Hq * n
        return 16384 + a(rows * D * 4) + 2 * a(rows * 4) if rows else 0
    assert pa.pa_workspace_size(1, 32, 128, 100000, 512) == expect(1, 32, 128, 100000, 512) == 3277824
    assert pa.pa_workspace_size(1, 32, 128, 100000, 1024) == 1647104
    assert pa.pa_workspace_layout(1, 32, 128, 100000, 1024) == (16384, 16384 + 1605632,
                                                               16384 + 1605632 + 12544, 98)
    assert pa.pa_workspace_layout(1, 32, 128, 100000, 512)[3] == 196
    assert pa.pa_workspace_size(16, 32, 128, 32768, 1024) == expect(16, 32, 128, 32768, 1024)
    assert pa.pa_workspace_size(0, 32, 128, 1000, 512) == 0
    assert pa.pa_workspace_size(3, 32, 128, 0, 512) == 0
    assert pa.pa_workspace_size(1, 32, 128, 1000, 24) == 0      # P not a multiple of 16
    assert pa.pa_workspace_size(-1, 32, 128, 1000, 512) == 0


def test_select_v2_threshold():
    assert pa.pa_select_v2(8192, 1, 4, 512) is False
    assert pa.pa_select_v2(8193, 1, 4, 512) is True
    assert pa.pa_select_v2(100000, 1, 4, 1024) is True


def call_v2(lib, **over):
    a = dict(out=FAKE, query=FAKE, key=FAKE, value=FAKE, bt=FAKE, sl=FAKE, S=2, Hq=8, Hkv=2, D=128,
             bs=16, nb=100, mb=64, L=1000, scale=0.088, dtype=1, P=512, ws=FAKE, wsb=1 << 30,
             stream=None)
    a.update(over)
    return lib.pa_decode_v2(a["out"], a["query"], a["key"], a["value"], a["bt"], a["sl"], a["S"],
                            a["Hq"], a["Hkv"], a["D"], a["bs"], a["nb"], a["mb"], a["L"],
                            a["scale"], a["dtype"], a["P"], a["ws"], a["wsb"], a["stream"])


CASES = [
    ("null query", dict(query=None), NULLP),
    ("null out", dict(out=None), NULLP),
    ("null block table", dict(bt=None), NULLP),
    ("null workspace", dict(ws=None), NULLP),
    ("heads not grouped", dict(Hq=9), SHAPE),
    ("negative seqs", dict(S=-1), SHAPE),
    ("max_seq_len beyond table", dict(L=64 * 16 + 1), SHAPE),
    ("group of 32", dict(Hq=64), UNSUP),
    ("head_dim 96", dict(D=96), UNSUP),
    ("block size 32", dict(bs=32), UNSUP),
    ("partition 24", dict(P=24), UNSUP),
    ("partition -16", dict(P=-16), UNSUP),
    ("too many seqs", dict(S=70000), UNSUP),
    ("workspace too small", dict(wsb=1000), WS),
    ("nan scale", dict(scale=math.nan), ARG),
    ("inf scale", dict(scale=math.inf), ARG),
    ("bad dtype", dict(dtype=7), ARG),
    ("misaligned key cache", dict(key=FAKE + 2), ARG),
    ("misaligned workspace", dict(ws=FAKE + 4), ARG),
]


@pytest.mark.parametrize("what,over,status", CASES, ids=[c[0] for c in CASES])
def test_v2_rejects_before_launch(what, over, status):
    assert call_v2(pa.load_library(), **over) == status


def test_v1_and_dispatch_reject_before_launch():
    lib = pa.load_library()
    common = (FAKE, FAKE, FAKE, FAKE, FAKE, 2, 8, 2, 128, 16, 100, 64, 1000, 0.088, 1)
    assert lib.pa_decode_v1(None, *common, None) == NULLP
    bad = (FAKE, FAKE, FAKE, FAKE, FAKE, 2, 8, 3, 128, 16, 100, 64, 1000, 0.088, 1)
    assert lib.pa_decode_v1(FAKE, *bad, None) == SHAPE
    # pa_decode picks V2 above 8192 tokens, which needs the workspace.
    big = (FAKE, FAKE, FAKE, FAKE, FAKE, 2, 8, 2, 128, 16, 100, 1024, 9000, 0.088, 1)
    assert lib.pa_decode(FAKE, *big, 1024, None, 0, None) == WS
    assert lib.pa_decode_v2_reduce(FAKE, FAKE, 2, 8, 128, 9000, 1, 1024, None, 0, None) == WS
    assert lib.pa_decode_v2_reduce(FAKE, FAKE, 2, 8, 96, 9000, 1, 1024, FAKE, 1 << 30, None) == UNSUP


def test_empty_batch_is_a_no_op():
    lib = pa.load_library()
    # num_seqs == 0: valid, nothing to launch, pointers may be NULL.
    assert call_v2(lib, S=0, out=None, query=None, key=None, value=None, bt=None, sl=None,
                   ws=None, wsb=0) == OK


def test_binding_refuses_cpu_tensors():
    import torch
    q = torch.zeros(1, 8, 64)
    kc = torch.zeros(4, 2, 16, 16, 4)
    vc = torch.zeros(4, 2, 64, 16)
    with pytest.raises(ValueError, match="GPU"):
        pa.pa_decode_v1(torch.zeros_like(q), q, kc, vc, torch.zeros(1, 4, dtype=torch.int32),
                        torch.ones(1, dtype=torch.int32), 0.125, 1)


def test_binding_checks_the_split_layout():
    import torch
    q = torch.zeros(1, 8, 64, dtype=torch.bfloat16)
    kc = torch.zeros(4, 2, 16, 16, 4, dtype=torch.bfloat16)  # x = 4 is the float32 grouping
    vc = torch.zeros(4, 2, 64, 16, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="split layout"):
        pa.pa_decode_v1(torch.zeros_like(q), q, kc, vc, torch.zeros(1, 4, dtype=torch.int32),
                        torch.ones(1, dtype=torch.int32), 0.125, 1)
    with pytest.raises(ValueError, match="expected"):
        pa.pa_decode_v1(torch.zeros_like(q), q, vc, vc, torch.zeros(1, 4, dtype=torch.int32),
                        torch.ones(1, dtype=torch.int32), 0.125, 1)


def test_workspace_init_and_launch_count_checks():
    lib = pa.load_library()
    lib.pa_workspace_init.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    assert lib.pa_workspace_init(None, 1 << 20, None) == NULLP
    assert lib.pa_workspace_init(FAKE, 16383, None) == WS
    assert lib.pa_workspace_init(FAKE + 4, 1 << 20, None) == ARG
    # pa_decode_v2_single refuses, before launching, problems the merge cannot take:
    # 625 * 8 = 5000 (sequence, kv head) pairs, more than the 4096 header counters.
    big = (FAKE, FAKE, FAKE, FAKE, FAKE, 625, 64, 8, 128, 16, 100, 2048, 20000, 0.088, 1)
    assert lib.pa_decode_v2_single(FAKE, *big, 1024, FAKE, 1 << 40, None) == UNSUP


def test_partition_size_rule():
    """partition_size = 0: 2048 tokens, or one partition per compute unit when the
    (sequence, kv head) pairs are few (no device here: 256 compute units)."""
    import torch
    if torch.cuda.is_available():
        return  # the rule depends on the device's compute units
    sel = pa.pa_select_partition_size
    assert sel(1, 4, 100000) == 1568          # 4 x ceil(100000 / 1568) = 256 units
    assert 4 * -(-100000 // 1568) == 256 and 4 * -(-100000 // 1552) > 256
    assert sel(16, 8, 32768) == 2048          # 2048 units at 2048 tokens
    assert sel(64, 8, 131072) == 2048
    assert sel(8, 8, 131072) == 2048
    assert sel(1, 8, 65536) == 2048           # exactly 256 units
    assert sel(1, 8, 65535) == 2048
    assert sel(1, 4, 8192) == 256             # 16 units at 2048: floor of 256 tokens
    assert sel(1, 1, 1000) == 256
    assert sel(0, 4, 100) == 2048 and sel(1, 4, 0) == 2048   # invalid: the default
    # The workspace is sized with the chosen value; 0 itself is not a size.
    assert pa.pa_workspace_size(1, 32, 128, 100000, 0) == 0
    lib = pa.load_library()
    args = (FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 32, 4, 128, 16, 8192, 6250, 100000, 0.088, 1)
    need = pa.pa_workspace_size(1, 32, 128, 100000, 1568)
    assert lib.pa_decode_v2(*args, 0, FAKE, need - 1, None) == WS
    assert lib.pa_decode_v2_reduce(FAKE, FAKE, 1, 32, 128, 100000, 1, 0, FAKE, need, None) == UNSUP


def test_noalloc_rejects_before_any_hip_call():
    """The allocation-free entry refuses problems whose workspace exceeds its scratch
    array (and every invalid argument) before touching the device."""
    lib = pa.load_library()
    # (out, query, key, value, block_tables, seq_lens, S, Hq, Hkv, D, block_size,
    #  num_blocks, max_blocks, max_seq_len, scale, dtype, P, stream)
    big = (FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 64, 64, 8, 128, 16, 100, 128, 2048, 0.088, 1)
    assert pa.pa_workspace_size(64, 64, 128, 2048, 16) > pa.api.NOALLOC_SCRATCH_BYTES
    assert lib.pa_decode_v2_noalloc(*big, 16, None) == WS
    assert lib.pa_decode_v2_noalloc(*big[:7], 9, *big[8:], 16, None) == SHAPE   # Hq % Hkv
    assert lib.pa_decode_v2_noalloc(*big, 24, None) == UNSUP                    # P % 16
    assert lib.pa_decode_v2_noalloc(*big[:14], float("nan"), 1, 16, None) == ARG
    assert lib.pa_decode_v2_noalloc(FAKE, None, *big[2:], 16, None) == NULLP


def test_select_v2_auto_rule():
    # Above 8192 tokens: V2, as the pages' rule; at or below 1024: V1, whatever the batch.
    assert pa.pa_select_v2_auto(8193, 256, 8, 1024) is True
    assert pa.pa_select_v2_auto(1024, 1, 1, 1024) is False
    # In between the answer depends on the device's compute units (V2 when the V1 grid
    # would fill less than half of them); without a GPU it falls back to the pages' rule.
    import torch
    if not torch.cuda.is_available():
        assert pa.pa_select_v2_auto(4096, 1, 8, 1024) is False


def test_multi_query_grid_limit():
    lib = pa.load_library()
    # num_kv_heads * ceil(G * q_len / 16) workgroups in grid y: 8 * ceil(8 * 131072 / 16) > 65535.
    args = (FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 131072, 64, 8, 128, 16, 100, 16384, 262144,
            0.088, 1, None)
    assert lib.pa_decode_v1_q(*args) == UNSUP
    assert lib.pa_decode_v1_q(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 0, 64, 8, 128, 16, 100, 16384,
                              262144, 0.088, 1, None) == SHAPE  # q_len 0


def test_prefill_argument_checks():
    lib = pa.load_library()
    # (out, query, key_cache, value_cache, block_tables, seq_lens, S, q_len, Hq, Hkv, D,
    #  block_size, num_blocks, max_blocks, max_seq_len, scale, dtype)
    base = (FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 64, 8, 2, 128, 16, 100, 64, 1024, 0.088)
    f32, bf16 = 0, 1
    assert lib.pa_prefill_v1(*base, f32, 2, None) == UNSUP      # bf16 only
    assert lib.pa_prefill_v1(*base, bf16, 3, None) == ARG       # column tiles 1, 2 or 4 (0: choose)
    assert lib.pa_prefill_v1(*base, bf16, -1, None) == ARG
    assert lib.pa_prefill_v2(*base, f32, 1024, FAKE, 1 << 30, 4, None) == UNSUP
    assert lib.pa_prefill_v2(*base, bf16, 1024, FAKE, 1 << 30, 8, None) == ARG
    assert lib.pa_prefill_v2(*base, bf16, 1024, FAKE, 16, 2, None) == WS
    # The shape checks of the _q entry points apply unchanged.
    assert lib.pa_prefill_v1(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 0, 8, 2, 128, 16, 100, 64, 1024,
                             0.088, bf16, 2, None) == SHAPE


def test_q_kernel_rule():
    """The q_len entry points' kernel choice (no device here: 256 compute units)."""
    import torch
    if torch.cuda.is_available():
        return  # the rule depends on the device's compute units
    bf, f32 = torch.bfloat16, torch.float32
    sel = pa.pa_select_q_kernel
    # S 1, Hq 32, Hkv 4: q_len 512 over 8192 tokens.
    assert sel(1, 1, 512, 32, 4, bf, 8192) == 1       # 1024 single-tile waves = 1 per SIMD
    assert sel(0, 1, 512, 32, 4, bf, 8192, 1024) == 2  # 8 partitions: 4096 two-tile waves
    assert sel(1, 1, 2048, 32, 4, bf, 8192) == 2      # 2048 two-tile waves
    assert sel(1, 1, 128, 32, 4, bf, 4096) == 0       # 256 waves: the decode kernel
    assert sel(0, 1, 8, 32, 4, bf, 8192, 1024) == 0   # 64 columns: the decode kernel
    assert sel(0, 1, 16, 32, 4, bf, 8192, 512) == 1   # 128 columns, 16 partitions
    assert sel(1, 1, 2048, 32, 4, f32, 8192) == 0     # fp32: the decode kernel
    assert sel(1, 1, 1, 32, 4, bf, 8192) == 0         # plain decode
    assert sel(0, 1, 512, 32, 4, bf, 8192, 24) == 0   # invalid partition size


def test_cache_repack_rejects_before_launch():
    """pa_cache_from_token_major: every bad argument is refused on the host."""
    lib = pa.load_library()
    f = lib.pa_cache_from_token_major
    A = 0x100000  # distinct fake buffers, never dereferenced (each call fails validation
    B = 0x200000  # or enqueues nothing)
    C = 0x300000
    D = 0x400000
    ok = (A, B, C, D, 10, 4, 128, 16, 1, None)
    assert f(A, B, C, D, 0, 4, 128, 16, 1, None) == OK           # no blocks: nothing to do
    assert f(A, B, C, D, -1, 4, 128, 16, 1, None) == SHAPE
    assert f(A, B, C, D, 10, 0, 128, 16, 1, None) == SHAPE
    assert f(A, B, C, D, 10, 4, 128, 32, 1, None) == UNSUP       # block size
    assert f(A, B, C, D, 10, 4, 12, 16, 1, None) == UNSUP        # bf16: D a multiple of 8
    assert f(A, B, C, D, 10, 4, 6, 16, 0, None) == UNSUP         # f32: D a multiple of 4
    assert f(A, B, C, D, 10, 4, 1024, 16, 1, None) == UNSUP      # D at most 512
    assert f(A, B, C, D, 10, 4, 128, 16, 5, None) == ARG         # dtype
    assert f(None, None, None, None, *ok[4:]) == NULLP           # nothing to repack
    assert f(A, None, None, D, *ok[4:]) == NULLP                 # key_out without key_in
    assert f(A + 8, B, C, D, *ok[4:]) == ARG                     # misaligned
    assert f(A, B, A + 16, D, *ok[4:]) == ARG                    # key_out overlaps key_in
    assert f(A, B, C, B + 4096, *ok[4:]) == ARG                  # value_out overlaps value_in
    assert f(A, A + 16, C, D, *ok[4:]) == ARG                    # the two outputs overlap
