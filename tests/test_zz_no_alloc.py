"""The allocation-free entry point (pa_decode_v2_noalloc) against pa_decode_v2:
two calls in a row on the library's per-device scratch array, the second with a
smaller input, each equal bit for bit to pa_decode_v2 with a caller workspace
and within the bf16 tolerance of the oracle."""
import numpy as np
import pytest
import torch

import split_kv_paged_pa_amd as pa
from parity import DeviceBatch, assert_close, oracle_out, require_gpu, to_f64
from split_kv_paged_pa_amd import workloads as wl

pytestmark = pytest.mark.gpu


def test_noalloc_two_calls_match_v2():
    require_gpu()
    cases = [
        # one long sequence, several partitions per Phase-1 workgroup (grouped entries)
        (wl.custom("noalloc_big", 140, "bf16", 32, 4, 128, [40000]), 512),
        # a smaller ragged batch afterwards, zero length included: one entry per partition
        (wl.custom("noalloc_small", 141, "bf16", 16, 2, 128, [3000, 0, 517, 64]), 256),
    ]
    sizes = []
    for spec, P in cases:
        b = wl.generate(spec)
        db = DeviceBatch(b)
        sizes.append(pa.pa_workspace_size(spec.num_seqs, spec.num_q_heads, spec.head_dim,
                                          db.max_seq_len, P))
        print(f"[case] noalloc {spec.name} P={P} workspace {sizes[-1]} B", flush=True)
        assert sizes[-1] <= pa.api.NOALLOC_SCRATCH_BYTES
        ref = db.run_v2(P)
        out = db.new_out()
        pa.pa_decode_v2_noalloc(out, *db.args(), P)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), spec.name
        assert_close(to_f64(out), oracle_out(b), "bf16", f"noalloc {spec.name}")
    assert sizes[1] < sizes[0]


def test_noalloc_refuses_oversized_problem():
    require_gpu()
    spec = wl.custom("noalloc_tiny", 142, "bf16", 8, 2, 64, [100])
    db = DeviceBatch(wl.generate(spec))
    # 64 sequences x 64 heads x 128 partitions of 16 tokens x 130 floats > 64 MiB
    q = torch.zeros(64, 64, 128, dtype=torch.bfloat16, device="cuda")
    kc = torch.zeros(16, 8, 16, 16, 8, dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros(16, 8, 128, 16, dtype=torch.bfloat16, device="cuda")
    bt = torch.zeros(64, 128, dtype=torch.int32, device="cuda")
    sl = torch.full((64,), 2048, dtype=torch.int32, device="cuda")
    out = torch.empty_like(q)
    with pytest.raises(pa.PagedAttentionError) as e:
        pa.pa_decode_v2_noalloc(out, q, kc, vc, bt, sl, 0.088, 2048, 16)
    assert e.value.status == 4  # PA_ERR_WORKSPACE_TOO_SMALL
    # The library still works afterwards.
    ref = db.run_v2(16)
    out = db.new_out()
    pa.pa_decode_v2_noalloc(out, *db.args(), 16)
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
