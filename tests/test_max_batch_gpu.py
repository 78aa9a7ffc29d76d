"""GPU parity at the largest batch the library takes: num_seqs = 65535 (the grid's
z limit), short ragged sequences (1 to 40 tokens, so one to three blocks each and
some partial blocks), through V1, V2 at a partition size that gives several
partitions per row, and two query tokens per sequence."""
import numpy as np
import pytest
import torch

import oracle
import split_kv_paged_pa_amd as pa
from parity import DeviceBatch, assert_close, oracle_out, require_gpu, to_f64
from split_kv_paged_pa_amd import workloads as wl

pytestmark = pytest.mark.gpu

MAX_SEQS = 65535


def test_max_num_seqs():
    require_gpu()
    lens = np.random.default_rng(141).integers(1, 41, MAX_SEQS)
    spec = wl.custom("max_seqs", 141, "bf16", 8, 2, 64, lens.tolist())
    b = wl.generate(spec)
    db = DeviceBatch(b)
    print(f"[case] num_seqs {MAX_SEQS}", flush=True)
    ref = oracle_out(b)
    assert_close(to_f64(db.run_v1()), ref, "bf16", "v1")
    assert_close(to_f64(db.run_v2(16)), ref, "bf16", "v2 P=16")
    _, kc, vc, bt, sl = b.numpy()
    q = torch.randn(MAX_SEQS, 2, spec.num_q_heads, spec.head_dim,
                    generator=torch.Generator().manual_seed(142)).to(torch.bfloat16)
    refq = oracle.decode_q(wl.to_numpy(q), kc, vc, bt, sl, spec.scale, dtype="bf16")
    out = torch.full_like(q.cuda(), float("nan"))
    pa.pa_decode_v1_q(out, q.cuda(), db.key_cache, db.value_cache, db.block_tables, db.seq_lens,
                      spec.scale, db.max_seq_len)
    assert_close(to_f64(out), refq, "bf16", "v1_q q_len=2")
