"""GPU parity with cache pools larger than 4 GiB: the sequences' blocks are moved
to the top of a 140,000-block pool (4.59 GB per cache), so every byte offset of a
key or value slab they use lies above 2^32.  Each entry point must give the
same bits as on the small pool the blocks came from (only the block ids differ),
and the small-pool results must match the oracle."""
import copy

import numpy as np
import pytest
import torch

import oracle
import split_kv_paged_pa_amd as pa
from parity import DeviceBatch, assert_close, oracle_out, require_gpu, to_f64
from split_kv_paged_pa_amd import workloads as wl

pytestmark = pytest.mark.gpu

BIG_BLOCKS = 140_000  # x Hkv x 16 x D x element size = 4.59 GB at the shapes below


def _to_top(db: DeviceBatch, blocks: int) -> DeviceBatch:
    """The same batch with its pool's blocks at ids [blocks - nb, blocks) of a pool
    of `blocks` blocks (the rest NaN) and the table rewritten to match."""
    nb = db.key_cache.shape[0]
    off = blocks - nb
    big = copy.copy(db)
    big.key_cache = torch.full((blocks,) + tuple(db.key_cache.shape[1:]), float("nan"),
                               dtype=db.key_cache.dtype, device=db.key_cache.device)
    big.value_cache = torch.full((blocks,) + tuple(db.value_cache.shape[1:]), float("nan"),
                                 dtype=db.value_cache.dtype, device=db.value_cache.device)
    big.key_cache[off:] = db.key_cache
    big.value_cache[off:] = db.value_cache
    bt = db.block_tables.clone()
    big.block_tables = torch.where(bt >= 0, bt + off, bt)
    slab = big.key_cache[0].numel() * big.key_cache.element_size()
    used = big.block_tables[big.block_tables >= 0]
    assert int(used.min()) * slab >= 1 << 32, "the moved blocks must sit above 4 GiB"
    return big


def _same_bits(a: torch.Tensor, b: torch.Tensor, what: str):
    assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), f"{what}: large pool differs"


def _free(*dbs):
    for d in dbs:
        d.key_cache = d.value_cache = None
    torch.cuda.empty_cache()


def test_large_pool_bf16_every_entry_point():
    require_gpu()
    spec = wl.custom("bigpool_bf16", 131, "bf16", 64, 8, 128, [3000, 700, 5000, 33])
    b = wl.generate(spec)
    db = DeviceBatch(b)
    big = _to_top(db, BIG_BLOCKS)
    print("[case] large pool bf16", flush=True)
    ref = oracle_out(b)

    small_v1, big_v1 = db.run_v1(), big.run_v1()
    assert_close(to_f64(small_v1), ref, "bf16", "v1")
    _same_bits(small_v1, big_v1, "v1")
    for P in (256, 512):  # P 512: equal spans; P 256: one partition per workgroup
        small, large = db.run_v2(P), big.run_v2(P)
        assert_close(to_f64(small), ref, "bf16", f"v2 P={P}")
        _same_bits(small, large, f"v2 P={P}")
    small_1 = db.new_out()
    pa.pa_decode_v2_single(small_1, *db.args(), 512, db.workspace(512))
    large_1 = big.new_out()
    pa.pa_decode_v2_single(large_1, *big.args(), 512, big.workspace(512))
    assert_close(to_f64(small_1), ref, "bf16", "single launch")
    _same_bits(small_1, large_1, "single launch")

    # Several query tokens per sequence: the decode kernel (q_len 3) and the tiled
    # prefill kernel (q_len 64), both causal over the cache.
    gen = torch.Generator().manual_seed(29)
    _, kc, vc, btn, sln = b.numpy()
    for q_len, fn in ((3, pa.pa_decode_v1_q), (64, None)):
        qf = torch.randn(spec.num_seqs, q_len, spec.num_q_heads, spec.head_dim, generator=gen)
        q = qf.to(torch.bfloat16)
        refq = oracle.decode_q(wl.to_numpy(q), kc, vc, btn, sln, spec.scale, dtype="bf16")
        qd = q.cuda()
        outs = []
        for d in (db, big):
            o = torch.full_like(qd, float("nan"))
            if fn is not None:
                fn(o, qd, d.key_cache, d.value_cache, d.block_tables, d.seq_lens, spec.scale,
                   d.max_seq_len)
            else:
                pa.pa_prefill_v1(o, qd, d.key_cache, d.value_cache, d.block_tables, d.seq_lens,
                                 spec.scale, d.max_seq_len, 2)
            outs.append(o)
        what = "v1_q q_len=3" if fn is not None else "prefill q_len=64"
        assert_close(to_f64(outs[0]), refq, "bf16", what)
        _same_bits(outs[0], outs[1], what)
    _free(db, big)


def test_large_pool_f32():
    require_gpu()
    spec = wl.custom("bigpool_f32", 132, "f32", 8, 4, 128, [2000, 4500])
    b = wl.generate(spec)
    db = DeviceBatch(b)
    big = _to_top(db, BIG_BLOCKS)
    print("[case] large pool f32", flush=True)
    ref = oracle_out(b)
    small_v1, big_v1 = db.run_v1(), big.run_v1()
    assert_close(to_f64(small_v1), ref, "f32", "v1")
    _same_bits(small_v1, big_v1, "v1")
    small, large = db.run_v2(512), big.run_v2(512)
    assert_close(to_f64(small), ref, "f32", "v2 P=512")
    _same_bits(small, large, "v2 P=512")
    _free(db, big)
