"""Seeded input generator: determinism, shapes and the config recipe."""
import numpy as np
import torch

from split_kv_paged_pa_amd import workloads as wl


def test_same_seed_same_bytes_any_thread_count():
    spec = wl.custom("det", 5, "bf16", 8, 2, 64, [300, 17, 1000], outlier_frac=0.01,
                     outlier_mult=20.0)
    a = wl.generate(spec, threads=1)
    b = wl.generate(spec, threads=7)
    for x, y in zip(a.numpy(), b.numpy()):
        assert np.array_equal(x.view(np.uint8), y.view(np.uint8))


def test_poison_layout():
    spec = wl.custom("poison", 6, "f32", 4, 2, 64, [33, 16, 1], num_blocks=12)
    b = wl.generate(spec)
    q, kc, vc, bt, sl = b.numpy_logical()
    used = set()
    for s, L in enumerate(sl):
        nblk = -(-int(L) // 16)
        assert np.all(bt[s, nblk:] == -1)
        for j in range(nblk):
            blk = bt[s, j]
            used.add(int(blk))
            valid = min(16, int(L) - 16 * j)
            assert np.all(np.isfinite(kc[blk, :, :valid])) and np.all(np.isfinite(vc[blk, :, :valid]))
            assert np.all(np.isnan(kc[blk, :, valid:])) and np.all(np.isnan(vc[blk, :, valid:]))
    for blk in set(range(12)) - used:
        assert np.all(np.isnan(kc[blk])) and np.all(np.isnan(vc[blk]))
    assert len(used) == 3 + 1 + 1


def test_named_configs():
    c1 = wl.config("tiny_f32_2k")
    assert (c1.num_q_heads, c1.num_kv_heads, c1.head_dim, c1.num_blocks) == (8, 2, 64, 256)
    assert c1.kv_bytes == 2 * 1024 * 1024 and c1.scale == 0.125
    c2 = wl.config("long_100k_gqa8")
    assert c2.kv_bytes == 204_800_000 and c2.max_blocks_per_seq == 6250
    assert c2.partition_sizes == (512, 1024) and c2.num_blocks == 8192
    c3 = wl.config("batch16_1k_32k")
    assert c3.num_seqs == 16 and c3.seq_lens.min() >= 1024 and c3.seq_lens.max() <= 32768
    c4 = wl.config("batch64_mixed_outliers")
    lens = c4.seq_lens
    assert c4.num_seqs == 64
    assert np.sum((lens >= 128) & (lens <= 4096)) == 48
    assert np.sum((lens >= 32768) & (lens <= 131072)) == 16
    assert c4.outlier_frac == 0.01 and c4.outlier_mult == 20.0
    used = int(np.sum(-(-lens.astype(np.int64) // 16)))
    assert c4.num_blocks >= used
    c5 = wl.config("batch8_131k_gqa5")
    assert c5.num_q_heads // c5.num_kv_heads == 5 and c5.kv_bytes == 4_294_967_296
    assert c5.num_blocks == 70000


def test_tiny_config_generates():
    b = wl.generate(wl.config("tiny_f32_2k"))
    assert b.query.shape == (1, 8, 64) and b.key_cache.shape == (256, 2, 16, 16, 4)
    assert b.value_cache.shape == (256, 2, 64, 16)
    assert b.block_tables.shape == (1, 128) and b.block_tables.dtype == torch.int32
    assert len(set(b.block_tables[0].tolist())) == 128
    assert b.query.dtype == torch.float32


def test_cache_layout_by_definition():
    """Keys [blocks][Hkv][D / x][16][x] (x = 16 bytes of values), values
    [blocks][Hkv][D][16]: element (block b, head h, slot t, dim d) checked at its
    index formula, element by element, against the logical draw."""
    for dtype, x in (("bf16", 8), ("f32", 4)):
        spec = wl.custom("layout", 9, dtype, 4, 2, 64, [40, 7], num_blocks=6)
        b = wl.generate(spec, poison=False)
        _, kc, vc, _, _ = b.numpy()
        _, kl, vl, _, _ = b.numpy_logical()
        kf, vf = kc.reshape(-1), vc.reshape(-1)
        nb, H, B, D = kl.shape
        for bb in range(nb):
            for h in range(H):
                for t in range(B):
                    for d in range(D):
                        ki = (((bb * H + h) * (D // x) + d // x) * B + t) * x + d % x
                        vi = ((bb * H + h) * D + d) * B + t
                        assert kf[ki] == kl[bb, h, t, d] and vf[vi] == vl[bb, h, t, d]
        k2, v2 = wl.pack_kv(kl, vl)
        assert np.array_equal(k2.view(np.uint8), kc.view(np.uint8))
        assert np.array_equal(v2.view(np.uint8), vc.view(np.uint8))
