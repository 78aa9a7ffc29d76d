"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Small batches (several blocks, partitions and waves, ragged tails, NaN-poisoned
unused slots and workspace) are compared on every output; the five named
workloads at full size are compared on every output.  Phase 1 and Phase 2 are
also checked alone.
"""
import numpy as np
import pytest
import torch

import oracle
import split_kv_paged_pa_amd as pa
from parity import DeviceBatch, assert_close, oracle_out, require_gpu, sample_rows, to_f64
from split_kv_paged_pa_amd import workloads as wl

pytestmark = pytest.mark.gpu

EDGE_LENS = [1, 15, 16, 17, 511, 512, 513, 1023, 1024, 1025, 3000, 0]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()
    print(f"\n[gpu] {torch.cuda.get_device_name(0)}", flush=True)


SMALL = [("f32", 64, 8, 2), ("f32", 128, 4, 4), ("bf16", 128, 32, 4), ("bf16", 64, 16, 1),
         ("bf16", 128, 40, 8), ("bf16", 128, 8, 8)]


@pytest.mark.parametrize("dtype,D,Hq,Hkv", SMALL, ids=lambda x: str(x))
@pytest.mark.parametrize("variant,P", [("v1", None), ("v2", 16), ("v2", 512), ("v2", 1024),
                                       ("v2", 4096)])
def test_small_ragged(dtype, D, Hq, Hkv, variant, P):
    spec = wl.custom("small", 101, dtype, Hq, Hkv, D, EDGE_LENS)
    b = wl.generate(spec)
    db = DeviceBatch(b)
    print(f"[case] small {dtype} D={D} Hq={Hq} Hkv={Hkv} {variant} P={P}", flush=True)
    out = db.run(variant, P)
    ref = oracle_out(b)
    assert_close(to_f64(out), ref, dtype, f"{variant} P={P}")


# fp32 stops at 0.3: at scale 2.0 (logits of magnitude ~50 at D = 128) the fp32
# rounding of q.k alone, about sqrt(D) * 2^-24 * |scale| * sum |q_d k_d|, moves
# the weights by ~1e-5 -- the fp32 bar, which is derived for scales near
# 1 / sqrt(D) (measured 1.5e-5 there; bf16's bar covers it).
SCALES = [("bf16", -0.11), ("bf16", 0.0), ("bf16", 0.3), ("bf16", 2.0),
          ("f32", -0.11), ("f32", 0.0), ("f32", 0.3)]


@pytest.mark.parametrize("dtype,scale", SCALES, ids=[f"{d}_{s}" for d, s in SCALES])
def test_decode_scale_values(dtype, scale):
    """Negative, zero, large and non-default positive scales through V1, V2 (per
    partition and equal spans), the single launch and q_len 3 on the decode
    kernel: the logits are scale * q.k before the max, whatever its sign."""
    spec = wl.custom(f"scale_{dtype}", 151, dtype, 32, 4, 128, [3000, 17, 1500], scale=scale)
    b = wl.generate(spec)
    db = DeviceBatch(b)
    print(f"[case] decode scale={scale} {dtype}", flush=True)
    ref = oracle_out(b)
    assert_close(to_f64(db.run_v1()), ref, dtype, f"v1 scale={scale}")
    for P in (64, 512):
        assert_close(to_f64(db.run_v2(P)), ref, dtype, f"v2 P={P} scale={scale}")
    out = db.new_out()
    pa.pa_decode_v2_single(out, *db.args(), 256, db.workspace(256))
    assert_close(to_f64(out), ref, dtype, f"single launch scale={scale}")
    q = _multi_query(spec, 3)
    _, kc, vc, bt, sl = b.numpy()
    refq = oracle.decode_q(wl.to_numpy(q.cpu()), kc, vc, bt, sl, scale, dtype=dtype)
    outq = torch.full_like(q, float("nan"))
    pa.pa_decode_v1_q(outq, q, db.key_cache, db.value_cache, db.block_tables, db.seq_lens, scale,
                      db.max_seq_len)
    assert_close(to_f64(outq), refq, dtype, f"v1_q q_len=3 scale={scale}")


def test_zero_length_rows_are_zero():
    spec = wl.custom("zeros", 102, "bf16", 8, 2, 128, [0, 40, 0])
    db = DeviceBatch(wl.generate(spec))
    for out in (db.run_v1(), db.run_v2(512)):
        o = to_f64(out)
        assert np.all(o[0] == 0) and np.all(o[2] == 0)
        assert np.all(np.isfinite(o[1]))


def test_all_empty_batch():
    spec = wl.custom("empty", 103, "f32", 4, 2, 64, [0, 0], num_blocks=1)
    db = DeviceBatch(wl.generate(spec))
    db.max_seq_len = 0
    o1 = to_f64(db.run_v1())
    o2 = to_f64(db.run_v2(512))
    assert np.all(o1 == 0) and np.all(o2 == 0)


def test_many_partitions_reduce_chunks():
    """P = 16 over 20000 tokens: 1250 partitions, more than one staging round of the reduce."""
    spec = wl.custom("manyparts", 104, "bf16", 16, 1, 128, [20000, 7])
    b = wl.generate(spec)
    out = DeviceBatch(b).run_v2(16)
    assert_close(to_f64(out), oracle_out(b), "bf16", "P=16, 1250 partitions")


GROUPED = [  # S * Hkv * ceil(max_len / P) between one and four units per compute unit
    # (on 256 CUs: spans of 2, 3, 4, 4, 4 and 4 partitions' length); name, lens, Hkv,
    # GQA group, P.  The last case, 16 columns, is cut into 85 spans of 65 blocks
    # per row: each span starts and ends inside one of the caller's 16-block
    # partitions.
    ("one_seq_p512", [20000], 8, 8, 512),
    ("one_seq_p256", [20000], 8, 8, 256),
    ("ragged_p256", [20000, 5, 13000], 4, 8, 256),
    ("ragged_p1024", [100000, 17, 65536, 1], 2, 8, 1024),
    ("one_seq_100k_p512", [100000], 4, 8, 512),
    ("unaligned_spans_g16", [87296, 87296, 86000], 1, 16, 256),
]


@pytest.mark.parametrize("name,lens,hkv,group,P", GROUPED, ids=[g[0] for g in GROUPED])
def test_grouped_partitions(name, lens, hkv, group, P):
    """Phase-1 workgroups that handle several consecutive partitions each."""
    spec = wl.custom(name, 112, "bf16", hkv * group, hkv, 128, lens)
    b = wl.generate(spec)
    db = DeviceBatch(b)
    print(f"[case] grouped {name}", flush=True)
    ref = oracle_out(b)
    assert_close(to_f64(db.run_v2(P)), ref, "bf16", f"grouped {name}")
    ws = db.workspace(P)
    pa.pa_decode_v2_partials(*db.args(), P, ws)
    tmp, es, ml = (to_f64(x) for x in pa.workspace_views(ws, spec.num_seqs, spec.num_q_heads,
                                                         spec.head_dim, db.max_seq_len, P))
    q, kc, vc, bt, sl = b.numpy()
    rtmp, res, rml = oracle.partials(q, kc, vc, bt, sl, spec.scale, P, dtype="bf16",
                                     max_partitions=tmp.shape[2])
    for s, L in enumerate(sl):
        n = oracle.num_partitions(L, P)
        assert np.all(np.abs(ml[s, :, :n] - rml[s, :, :n]) <= 1e-5 * (1 + np.abs(rml[s, :, :n])))
        assert_close(tmp[s, :, :n], rtmp[s, :, :n], "bf16", f"grouped partials s={s}")


@pytest.mark.parametrize("name,lens,hkv,group,P", GROUPED, ids=[g[0] for g in GROUPED])
def test_grouped_entries(name, lens, hkv, group, P):
    """Phase 1 as pa_decode_v2 runs it (pa_decode_v2_groups): with few partitions,
    equal spans of entry_tokens tokens, each entry the partial of the span's tokens
    -- compared with the oracle's partials at partition size entry_tokens.  Then
    Phase 2 over those entries reproduces pa_decode_v2 bit for bit."""
    spec = wl.custom(name, 112, "bf16", hkv * group, hkv, 128, lens)
    b = wl.generate(spec)
    db = DeviceBatch(b)
    ws = db.workspace(P)
    et = pa.pa_decode_v2_groups(*db.args(), P, ws)
    print(f"[case] grouped entries {name}: {et} tokens per entry", flush=True)
    assert et % 16 == 0 and et != P, "these shapes take equal spans on 256 CUs"
    if name.startswith("unaligned"):
        assert et == 65 * 16, "85 spans of 65 blocks"
    tmp, es, ml = (to_f64(x) for x in pa.workspace_views(ws, spec.num_seqs, spec.num_q_heads,
                                                         spec.head_dim, db.max_seq_len, P))
    q, kc, vc, bt, sl = b.numpy()
    rtmp, res, rml = oracle.partials(q, kc, vc, bt, sl, spec.scale, et, dtype="bf16")
    for s_, L in enumerate(sl):
        n = oracle.num_partitions(L, et)
        assert n <= tmp.shape[2]
        assert np.all(np.abs(ml[s_, :, :n] - rml[s_, :, :n]) <= 1e-5 * (1 + np.abs(rml[s_, :, :n])))
        assert np.all(np.abs(es[s_, :, :n] - res[s_, :, :n]) <= 1e-2 * res[s_, :, :n])
        assert_close(tmp[s_, :, :n], rtmp[s_, :, :n], "bf16", f"span entries s={s_}")
        # The spans past a shorter sequence's end mark their entries empty.
        spans = oracle.num_partitions(db.max_seq_len, et)
        assert np.all(ml[s_, :, n:spans] == -np.inf)
    out = db.new_out()
    pa.pa_decode_v2_reduce_entries(out, db.seq_lens, db.max_seq_len, P, et, ws)
    ref = db.run_v2(P)
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))


def test_outlier_keys_stability():
    spec = wl.custom("outliers", 105, "bf16", 16, 2, 128, [5000, 300, 9000],
                     outlier_frac=0.02, outlier_mult=40.0)
    b = wl.generate(spec)
    ref = oracle_out(b)
    db = DeviceBatch(b)
    for variant, P in (("v1", None), ("v2", 512), ("v2", 1024)):
        assert_close(to_f64(db.run(variant, P)), ref, "bf16", f"outliers {variant} P={P}")


def test_deterministic_bitwise():
    spec = wl.custom("det", 106, "bf16", 32, 4, 128, [7777, 300])
    db = DeviceBatch(wl.generate(spec))
    for variant, P in (("v1", None), ("v2", 512)):
        a = db.run(variant, P)
        b = db.run(variant, P)
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), variant


def test_block_relabel_bitwise():
    """Permuting the pool and rewriting the table gives bit-identical output."""
    spec = wl.custom("relabel", 107, "bf16", 8, 2, 128, [900, 33, 2048])
    b = wl.generate(spec)
    db = DeviceBatch(b)
    base = [db.run_v1(), db.run_v2(512)]
    perm = torch.randperm(b.key_cache.shape[0], generator=torch.Generator().manual_seed(0))
    inv = torch.argsort(perm)
    bt = b.block_tables.clone()
    valid = bt >= 0
    bt[valid] = inv[bt[valid].long()].int()
    b2 = wl.Batch(spec, b.query, b.key_cache[perm].contiguous(), b.value_cache[perm].contiguous(),
                  bt, b.seq_lens)
    db2 = DeviceBatch(b2)
    moved = [db2.run_v1(), db2.run_v2(512)]
    for x, y in zip(base, moved):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))


def test_out_of_range_block_ids_are_skipped():
    """Ids outside [0, num_blocks) are never read; their tokens leave the softmax."""
    spec = wl.custom("badids", 108, "f32", 8, 2, 64, [100, 64])
    b = wl.generate(spec)
    db = DeviceBatch(b)
    bt = b.block_tables.clone()
    bt[0, 2] = -7
    bt[1, 0] = b.key_cache.shape[0] + 3
    db.block_tables = bt.to("cuda")
    # Reference: the same sequences with those blocks' tokens zero-weighted, i.e. the
    # oracle over a copy whose removed tokens carry logit -inf: rebuild without them.
    q, kc, vc, bt_np, _ = b.numpy_logical()
    keep0 = [j for j in range(7) if j != 2]
    keep1 = [1, 2, 3]
    rows = []
    for s, keep, L in ((0, keep0, 100), (1, keep1, 64)):
        toks = [t for t in range(L) if (t // 16) in keep]
        dense_k = np.stack([kc[bt_np[s, t // 16], :, t % 16] for t in toks])
        dense_v = np.stack([vc[bt_np[s, t // 16], :, t % 16] for t in toks])
        n = len(toks)
        nb = -(-n // 16)
        kk = np.full((nb, 2, 16, 64), np.nan, np.float32)
        vv = np.full((nb, 2, 16, 64), np.nan, np.float32)
        for i in range(n):
            kk[i // 16, :, i % 16] = dense_k[i]
            vv[i // 16, :, i % 16] = dense_v[i]
        ref = oracle.decode(np.ascontiguousarray(q[s:s + 1]), *wl.pack_kv(kk, vv),
                            np.arange(nb, dtype=np.int32)[None], np.array([n], np.int32),
                            spec.scale, dtype="f32")
        rows.append(ref[0])
    ref = np.stack(rows)
    for out in (db.run_v1(), db.run_v2(32)):
        assert_close(to_f64(out), ref, "f32", "skipped block ids")


def test_phase1_partials_match_oracle():
    spec = wl.custom("p1", 109, "bf16", 32, 4, 128, [3000, 17, 1024, 0])
    b = wl.generate(spec)
    db = DeviceBatch(b)
    P = 512
    ws = db.workspace(P)
    pa.pa_decode_v2_partials(*db.args(), P, ws)
    tmp, es, ml = (to_f64(x) for x in pa.workspace_views(ws, spec.num_seqs, spec.num_q_heads,
                                                         spec.head_dim, db.max_seq_len, P))
    q, kc, vc, bt, sl = b.numpy()
    rtmp, res, rml = oracle.partials(q, kc, vc, bt, sl, spec.scale, P, dtype="bf16",
                                     max_partitions=tmp.shape[2])
    for s, L in enumerate(sl):
        n = oracle.num_partitions(L, P)
        assert np.all(np.abs(ml[s, :, :n] - rml[s, :, :n]) <= 1e-5 * (1 + np.abs(rml[s, :, :n])))
        assert np.all(np.abs(es[s, :, :n] - res[s, :, :n]) <= 1e-2 * res[s, :, :n])
        assert_close(tmp[s, :, :n], rtmp[s, :, :n], "bf16", f"tmp_output s={s}")


def test_phase2_alone_on_oracle_partials():
    """Phase 2 fed float32-rounded oracle partials vs the oracle merge of the same values."""
    spec = wl.custom("p2", 110, "f32", 8, 2, 128, [5000, 1, 700, 0])
    b = wl.generate(spec)
    db = DeviceBatch(b)
    P = 256
    q, kc, vc, bt, sl = b.numpy()
    rtmp, res, rml = oracle.partials(q, kc, vc, bt, sl, spec.scale, P, dtype="f32")
    f32 = [np.nan_to_num(x).astype(np.float32) for x in (rtmp, res, rml)]
    ref = oracle.merge(*(x.astype(np.float64) for x in f32), sl, P)
    ws = db.workspace(P)
    tmp, es, ml = pa.workspace_views(ws, spec.num_seqs, spec.num_q_heads, spec.head_dim,
                                     db.max_seq_len, P)
    tmp.copy_(torch.from_numpy(f32[0]))
    es.copy_(torch.from_numpy(f32[1]))
    ml.copy_(torch.from_numpy(f32[2]))
    out = torch.full_like(db.query, float("nan"))
    pa.pa_decode_v2_reduce(out, db.seq_lens, db.max_seq_len, P, ws)
    g = to_f64(out)
    err = np.abs(g - ref)
    # float32 rounding bound: the merge sums weighted partial outputs of either sign, so
    # its error scales with sum_p (w_p / W) |o_p|, the same merge over |o_p|.
    mag = oracle.merge(np.abs(f32[0]).astype(np.float64), *(x.astype(np.float64) for x in f32[1:]),
                       sl, P)
    assert np.all(err <= 4e-6 * mag + 1e-30), float(np.max(err / np.maximum(mag, 1e-30)))


def test_dispatch_threshold():
    """pa_decode follows the 8192 rule: V1 (no workspace needed) at 8192, V2 above."""
    assert not pa.pa_select_v2(8192, 1, 4, 1024) and pa.pa_select_v2(8193, 1, 4, 1024)
    for L in (8192, 8193):
        spec = wl.custom("dispatch", 111, "bf16", 8, 2, 128, [L])
        b = wl.generate(spec)
        db = DeviceBatch(b)
        out = db.new_out()
        if L == 8192:
            pa.pa_decode(out, *db.args(), 1024, None)
        else:
            with pytest.raises(pa.PagedAttentionError):
                pa.pa_decode(out, *db.args(), 1024, None)
            pa.pa_decode(out, *db.args(), 1024, db.workspace(1024))
        assert_close(to_f64(out), oracle_out(b), "bf16", f"pa_decode L={L}")


# ---------------------------------------------------------------------------
# Single-launch V2 (pa_decode_v2_single): the last workgroup of each
# (sequence, kv head) merges.
# ---------------------------------------------------------------------------
FUSED = [  # name, dtype, Hq, Hkv, D, lens, P
    ("ragged_bf16", "bf16", 32, 4, 128, EDGE_LENS, 512),
    ("gqa5", "bf16", 40, 8, 128, [3000, 1, 700, 0, 4097], 256),
    ("f32_d64", "f32", 8, 2, 64, [5000, 16, 17], 128),
    ("grouped_long", "bf16", 64, 8, 128, [20000], 512),
    ("g16_d128", "bf16", 16, 1, 128, [9000, 33], 64),
    ("long_100k_shape", "bf16", 32, 4, 128, [100000], 1024),
    # 8 x 4 rows x 36 partitions: several partitions per workgroup, folded.
    ("partitions", "bf16", 32, 4, 128, [9000, 8000, 7000, 100, 9000, 1, 5000, 9000], 256),
]


def _header(ws):
    return ws.view(torch.uint8)[:pa.api.WORKSPACE_HEADER_BYTES].cpu()


def run_single(db, P, ws):
    out = db.new_out()
    pa.pa_decode_v2_single(out, *db.args(), P, ws)
    return out


@pytest.mark.parametrize("name,dtype,Hq,Hkv,D,lens,P", FUSED, ids=[f[0] for f in FUSED])
def test_single_launch_v2(name, dtype, Hq, Hkv, D, lens, P):
    """One launch against the oracle and against pa_decode_v2 on the same inputs;
    bitwise repeatable; the counter header is zero again afterwards."""
    spec = wl.custom(name, 113, dtype, Hq, Hkv, D, lens)
    b = wl.generate(spec)
    db = DeviceBatch(b)
    print(f"[case] single launch {name}", flush=True)
    ref = oracle_out(b)
    ws = db.workspace(P)
    out = run_single(db, P, ws)
    assert_close(to_f64(out), ref, dtype, f"single launch {name}")
    assert torch.count_nonzero(_header(ws)) == 0, "arrival counters not left at zero"
    again = run_single(db, P, ws)
    assert torch.equal(out.view(torch.uint8), again.view(torch.uint8)), "not repeatable"
    assert_close(to_f64(db.run_v2(P)), ref, dtype, f"two launches {name}")


def test_single_launch_workspace_reuse_across_shapes():
    """One workspace serves calls of different shapes in turn: the counters each call
    uses are left at zero, so the next shape starts clean."""
    specs = [wl.custom("reuseA", 114, "bf16", 32, 4, 128, [3000, 900, 17]),
             wl.custom("reuseB", 115, "bf16", 64, 8, 128, [5000]),
             wl.custom("reuseC", 116, "f32", 8, 1, 64, [1, 2000, 70, 0, 4000])]
    P = 256
    size = max(pa.pa_workspace_size(sp.num_seqs, sp.num_q_heads, sp.head_dim, sp.max_seq_len, P)
               for sp in specs)
    ws = torch.zeros(size, dtype=torch.uint8, device="cuda")
    batches = [wl.generate(sp) for sp in specs]
    refs = [oracle_out(b) for b in batches]
    for rnd in range(2):
        for sp, b, ref in zip(specs, batches, refs):
            db = DeviceBatch(b)
            out = run_single(db, P, ws)
            assert_close(to_f64(out), ref, sp.dtype, f"{sp.name} round {rnd}")
            assert torch.count_nonzero(_header(ws)) == 0


def test_single_launch_refuses_what_does_not_fit():
    """More group partials than the merge table holds: PA_ERR_UNSUPPORTED, nothing
    written; pa_decode_v2 handles the same problem."""
    spec = wl.custom("nofit", 117, "bf16", 16, 2, 128, [12000, 40])
    b = wl.generate(spec)
    db = DeviceBatch(b)
    out = db.new_out()
    with pytest.raises(pa.PagedAttentionError) as e:
        pa.pa_decode_v2_single(out, *db.args(), 16, db.workspace(16))
    assert e.value.status == 3  # PA_ERR_UNSUPPORTED
    assert torch.isnan(out).all()
    assert_close(to_f64(db.run_v2(16)), oracle_out(b), "bf16", "two launches, P=16")


def test_single_launch_empty_batch_zero_rows():
    spec = wl.custom("single_empty", 118, "bf16", 8, 2, 128, [0, 0], num_blocks=1)
    db = DeviceBatch(wl.generate(spec))
    db.max_seq_len = 0
    assert np.all(to_f64(run_single(db, 512, db.workspace(512))) == 0)


AUTO = [  # lens, Hkv, expected choice on a 256-CU device
    ([4096, 3000], 8, True),           # 16 units < 128: V2 below the pages' threshold
    ([2048] * 20, 8, False),           # 160 units >= 128: V1
    ([700, 1024, 5], 4, False),        # max_seq_len <= 1024: V1
    ([9000, 12], 2, True),             # above 8192: V2
]


@pytest.mark.parametrize("lens,hkv,v2", AUTO, ids=["few_units", "many_units", "short", "long"])
def test_decode_auto(lens, hkv, v2):
    """pa_decode_auto follows the measured MI355X rule and matches the oracle."""
    spec = wl.custom("auto", 120, "bf16", hkv * 8, hkv, 128, lens)
    b = wl.generate(spec)
    db = DeviceBatch(b)
    if torch.cuda.get_device_properties(0).multi_processor_count == 256:
        assert pa.pa_select_v2_auto(db.max_seq_len, spec.num_seqs, hkv, 512) is v2
    out = db.new_out()
    pa.pa_decode_auto(out, *db.args(), 512, db.workspace(512))
    assert_close(to_f64(out), oracle_out(b), "bf16", "pa_decode_auto")


# ---------------------------------------------------------------------------
# q_len query tokens per sequence (causal over the cache).
# ---------------------------------------------------------------------------
MULTI = [  # dtype, D, Hq, Hkv, q_len, P
    ("bf16", 128, 32, 4, 2, 512),
    ("bf16", 128, 16, 4, 4, 16),
    ("f32", 64, 8, 2, 3, 512),
    ("bf16", 64, 5, 1, 3, 1024),
    ("bf16", 128, 16, 16, 4, 256),
]
MULTI_LENS = [1, 2, 3, 4, 15, 16, 17, 100, 513, 1025, 3000, 0]


def _multi_query(spec, q_len, dev="cuda"):
    rng = np.random.default_rng(spec.seed)
    qf = rng.standard_normal((spec.num_seqs, q_len, spec.num_q_heads, spec.head_dim),
                             dtype=np.float32)
    return torch.from_numpy(qf).to(wl.torch_dtype(spec.dtype)).to(dev)


@pytest.mark.parametrize("dtype,D,Hq,Hkv,q_len,P", MULTI, ids=lambda x: str(x))
def test_multi_query_decode(dtype, D, Hq, Hkv, q_len, P):
    spec = wl.custom("multiq", 121, dtype, Hq, Hkv, D, MULTI_LENS)
    b = wl.generate(spec)
    db = DeviceBatch(b)
    q = _multi_query(spec, q_len)
    print(f"[case] multi-query {dtype} D={D} Hq={Hq} Hkv={Hkv} q_len={q_len} P={P}", flush=True)
    _, kc, vc, bt, sl = b.numpy()
    ref = oracle.decode_q(wl.to_numpy(q.cpu()), kc, vc, bt, sl, spec.scale, dtype=dtype)
    out1 = torch.full_like(q, float("nan"))
    pa.pa_decode_v1_q(out1, q, db.key_cache, db.value_cache, db.block_tables, db.seq_lens,
                      spec.scale, db.max_seq_len)
    assert_close(to_f64(out1), ref, dtype, f"v1 q_len={q_len}")
    ws = pa.new_workspace(spec.num_seqs, q_len * Hq, D, db.max_seq_len, P)
    ws.fill_(0xFF)
    out2 = torch.full_like(q, float("nan"))
    pa.pa_decode_v2_q(out2, q, db.key_cache, db.value_cache, db.block_tables, db.seq_lens,
                      spec.scale, db.max_seq_len, P, ws)
    assert_close(to_f64(out2), ref, dtype, f"v2 q_len={q_len} P={P}")


def test_multi_query_q1_is_plain_decode():
    """q_len = 1 through the q_len entry points equals the plain ones bit for bit."""
    spec = wl.custom("q1", 122, "bf16", 32, 4, 128, [3000, 17, 0, 1024])
    db = DeviceBatch(wl.generate(spec))
    q4 = db.query[:, None].contiguous()
    o1 = torch.empty_like(q4)
    pa.pa_decode_v1_q(o1, q4, db.key_cache, db.value_cache, db.block_tables, db.seq_lens,
                      spec.scale, db.max_seq_len)
    o2 = torch.empty_like(q4)
    pa.pa_decode_v2_q(o2, q4, db.key_cache, db.value_cache, db.block_tables, db.seq_lens,
                      spec.scale, db.max_seq_len, 512, db.workspace(512))
    assert torch.equal(o1[:, 0].view(torch.int16), db.run_v1().view(torch.int16))
    assert torch.equal(o2[:, 0].view(torch.int16), db.run_v2(512).view(torch.int16))


CHUNKED = [  # name, dtype, D, Hq, Hkv, q_len, lens, P: more than 16 (token, head) columns per kv head
    ("g8_q3", "bf16", 128, 16, 2, 3, [1, 2, 40, 1000, 0], 256),
    ("g4_q9", "bf16", 128, 8, 2, 9, [5, 9, 10, 700, 2000], 512),
    # 4 or more chunks: each wave of a workgroup owns a chunk (wave columns).
    ("prefill_q64", "bf16", 128, 8, 2, 64, [64, 100, 300, 0, 17], 128),
    ("wc_g8_q8", "bf16", 128, 32, 4, 8, [8, 9, 1000, 4097], 1024),
    # 68 columns = 5 chunks: the second workgroup of a kv head has one wave with columns.
    ("wc_g4_q17_f32", "f32", 64, 8, 2, 17, [1, 17, 18, 500, 0], 256),
    ("wc_g1_q100_d64", "bf16", 64, 3, 3, 100, [100, 250, 33], 64),
]


@pytest.mark.parametrize("name,dtype,D,Hq,Hkv,q_len,lens,P", CHUNKED, ids=[c[0] for c in CHUNKED])
def test_multi_query_column_chunks(name, dtype, D, Hq, Hkv, q_len, lens, P):
    """G * q_len > 16: 16 columns per chunk; one chunk per workgroup below 4 chunks,
    one per wave from 4 on."""
    spec = wl.custom(name, 123, dtype, Hq, Hkv, D, lens)
    b = wl.generate(spec)
    db = DeviceBatch(b)
    q = _multi_query(spec, q_len)
    print(f"[case] column chunks {name}", flush=True)
    _, kc, vc, bt, sl = b.numpy()
    ref = oracle.decode_q(wl.to_numpy(q.cpu()), kc, vc, bt, sl, spec.scale, dtype=dtype)
    out1 = torch.full_like(q, float("nan"))
    pa.pa_decode_v1_q(out1, q, db.key_cache, db.value_cache, db.block_tables, db.seq_lens,
                      spec.scale, db.max_seq_len)
    assert_close(to_f64(out1), ref, dtype, f"v1 {name}")
    ws = pa.new_workspace(spec.num_seqs, q_len * Hq, D, db.max_seq_len, P)
    ws.view(torch.uint8).fill_(0xFF)
    pa.pa_workspace_init(ws)
    out2 = torch.full_like(q, float("nan"))
    pa.pa_decode_v2_q(out2, q, db.key_cache, db.value_cache, db.block_tables, db.seq_lens,
                      spec.scale, db.max_seq_len, P, ws)
    assert_close(to_f64(out2), ref, dtype, f"v2 {name}")


# ---------------------------------------------------------------------------
# Tiled prefill (pa_prefill_v1 / pa_prefill_v2): the q_len computation on the
# kernel that holds several 16-column tiles per wave.
# ---------------------------------------------------------------------------
PREFILL = [  # name, D, Hq, Hkv, q_len, lens, P
    ("g4_q64", 128, 8, 2, 64, [64, 100, 300, 0, 17], 128),          # 256 columns per kv head
    ("g8_q40_d64", 64, 32, 4, 40, [40, 1000, 39, 2049], 256),       # 320: ragged wave groups
    ("g1_q100", 128, 3, 3, 100, [100, 250, 33], 64),                # G = 1
    ("g5_q33_p16", 128, 10, 2, 33, [33, 500, 5, 47], 16),           # G = 5; steps span partitions
    ("g2_q7", 64, 4, 2, 7, [7, 3, 90], 32),                         # 14 columns: one partial tile
]


def _prefill_run(db, q, P, tiles, scale=None):
    scale = db.spec.scale if scale is None else scale
    out1 = torch.full_like(q, float("nan"))
    pa.pa_prefill_v1(out1, q, db.key_cache, db.value_cache, db.block_tables, db.seq_lens, scale,
                     db.max_seq_len, tiles)
    S, q_len, Hq, D = q.shape
    ws = pa.new_workspace(S, q_len * Hq, D, db.max_seq_len, P)
    ws.view(torch.uint8).fill_(0xFF)
    pa.pa_workspace_init(ws)
    out2 = torch.full_like(q, float("nan"))
    pa.pa_prefill_v2(out2, q, db.key_cache, db.value_cache, db.block_tables, db.seq_lens, scale,
                     db.max_seq_len, P, ws, tiles)
    return out1, out2


@pytest.mark.parametrize("tiles", [1, 2, 4])
@pytest.mark.parametrize("name,D,Hq,Hkv,q_len,lens,P", PREFILL, ids=[c[0] for c in PREFILL])
def test_prefill(name, D, Hq, Hkv, q_len, lens, P, tiles):
    spec = wl.custom("prefill_" + name, 125, "bf16", Hq, Hkv, D, lens)
    b = wl.generate(spec)
    db = DeviceBatch(b)
    q = _multi_query(spec, q_len)
    print(f"[case] prefill {name} tiles={tiles}", flush=True)
    _, kc, vc, bt, sl = b.numpy()
    ref = oracle.decode_q(wl.to_numpy(q.cpu()), kc, vc, bt, sl, spec.scale, dtype="bf16")
    out1, out2 = _prefill_run(db, q, P, tiles)
    assert_close(to_f64(out1), ref, "bf16", f"prefill v1 {name} tiles={tiles}")
    assert_close(to_f64(out2), ref, "bf16", f"prefill v2 {name} P={P} tiles={tiles}")


@pytest.mark.parametrize("scale", [-0.11, 0.0, 0.3])
def test_prefill_scale_values(scale):
    """Negative and zero scales: the kernel takes its maxima before scaling."""
    spec = wl.custom("prefill_scale", 126, "bf16", 8, 2, 128, [70, 300])
    b = wl.generate(spec)
    db = DeviceBatch(b)
    q = _multi_query(spec, 24)
    _, kc, vc, bt, sl = b.numpy()
    ref = oracle.decode_q(wl.to_numpy(q.cpu()), kc, vc, bt, sl, scale, dtype="bf16")
    for tiles in (1, 4):
        out1, out2 = _prefill_run(db, q, 64, tiles, scale=scale)
        assert_close(to_f64(out1), ref, "bf16", f"prefill v1 scale={scale}")
        assert_close(to_f64(out2), ref, "bf16", f"prefill v2 scale={scale}")


def test_prefill_skipped_block_ids():
    """Ids outside [0, num_blocks) are never read and their tokens leave every
    query's softmax; positions (and so the causal limits) do not move.  Reference:
    the oracle's single-query decode of each query token over its visible tokens
    with the skipped blocks' tokens removed."""
    spec = wl.custom("prefill_badids", 127, "bf16", 8, 2, 64, [100, 70])
    b = wl.generate(spec)
    db = DeviceBatch(b)
    bt = b.block_tables.clone()
    bt[0, 2] = -7
    bt[1, 0] = b.key_cache.shape[0] + 3
    db.block_tables = bt.to("cuda")
    q_len = 40
    q = _multi_query(spec, q_len)
    qn = wl.to_numpy(q.cpu())
    _, kc, vc, bt_np, _ = b.numpy_logical()
    skip = {0: {2}, 1: {0}}
    ref = np.zeros(q.shape, np.float64)
    for s, L in ((0, 100), (1, 70)):
        for j in range(q_len):
            toks = [t for t in range(L - q_len + j + 1) if (t // 16) not in skip[s]]
            n = len(toks)
            if n == 0:
                continue
            nb = -(-n // 16)
            kk = np.full((nb, 2, 16, 64), 0x7FC0, np.uint16)  # bf16 NaN bit patterns
            vv = np.full((nb, 2, 16, 64), 0x7FC0, np.uint16)
            for i, t in enumerate(toks):
                kk[i // 16, :, i % 16] = kc[bt_np[s, t // 16], :, t % 16]
                vv[i // 16, :, i % 16] = vc[bt_np[s, t // 16], :, t % 16]
            ref[s, j] = oracle.decode(np.ascontiguousarray(qn[s, j][None]), *wl.pack_kv(kk, vv, 2),
                                      np.arange(nb, dtype=np.int32)[None], np.array([n], np.int32),
                                      spec.scale, dtype="bf16")[0]
    for tiles in (2, 4):
        out1, out2 = _prefill_run(db, q, 32, tiles)
        assert_close(to_f64(out1), ref, "bf16", "prefill v1 skipped ids")
        assert_close(to_f64(out2), ref, "bf16", "prefill v2 skipped ids")


def test_prefill_long_sampled():
    """q_len 512 over an 8192-token cache (Hq 32, Hkv 4, D 128) in the launch shapes
    the prefill timings use; sampled query tokens against the oracle's single-query
    decode over each token's visible prefix (L - q_len + j + 1 tokens)."""
    spec = wl.custom("prefill_long", 128, "bf16", 32, 4, 128, [8192])
    b = wl.generate(spec)
    db = DeviceBatch(b)
    q_len = 512
    q = _multi_query(spec, q_len)
    qn = wl.to_numpy(q.cpu())
    _, kc, vc, bt, _ = b.numpy()
    js = np.array([0, 1, 15, 16, 200, 383, 510, 511])
    ref = oracle.decode(np.ascontiguousarray(qn[0, js]), kc, vc, np.repeat(bt, len(js), 0),
                        (8192 - q_len + js + 1).astype(np.int32), spec.scale, dtype="bf16")
    for tiles in (2, 4):
        out1, out2 = _prefill_run(db, q, 1024, tiles)
        for out, what in ((out1, "v1"), (out2, "v2")):
            got = to_f64(out)
            assert np.all(np.isfinite(got)), what
            assert_close(got[0, js], ref, "bf16", f"prefill long {what} tiles={tiles}")
    # The q_len entry points take the prefill kernel at this shape on their own.
    assert pa.pa_select_q_kernel(1, 1, q_len, 32, 4, torch.bfloat16, 8192) > 0
    assert pa.pa_select_q_kernel(0, 1, q_len, 32, 4, torch.bfloat16, 8192, 1024) > 0
    o1 = torch.full_like(q, float("nan"))
    pa.pa_decode_v1_q(o1, q, db.key_cache, db.value_cache, db.block_tables, db.seq_lens,
                      spec.scale, db.max_seq_len)
    ws = pa.new_workspace(1, q_len * 32, 128, db.max_seq_len, 1024)
    o2 = torch.full_like(q, float("nan"))
    pa.pa_decode_v2_q(o2, q, db.key_cache, db.value_cache, db.block_tables, db.seq_lens,
                      spec.scale, db.max_seq_len, 1024, ws)
    for out, what in ((o1, "v1_q"), (o2, "v2_q")):
        got = to_f64(out)
        assert np.all(np.isfinite(got)), what
        assert_close(got[0, js], ref, "bf16", f"prefill long via {what}")


def test_prefill_auto_batch():
    """Twelve sequences of mixed length (some shorter than q_len, one empty),
    q_len 48, GQA 8: the q_len entry points choose the prefill kernel on their
    own (one column tile single pass, two split at P 512 on a 256-CU device) and
    match the oracle."""
    lens = [48, 3000, 0, 17, 640, 1200, 47, 2500, 96, 1, 2049, 777]
    spec = wl.custom("prefill_auto_batch", 129, "bf16", 32, 4, 128, lens)
    b = wl.generate(spec)
    db = DeviceBatch(b)
    q_len, P = 48, 512
    q = _multi_query(spec, q_len)
    _, kc, vc, bt, sl = b.numpy()
    ref = oracle.decode_q(wl.to_numpy(q.cpu()), kc, vc, bt, sl, spec.scale, dtype="bf16")
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    k1 = pa.pa_select_q_kernel(1, len(lens), q_len, 32, 4, torch.bfloat16, db.max_seq_len)
    k2 = pa.pa_select_q_kernel(0, len(lens), q_len, 32, 4, torch.bfloat16, db.max_seq_len, P)
    print(f"[case] prefill auto batch: {cus} CUs, kernels v1 {k1} v2 {k2}", flush=True)
    if cus == 256:
        assert (k1, k2) == (1, 2)
    o1 = torch.full_like(q, float("nan"))
    pa.pa_decode_v1_q(o1, q, db.key_cache, db.value_cache, db.block_tables, db.seq_lens,
                      spec.scale, db.max_seq_len)
    assert_close(to_f64(o1), ref, "bf16", "auto batch v1_q")
    ws = pa.new_workspace(len(lens), q_len * 32, 128, db.max_seq_len, P)
    ws.view(torch.uint8).fill_(0xFF)
    pa.pa_workspace_init(ws)
    o2 = torch.full_like(q, float("nan"))
    pa.pa_decode_v2_q(o2, q, db.key_cache, db.value_cache, db.block_tables, db.seq_lens,
                      spec.scale, db.max_seq_len, P, ws)
    assert_close(to_f64(o2), ref, "bf16", "auto batch v2_q")


def test_graph_capture_replays():
    """The V2 step (two launches, no allocation, no memset) captured in a HIP graph:
    every replay, with eager work and synchronisations between replays, matches the
    eager result bit for bit; the inputs change between replays through the same
    device buffers."""
    spec = wl.custom("graph", 124, "bf16", 32, 4, 128, [9000, 300, 17])
    b = wl.generate(spec)
    db = DeviceBatch(b)
    P = 512
    ws = db.workspace(P)
    out = db.new_out()
    qs = [db.query.clone(), (db.query * 0.5).contiguous(), (db.query * -1.0).contiguous()]
    q_buf = qs[0].clone()
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):  # warm-up outside capture
        pa.pa_decode_v2(out, q_buf, db.key_cache, db.value_cache, db.block_tables, db.seq_lens,
                        spec.scale, db.max_seq_len, P, ws, stream=stream)
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        pa.pa_decode_v2(out, q_buf, db.key_cache, db.value_cache, db.block_tables, db.seq_lens,
                        spec.scale, db.max_seq_len, P, ws, stream=stream)
    for rep in range(6):
        q = qs[rep % 3]
        q_buf.copy_(q)
        expect = db.new_out()
        pa.pa_decode_v2(expect, q, db.key_cache, db.value_cache, db.block_tables, db.seq_lens,
                        spec.scale, db.max_seq_len, P, db.workspace(P))
        torch.cuda.synchronize()
        out.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), expect.view(torch.int16)), f"replay {rep}"


def test_graph_capture_replays_prefill():
    """The split q_len path on the prefill kernel and the one-wave-per-row reduce,
    captured in a HIP graph: every replay matches the eager result bit for bit."""
    spec = wl.custom("graph_prefill", 130, "bf16", 32, 4, 128, [3000, 700, 48])
    b = wl.generate(spec)
    db = DeviceBatch(b)
    q_len, P = 48, 512
    assert pa.pa_select_q_kernel(0, 3, q_len, 32, 4, torch.bfloat16, db.max_seq_len, P) > 0
    qs = [_multi_query(spec, q_len)]
    qs += [(qs[0] * 0.5).contiguous(), (qs[0] * -1.0).contiguous()]
    q_buf = qs[0].clone()
    out = torch.empty_like(q_buf)
    ws = pa.new_workspace(3, q_len * 32, 128, db.max_seq_len, P)
    args = (db.key_cache, db.value_cache, db.block_tables, db.seq_lens, spec.scale, db.max_seq_len, P)
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):  # warm-up outside capture
        pa.pa_decode_v2_q(out, q_buf, *args, ws, stream=stream)
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        pa.pa_decode_v2_q(out, q_buf, *args, ws, stream=stream)
    for rep in range(6):
        q = qs[rep % 3]
        q_buf.copy_(q)
        expect = torch.full_like(q, float("nan"))
        pa.pa_decode_v2_q(expect, q, *args, pa.new_workspace(3, q_len * 32, 128, db.max_seq_len, P))
        torch.cuda.synchronize()
        out.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), expect.view(torch.int16)), f"replay {rep}"


# ---------------------------------------------------------------------------
# The five named workloads at full size, every (sequence, head) row compared
# with the oracle.  Partition sizes: the workload's own, 0 (the library's
# choice), plus 2048 for the 100K-token sequence.
# ---------------------------------------------------------------------------
FULL = [("tiny_f32_2k", (0,)), ("long_100k_gqa8", (2048, 0)), ("batch16_1k_32k", (0,)),
        ("batch64_mixed_outliers", (0,)), ("batch8_131k_gqa5", (0,))]


@pytest.mark.parametrize("name,extra_P", FULL, ids=[f[0] for f in FULL])
def test_named_workload(name, extra_P):
    spec = wl.config(name)
    print(f"[case] {name}: generating", flush=True)
    b = wl.generate(spec)
    db = DeviceBatch(b)
    print(f"[case] {name}: oracle on all {spec.num_seqs * spec.num_q_heads} rows", flush=True)
    ref = oracle_out(b)
    variants = [("v2", P) for P in tuple(spec.partition_sizes) + tuple(extra_P)] + [("v1", None)]
    for variant, P in variants:
        print(f"[case] {name}: {variant} P={P}", flush=True)
        out = to_f64(db.run(variant, P))
        err = assert_close(out, ref, spec.dtype, f"{name} {variant} P={P}")
        print(f"[case] {name}: {variant} P={P} max abs err {err:.3e}", flush=True)
    del db
    torch.cuda.empty_cache()


@pytest.mark.parametrize("S,P", [(200, 256), (257, 512), (96, 4096)])
def test_many_ragged_sequences(S, P):
    """Many ragged sequences, zero-length ones among them: Phase 1's grid rotates
    each row's partition index (rows whose length is a multiple of 8 included:
    12 and 8 partitions at P = 256 and 4096).  Every row against the oracle, the
    partials too."""
    rng = np.random.default_rng(S)
    lens = rng.integers(0, 3000 if P < 4096 else 32768, size=S, endpoint=True)
    lens[rng.integers(S, size=S // 8)] = 0
    spec = wl.custom(f"many{S}", 132, "bf16", 8, 2, 64, lens)
    b = wl.generate(spec)
    db = DeviceBatch(b)
    print(f"[case] many sequences S={S} P={P}", flush=True)
    assert_close(to_f64(db.run_v2(P)), oracle_out(b), "bf16", f"many S={S} P={P}")
    ws = db.workspace(P)
    pa.pa_decode_v2_partials(*db.args(), P, ws)
    tmp, es, ml = (to_f64(x) for x in pa.workspace_views(ws, spec.num_seqs, spec.num_q_heads,
                                                         spec.head_dim, db.max_seq_len, P))
    q, kc, vc, bt, sl = b.numpy()
    rtmp, res, rml = oracle.partials(q, kc, vc, bt, sl, spec.scale, P, dtype="bf16",
                                     max_partitions=tmp.shape[2])
    for s_, L in enumerate(sl):
        n = oracle.num_partitions(L, P)
        assert np.all(np.abs(ml[s_, :, :n] - rml[s_, :, :n]) <= 1e-5 * (1 + np.abs(rml[s_, :, :n])))
        assert_close(tmp[s_, :, :n], rtmp[s_, :, :n], "bf16", f"partials s={s_}")


def test_reduce_workgroup_per_row_all_rows():
    """2048 (sequence, head) rows with up to 32 partitions each: Phase 2 takes one
    16-wave workgroup per row (the form the 64-sequence batch uses); every row is
    compared with the oracle."""
    lens = np.random.default_rng(5).integers(2500, 4096, size=64, endpoint=True)
    spec = wl.custom("rows2048", 131, "bf16", 32, 4, 128, lens)
    b = wl.generate(spec)
    db = DeviceBatch(b)
    assert spec.num_seqs * spec.num_q_heads >= 2048
    out = to_f64(db.run_v2(128))
    assert_close(out, oracle_out(b), "bf16", "2048 rows, P=128")
