"""Pins of the CPU oracle to facts that do not come from the oracle itself.

Each pin_* function raises AssertionError when the oracle (the default one, or
the library handle `lib`) disagrees with a closed form, an invariant, a
library routine, or a count the pages print.  test_oracle_pins.py runs them on
the real oracle; test_oracle_mutants.py runs them on copies of the oracle with
one planted mistake each and checks that some pin fails.
"""
import json
import math
import os

import numpy as np
import torch

import oracle
from split_kv_paged_pa_amd import workloads as wl

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def widen(a):
    """float32 array, or bf16 bit patterns (uint16), as exact float64 values."""
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def dense_kv(kc, vc, bt, L, s):
    """Dense [Hkv, L, D] keys/values of sequence s, gathered with numpy fancy indexing
    from logical [blocks, Hkv, 16, D] keys and values."""
    nblk = -(-L // wl.BLOCK_SIZE)
    blocks = bt[s, :nblk]
    k = widen(kc[blocks]).transpose(1, 0, 2, 3).reshape(kc.shape[1], nblk * wl.BLOCK_SIZE, -1)
    v = widen(vc[blocks]).transpose(1, 0, 2, 3).reshape(vc.shape[1], nblk * wl.BLOCK_SIZE, -1)
    return k[:, :L], v[:, :L]


def sdpa_reference(q, kc, vc, bt, sl, scale):
    """Dense attention through torch's scaled_dot_product_attention in float64
    (logical [blocks, Hkv, 16, D] keys and values)."""
    S, Hq, D = q.shape
    Hkv = kc.shape[1]
    G = Hq // Hkv
    out = np.zeros((S, Hq, D))
    qw = widen(q)
    for s in range(S):
        L = int(sl[s])
        if L == 0:
            continue
        k, v = dense_kv(kc, vc, bt, L, s)
        kt = torch.from_numpy(np.ascontiguousarray(k)).repeat_interleave(G, dim=0)[None]
        vt = torch.from_numpy(np.ascontiguousarray(v)).repeat_interleave(G, dim=0)[None]
        qt = torch.from_numpy(qw[s])[None, :, None, :]
        o = torch.nn.functional.scaled_dot_product_attention(
            qt, kt, vt, scale=float(np.float64(np.float32(scale))))
        out[s] = o[0, :, 0, :].numpy()
    return out


def _run(batch, lib=None, **kw):
    q, kc, vc, bt, sl = batch.numpy()
    return oracle.decode(q, kc, vc, bt, sl, batch.spec.scale, dtype=batch.spec.dtype, lib=lib, **kw)


def _decode(q, k, v, bt, sl, spec, lib=None):
    """The oracle on logical [blocks, Hkv, 16, D] keys and values, stored into the
    cache layout by the generator's pack_kv first."""
    kc, vc = wl.pack_kv(k, v)
    return oracle.decode(q, kc, vc, bt, sl, spec.scale, dtype=spec.dtype, lib=lib)


def pin_single_token(lib=None):
    """L = 1: the softmax has one term, so the output is that token's value row exactly."""
    for dtype in ("f32", "bf16"):
        spec = wl.custom("one", 11, dtype, 6, 2, 64, [1, 1, 1], num_blocks=9)
        b = wl.generate(spec)
        q, kc, vc, bt, sl = b.numpy_logical()
        out = _run(b, lib)
        for s in range(3):
            for h in range(6):
                expect = widen(vc[bt[s, 0], h // 3, 0])
                assert np.array_equal(out[s, h], expect), f"L=1 {dtype} s={s} h={h}"


def pin_uniform_keys(lib=None):
    """All keys equal (or q = 0): every weight is the same, so the output is the
    plain mean of the value rows of the sequence."""
    for zero_q in (False, True):
        spec = wl.custom("uniform", 12, "bf16", 8, 2, 64, [37, 16, 300], num_blocks=40)
        b = wl.generate(spec)
        q, kc, vc, bt, sl = b.numpy_logical()
        q = q.copy()
        if zero_q:
            q[:] = 0
        else:
            kc[np.isfinite(widen(kc))] = kc[bt[0, 0], 0, 0, 0]  # one bf16 value everywhere finite
        out = _decode(q, kc, vc, bt, sl, spec, lib)
        for s in range(3):
            L = int(sl[s])
            _, v = dense_kv(kc, vc, bt, L, s)
            for h in range(8):
                expect = v[h // 4].mean(axis=0)
                assert np.max(np.abs(out[s, h] - expect)) <= 1e-13, f"mean of V, s={s} h={h}"


def pin_positional_values(lib=None):
    """Identical keys and v_t = t * e0 in float32: the output's first element is
    (L - 1) / 2 exactly and the rest are 0.  Pins the token order of the block
    gather and the exclusion of the NaN slots past the end of the sequence."""
    lens = [1, 15, 16, 17, 100, 333]
    spec = wl.custom("positional", 13, "f32", 4, 4, 64, lens, num_blocks=64)
    b = wl.generate(spec)
    q, kc, vc, bt, sl = b.numpy_logical()
    for s, L in enumerate(lens):
        for t in range(L):
            blk, r = bt[s, t // 16], t % 16
            kc[blk, :, r, :] = 0.5
            vc[blk, :, r, :] = 0.0
            vc[blk, :, r, 0] = float(t)
    out = _decode(q, kc, vc, bt, sl, spec, lib)
    for s, L in enumerate(lens):
        assert np.all(out[s, :, 0] == (L - 1) / 2), f"positional mean, L={L}"
        assert np.all(out[s, :, 1:] == 0.0), f"positional rest, L={L}"


def pin_closed_form(lib=None):
    """Two tokens with softmax weights 1/4 and 3/4 (tests/golden/closed_form_two_tokens.json)."""
    with open(os.path.join(GOLDEN, "closed_form_two_tokens.json")) as f:
        g = json.load(f)
    D = g["head_dim"]
    spec = wl.custom("closed", 14, "f32", 1, 1, D, [2], num_blocks=2, scale=g["scale"])
    b = wl.generate(spec)
    q, kc, vc, bt, sl = b.numpy_logical()
    q = q.copy()
    q[:] = 0
    q[0, 0, 0] = 1.0
    blk = bt[0, 0]
    kc[blk, 0, :2, :] = 0
    kc[blk, 0, 1, 0] = np.float32(8.0 * math.log(3.0))
    assert abs(float(kc[blk, 0, 1, 0]) - g["k1_coefficient_float32"]) < 1e-6
    vc[blk, 0, :2, :] = 0
    vc[blk, 0, 0, 0] = 4.0
    vc[blk, 0, 1, 1] = 4.0
    out = _decode(q, kc, vc, bt, sl, spec, lib)[0, 0]
    expect = np.zeros(D)
    expect[0] = g["expected_out"]["0"]
    expect[1] = g["expected_out"]["1"]
    assert np.max(np.abs(out - expect)) <= g["abs_tolerance"], f"closed form {out[:3]}"


def pin_head_mapping(lib=None):
    """Values of kv head k all equal k + 1: query head h must return h // G + 1."""
    spec = wl.custom("heads", 15, "bf16", 12, 3, 64, [50, 7], num_blocks=16)
    b = wl.generate(spec)
    q, kc, vc, bt, sl = b.numpy_logical()
    vals = widen(vc)
    for k in range(3):
        fin = np.isfinite(vals[:, k])
        sub = vc[:, k]
        sub[fin] = np.array([k + 1], np.float32).view(np.uint32)[0] >> 16
    out = _decode(q, kc, vc, bt, sl, spec, lib)
    for h in range(12):
        assert np.max(np.abs(out[:, h, :] - (h // 4 + 1))) <= 1e-14, f"head mapping h={h}"


def pin_dense_library(lib=None):
    """Ragged GQA batch (with NaN poison) against torch's dense float64 attention."""
    for dtype, D, Hq, Hkv in (("f32", 64, 8, 2), ("bf16", 128, 10, 2), ("bf16", 64, 4, 4)):
        spec = wl.custom("dense", 16, dtype, Hq, Hkv, D, [1, 15, 16, 17, 250, 513, 0], num_blocks=80)
        b = wl.generate(spec)
        q, kc, vc, bt, sl = b.numpy_logical()
        out = _run(b, lib)
        ref = sdpa_reference(q, kc, vc, bt, sl, spec.scale)
        assert np.all(np.isfinite(out)), "non-finite output"
        assert np.max(np.abs(out - ref)) <= 1e-12, f"dense mismatch {np.max(np.abs(out - ref))}"


def pin_outlier_stability(lib=None):
    """Keys with x40 outlier rows push logits far past ln(FLT_MAX); the output must
    stay finite and equal the dense library result."""
    spec = wl.custom("outliers", 17, "bf16", 8, 1, 128, [700, 65], num_blocks=60,
                     outlier_frac=0.05, outlier_mult=40.0)
    b = wl.generate(spec)
    q, kc, vc, bt, sl = b.numpy_logical()
    qw = widen(q)
    top = max(float(np.max(dense_kv(kc, vc, bt, int(sl[s]), s)[0][0] @ qw[s].T)) for s in range(2))
    assert top * spec.scale > math.log(np.finfo(np.float32).max), "test input too mild"
    out = _run(b, lib)
    ref = sdpa_reference(q, kc, vc, bt, sl, spec.scale)
    assert np.all(np.isfinite(out))
    assert np.max(np.abs(out - ref)) <= 1e-12


def pin_relabel_and_linearity(lib=None):
    """Renaming physical blocks (pool permuted, table rewritten) changes nothing,
    bit for bit; doubling V doubles the output, bit for bit."""
    spec = wl.custom("relabel", 18, "bf16", 4, 2, 64, [90, 33], num_blocks=20)
    b = wl.generate(spec)
    q, kc, vc, bt, sl = b.numpy()
    base = _run(b, lib)
    perm = np.random.default_rng(0).permutation(kc.shape[0])
    inv = np.argsort(perm)
    kc2, vc2 = np.ascontiguousarray(kc[perm]), np.ascontiguousarray(vc[perm])
    bt2 = np.where(bt >= 0, inv[np.maximum(bt, 0)], -1).astype(np.int32)
    moved = oracle.decode(q, kc2, vc2, bt2, sl, spec.scale, dtype="bf16", lib=lib)
    assert np.array_equal(base, moved), "block relabelling changed the output"
    v2 = (widen(vc) * 2).astype(np.float32).view(np.uint32)
    vc3 = (v2 >> 16).astype(np.uint16)
    doubled = oracle.decode(q, kc, vc3, bt, sl, spec.scale, dtype="bf16", lib=lib)
    assert np.array_equal(doubled, 2 * base), "doubling V did not double the output"


def pin_partitioned_equals_full(lib=None):
    """Phase 1 + Phase 2 at several partition sizes equals the one-pass softmax
    to 1e-12; with one partition (P >= L) the merge returns o_0 unchanged."""
    spec = wl.custom("parts", 19, "bf16", 8, 2, 64, [1, 16, 17, 511, 512, 513, 1500, 0],
                     num_blocks=300, outlier_frac=0.01, outlier_mult=20.0)
    b = wl.generate(spec)
    q, kc, vc, bt, sl = b.numpy()
    full = oracle.decode(q, kc, vc, bt, sl, spec.scale, dtype="bf16", lib=lib)
    for P in (16, 512, 1024, 2048):
        tmp, es, ml = oracle.partials(q, kc, vc, bt, sl, spec.scale, P, dtype="bf16", lib=lib)
        merged = oracle.merge(tmp, es, ml, sl, P, lib=lib)
        assert np.max(np.abs(merged - full)) <= 1e-12, f"P={P}"
        for s, L in enumerate(sl):
            n = oracle.num_partitions(L, P)
            assert np.all(np.isfinite(ml[s, :, :n])) and np.all(np.isnan(ml[s, :, n:])), f"P={P}"
    tmp, es, ml = oracle.partials(q, kc, vc, bt, sl, spec.scale, 2048, dtype="bf16", lib=lib)
    merged = oracle.merge(tmp, es, ml, sl, 2048, lib=lib)
    for s, L in enumerate(sl):
        if L:
            assert np.array_equal(merged[s], tmp[s, :, 0]), "single partition must pass through"


def pin_partition_statistics(lib=None):
    """Each partition's max logit and exp-sum match the dense logits of its token
    range, and its partial output is that range's own softmax average."""
    spec = wl.custom("stats", 20, "f32", 4, 2, 64, [700], num_blocks=50)
    b = wl.generate(spec)
    q, kc, vc, bt, sl = b.numpy()
    P = 256
    tmp, es, ml = oracle.partials(q, kc, vc, bt, sl, spec.scale, P, dtype="f32", lib=lib)
    _, kl, vl, _, _ = b.numpy_logical()
    k, v = dense_kv(kl, vl, bt, 700, 0)
    qw = widen(q)[0]
    sc = float(np.float32(spec.scale))
    for h in range(4):
        z = sc * (k[h // 2] @ qw[h])
        for p in range(3):
            zz = z[p * P:(p + 1) * P]
            assert abs(ml[0, h, p] - zz.max()) <= 1e-12
            w = np.exp(zz - zz.max())
            assert abs(es[0, h, p] - w.sum()) <= 1e-10 * w.sum()
            o = (w[:, None] * v[h // 2][p * P:(p + 1) * P]).sum(0) / w.sum()
            assert np.max(np.abs(tmp[0, h, p] - o)) <= 1e-12


def pin_page_counts(lib=None):
    """One 100000-token sequence: 6250 blocks, 98 partitions of 1024 and 196 of 512
    (tests/golden/page_counts.json)."""
    with open(os.path.join(GOLDEN, "page_counts.json")) as f:
        g = json.load(f)
    L = g["tokens"]
    spec = wl.custom("pagecounts", 21, "bf16", 1, 1, 64, [L], num_blocks=g["blocks"])
    b = wl.generate(spec, poison=True)
    q, kc, vc, bt, sl = b.numpy()
    _, kl, vl, _, _ = b.numpy_logical()
    assert int(np.sum(bt >= 0)) == g["blocks"]
    for P, n in g["partitions"].items():
        tmp, es, ml = oracle.partials(q, kc, vc, bt, sl, spec.scale, int(P), dtype="bf16",
                                      max_partitions=n + 2, lib=lib)
        assert int(np.sum(np.isfinite(ml[0, 0]))) == n, f"P={P}"
        last = g["last_partition_tokens"][P]
        k, v = dense_kv(kl, vl, bt, L, 0)
        z = float(np.float32(spec.scale)) * (k[0][-last:] @ widen(q)[0, 0])
        assert abs(ml[0, 0, n - 1] - z.max()) <= 1e-12, f"last partition of P={P}"


def pin_multi_query_causal(lib=None):
    """q_len query tokens per sequence against torch's dense float64 attention with an
    explicit mask: token j of a length-L sequence sees cache tokens 0 .. L - q_len + j
    (mask row j = tril with diagonal offset L - q_len); a token that sees nothing is
    a zero row."""
    for dtype, D, Hq, Hkv, q_len, lens in (("f32", 64, 8, 2, 3, [1, 2, 3, 17, 40, 0]),
                                            ("bf16", 128, 8, 8, 2, [16, 33, 300]),
                                            ("bf16", 64, 4, 1, 4, [5, 64, 129])):
        spec = wl.custom("multiq", 22, dtype, Hq, Hkv, D, lens)
        b = wl.generate(spec)
        q1, kc, vc, bt, sl = b.numpy()
        _, kl, vl, _, _ = b.numpy_logical()
        S = spec.num_seqs
        rng = np.random.default_rng(5)
        qf = rng.standard_normal((S, q_len, Hq, D)).astype(np.float32)
        q = qf if dtype == "f32" else (qf.view(np.uint32) >> 16).astype(np.uint16)
        out = oracle.decode_q(q, kc, vc, bt, sl, spec.scale, dtype=dtype, lib=lib)
        qw = widen(q)
        G = Hq // Hkv
        for s_ in range(S):
            L = int(sl[s_])
            ref = np.zeros((q_len, Hq, D))
            if L > 0:
                k, v = dense_kv(kl, vl, bt, L, s_)
                mask = torch.ones(q_len, L, dtype=torch.bool).tril(diagonal=L - q_len)
                kt = torch.from_numpy(np.ascontiguousarray(k)).repeat_interleave(G, dim=0)[None]
                vt = torch.from_numpy(np.ascontiguousarray(v)).repeat_interleave(G, dim=0)[None]
                qt = torch.from_numpy(np.ascontiguousarray(qw[s_].transpose(1, 0, 2)))[None]
                o = torch.nn.functional.scaled_dot_product_attention(
                    qt, kt, vt, attn_mask=mask, scale=float(np.float64(np.float32(spec.scale))))
                ref = o[0].numpy().transpose(1, 0, 2)
                ref = np.where(mask.any(dim=1).numpy()[:, None, None], ref, 0.0)
            assert np.max(np.abs(out[s_] - ref)) <= 1e-12, f"multi-query {dtype} s={s_} L={L}"


ALL_PINS = [pin_single_token, pin_uniform_keys, pin_positional_values, pin_closed_form,
            pin_head_mapping, pin_dense_library, pin_outlier_stability, pin_relabel_and_linearity,
            pin_partitioned_equals_full, pin_partition_statistics, pin_page_counts,
            pin_multi_query_causal]
