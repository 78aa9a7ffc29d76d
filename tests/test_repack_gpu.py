"""pa_cache_from_token_major on the GPU: token-major caches into the split
layout, compared bit for bit with the layout's definition (include/pa_decode.h:
K[t][d] at [..][d / x][t][d % x], V[t][d] at [..][d][t]), and a decode on the
repacked cache compared bit for bit with one on the cache it came from."""
import numpy as np
import pytest
import torch

import split_kv_paged_pa_amd as pa
from split_kv_paged_pa_amd import workloads as wl

pytestmark = pytest.mark.gpu


def _split_reference(k_tm, v_tm):
    nb, hkv, b, d = k_tm.shape
    x = pa.api.key_group(k_tm.dtype)
    k = k_tm.view(nb, hkv, b, d // x, x).permute(0, 1, 3, 2, 4).contiguous()
    v = v_tm.permute(0, 1, 3, 2).contiguous()
    return k, v


def _bits(t):
    t = t.cpu().contiguous()
    return t.view(torch.int16 if t.element_size() == 2 else torch.int32).numpy()


@pytest.mark.parametrize("dtype,nb,hkv,d", [(torch.bfloat16, 37, 4, 128), (torch.float32, 5, 3, 64),
                                            (torch.bfloat16, 1, 1, 8), (torch.float32, 9, 2, 512)])
def test_repack_matches_layout_definition(dtype, nb, hkv, d):
    print(f"[case] repack {dtype} nb={nb} hkv={hkv} d={d}", flush=True)
    g = torch.Generator().manual_seed(11 + nb)
    k_tm = torch.randn(nb, hkv, 16, d, generator=g).to(dtype)
    v_tm = torch.randn(nb, hkv, 16, d, generator=g).to(dtype)
    k_ref, v_ref = _split_reference(k_tm, v_tm)
    k, v = pa.split_layout(k_tm.cuda(), v_tm.cuda())
    torch.cuda.synchronize()
    assert np.array_equal(_bits(k), _bits(k_ref))
    assert np.array_equal(_bits(v), _bits(v_ref))


def test_repack_one_cache_at_a_time():
    print("[case] repack keys only / values only", flush=True)
    g = torch.Generator().manual_seed(5)
    k_tm = torch.randn(6, 2, 16, 64, generator=g).to(torch.bfloat16)
    v_tm = torch.randn(6, 2, 16, 64, generator=g).to(torch.bfloat16)
    k_ref, v_ref = _split_reference(k_tm, v_tm)
    k = torch.full(k_ref.shape, 7.0, dtype=torch.bfloat16, device="cuda")
    v = torch.full(v_ref.shape, 7.0, dtype=torch.bfloat16, device="cuda")
    pa.pa_cache_from_token_major(k, None, k_tm.cuda(), None)
    torch.cuda.synchronize()
    assert np.array_equal(_bits(k), _bits(k_ref))
    assert bool((v.cpu() == 7.0).all())  # untouched
    pa.pa_cache_from_token_major(None, v, None, v_tm.cuda())
    torch.cuda.synchronize()
    assert np.array_equal(_bits(v), _bits(v_ref))


def test_repacked_cache_decodes_identically():
    """A generated split-layout cache, written out token-major and repacked,
    comes back bit for bit, and a V2 decode on it is bitwise the same."""
    spec = wl.custom("repack_roundtrip", 321, "bf16", 16, 4, 128, [40, 1000, 4097])
    b = wl.generate(spec)
    print("[case] repack round trip on", spec.name, flush=True)
    kc, vc = b.key_cache, b.value_cache  # split layout, CPU
    nb, hkv, dx, blk, x = kc.shape
    k_tm = kc.permute(0, 1, 3, 2, 4).reshape(nb, hkv, blk, dx * x).contiguous()
    v_tm = vc.permute(0, 1, 3, 2).contiguous()
    k2, v2 = pa.split_layout(k_tm.cuda(), v_tm.cuda())
    torch.cuda.synchronize()
    assert np.array_equal(_bits(k2), _bits(kc))
    assert np.array_equal(_bits(v2), _bits(vc))
    q = b.query.cuda()
    bt, sl = b.block_tables.cuda(), b.seq_lens.cuda()
    L = int(b.seq_lens.max())
    outs = []
    for k_, v_ in ((kc.cuda(), vc.cuda()), (k2, v2)):
        out = torch.empty_like(q)
        ws = pa.new_workspace(spec.num_seqs, spec.num_q_heads, spec.head_dim, L, 512)
        pa.pa_workspace_init(ws)
        pa.pa_decode_v2(out, q, k_, v_, bt, sl, spec.scale, L, 512, ws)
        outs.append(out)
    torch.cuda.synchronize()
    assert np.array_equal(_bits(outs[0]), _bits(outs[1]))
