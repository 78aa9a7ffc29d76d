"""Helpers for the GPU parity tests: move a generated batch to the GPU, run the
HIP path through the Python binding of the C ABI, and compare with the oracle.

Tolerances (element by element, the oracle in float64 as the reference r):
  float32 inputs:  |gpu - r| <= 1e-5
  bf16 inputs:     |gpu - r| <= 2e-2 + 1e-2 * |r|
"""
import numpy as np
import torch

import oracle
import split_kv_paged_pa_amd as pa
from split_kv_paged_pa_amd import workloads as wl


def require_gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    pa.load_library()


class DeviceBatch:
    def __init__(self, batch: wl.Batch, device="cuda"):
        self.batch = batch
        self.spec = batch.spec
        self.query = batch.query.to(device)
        self.key_cache = batch.key_cache.to(device)
        self.value_cache = batch.value_cache.to(device)
        self.block_tables = batch.block_tables.to(device)
        self.seq_lens = batch.seq_lens.to(device)
        self.max_seq_len = batch.spec.max_seq_len

    def args(self):
        return (self.query, self.key_cache, self.value_cache, self.block_tables, self.seq_lens,
                self.spec.scale, self.max_seq_len)

    def new_out(self):
        return torch.full_like(self.query, float("nan"))

    def run_v1(self):
        out = self.new_out()
        pa.pa_decode_v1(out, *self.args())
        return out

    def workspace(self, P, poison=True):
        """A workspace for partition size P (0: the library's choice, sized with the
        value pa_select_partition_size returns)."""
        if P == 0:
            P = pa.pa_select_partition_size(self.spec.num_seqs, self.spec.num_kv_heads,
                                            self.max_seq_len)
        ws = pa.new_workspace(self.spec.num_seqs, self.spec.num_q_heads, self.spec.head_dim,
                              self.max_seq_len, P)
        if poison:
            ws.view(torch.uint8).fill_(0xFF)  # all-ones float32 words are NaN
            pa.pa_workspace_init(ws)          # the counter header must start at zero
        return ws

    def run_v2(self, P, ws=None):
        out = self.new_out()
        ws = self.workspace(P) if ws is None else ws
        pa.pa_decode_v2(out, *self.args(), P, ws)
        return out

    def run(self, variant, P=None):
        return self.run_v1() if variant == "v1" else self.run_v2(P)


def oracle_out(batch: wl.Batch, rows=None):
    q, kc, vc, bt, sl = batch.numpy()
    return oracle.decode(q, kc, vc, bt, sl, batch.spec.scale, dtype=batch.spec.dtype, rows=rows)


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float64).numpy()


def assert_close(gpu: np.ndarray, ref: np.ndarray, dtype: str, what: str):
    assert gpu.shape == ref.shape, (gpu.shape, ref.shape)
    if gpu.size == 0:
        return 0.0
    assert np.all(np.isfinite(gpu)), f"{what}: non-finite GPU output"
    err = np.abs(gpu - ref)
    bound = 1e-5 if dtype == "f32" else 2e-2 + 1e-2 * np.abs(ref)
    bad = err > bound
    rel = err / np.maximum(np.abs(ref), 1e-30)
    msg = (f"{what}: max abs err {err.max():.3e}, max rel err {rel.max():.3e}, "
           f"{int(bad.sum())} of {bad.size} out of tolerance")
    if bad.any():
        idx = np.unravel_index(np.argmax(err - bound), err.shape)
        msg += f"; worst at {idx}: gpu {gpu[idx]!r} ref {ref[idx]!r}"
    assert not bad.any(), msg
    return float(err.max())


def sample_rows(spec: wl.Spec, n: int, seed: int = 0):
    """n (s, h) pairs covering every sequence at least once."""
    rng = np.random.default_rng(seed)
    S, Hq = spec.num_seqs, spec.num_q_heads
    rows = [(s, int(rng.integers(Hq))) for s in range(S)]
    while len(rows) < max(n, S):
        rows.append((int(rng.integers(S)), int(rng.integers(Hq))))
    return np.array(sorted(set(rows)), np.int32)
