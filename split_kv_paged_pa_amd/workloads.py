"""Seeded synthetic decode batches for paged attention.

This module only draws random numbers and lays them out in the paged format;
it holds none of the attention arithmetic, so the HIP path and the CPU oracle
can both be fed from it without sharing any computation.

Recipe (every draw is reproducible from (config seed, stream, chunk)):
  - query, keys and values ~ N(0, 1), drawn in float32 with numpy's PCG64 and
    rounded to nearest-even into the config dtype (torch's float->bf16 cast);
  - keys and values are drawn per *logical* 16-token block, in sequence order,
    in fixed chunks of logical blocks, each chunk from its own seed
    (root, stream, chunk index), so the values do not depend on the thread
    count nor on where the blocks land in the pool;
  - physical placement: one seeded permutation of the pool, handed out to the
    sequences in order as consecutive slices (a fragmented, random block
    table); unused table entries are -1;
  - optional key outliers: each (token slot, kv head) key row is chosen with
    probability `outlier_frac` and multiplied by `outlier_mult` in float32
    before rounding;
  - poison (default on): unused pool blocks and the slots past the end of each
    sequence's last block are NaN, so any read of them shows up in the output.

Cache layout (the split layout of paged caches): keys
[num_blocks][num_kv_heads][head_dim / x][16][x] with x = 16 bytes of values
(8 bf16, 4 float32), values [num_blocks][num_kv_heads][head_dim][16].  The
random draws are made per token row ([block][kv head][slot][d], "logical"
order) and then stored in that layout; pack_kv / unpack_kv convert between the
two orders.

Streams: query 0, keys 1, values 2, block permutation 3, sequence lengths 4,
outlier rows 5, length order 6.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np
import torch

BLOCK_SIZE = 16
_CHUNK_BLOCKS = 64
_STREAM_Q, _STREAM_K, _STREAM_V, _STREAM_PERM, _STREAM_LENS, _STREAM_OUTLIER, _STREAM_ORDER = range(7)


def _rng(seed: int, *keys: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, *keys])))


@dataclass
class Spec:
    """Shape and distribution of one synthetic decode batch."""
    name: str
    seed: int
    dtype: str                      # "f32" or "bf16"
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    seq_lens: np.ndarray            # int32 [num_seqs]
    num_blocks: int                 # physical pool size
    scale: float
    partition_sizes: tuple = (512,)
    outlier_frac: float = 0.0
    outlier_mult: float = 1.0
    note: str = ""

    @property
    def num_seqs(self) -> int:
        return int(len(self.seq_lens))

    @property
    def max_seq_len(self) -> int:
        return int(max(self.seq_lens)) if len(self.seq_lens) else 0

    @property
    def max_blocks_per_seq(self) -> int:
        return max(1, -(-self.max_seq_len // BLOCK_SIZE))

    @property
    def elem_size(self) -> int:
        return 4 if self.dtype == "f32" else 2

    @property
    def kv_bytes(self) -> int:
        """Bytes of K and V rows of the actual tokens (each read once)."""
        return int(np.sum(self.seq_lens, dtype=np.int64)) * self.num_kv_heads * self.head_dim * \
            self.elem_size * 2


def key_group(elem_size: int) -> int:
    """Values per 16-byte group of the key layout."""
    return 16 // elem_size


def _swap(a, i, j):
    return a.transpose(i, j) if isinstance(a, torch.Tensor) else a.swapaxes(i, j)


def pack_kv(k, v, elem_size: int | None = None):
    """Logical [num_blocks, Hkv, 16, D] keys and values (numpy or torch, bf16 as
    uint16 in numpy) -> contiguous caches in the split layout:
    keys [num_blocks, Hkv, D / x, 16, x], values [num_blocks, Hkv, D, 16].
    x follows the arrays' element size unless elem_size (of the dtype the
    caches will be stored in) is given."""
    nb, H, B, D = k.shape
    if elem_size is None:
        elem_size = k.element_size() if isinstance(k, torch.Tensor) else k.itemsize
    x = key_group(elem_size)
    kc = _swap(k.reshape(nb, H, B, D // x, x), 2, 3)
    vc = _swap(v, 2, 3)
    if isinstance(k, torch.Tensor):
        return kc.contiguous(), vc.contiguous()
    return np.ascontiguousarray(kc), np.ascontiguousarray(vc)


def unpack_kv(kc, vc):
    """Inverse of pack_kv: logical [num_blocks, Hkv, 16, D] copies."""
    nb, H, Dx, B, x = kc.shape
    k = _swap(kc, 2, 3).reshape(nb, H, B, Dx * x)
    v = _swap(vc, 2, 3)
    if isinstance(kc, torch.Tensor):
        return k.contiguous(), v.contiguous()
    return np.ascontiguousarray(k), np.ascontiguousarray(v)


def _inv_sqrt(d: int) -> float:
    return float(np.float32(1.0 / math.sqrt(d)))


def config(name: str) -> Spec:
    """The five named decode workloads."""
    if name == "tiny_f32_2k":
        return Spec(name, 1, "f32", 8, 2, 64, np.array([2048], np.int32), 256, _inv_sqrt(64),
                    (512,), note="1 seq x 2048 tokens, 8/2 heads, D 64, fp32, 256-block pool")
    if name == "long_100k_gqa8":
        return Spec(name, 2, "bf16", 32, 4, 128, np.array([100000], np.int32), 8192,
                    _inv_sqrt(128), (512, 1024),
                    note="1 seq x 100000 tokens (6250 blocks in an 8192-block pool), 32/4 heads, D 128")
    if name == "batch16_1k_32k":
        lens = _rng(3, _STREAM_LENS).integers(1024, 32768, size=16, endpoint=True).astype(np.int32)
        return Spec(name, 3, "bf16", 32, 8, 128, lens, 40000, _inv_sqrt(128), (1024, 512),
                    note="16 seqs, lengths U[1024, 32768], 32/8 heads, 40000-block shared pool")
    if name == "batch64_mixed_outliers":
        r = _rng(4, _STREAM_LENS)
        short = r.integers(128, 4096, size=48, endpoint=True)
        long_ = r.integers(32768, 131072, size=16, endpoint=True)
        lens = np.concatenate([short, long_])
        lens = lens[_rng(4, _STREAM_ORDER).permutation(64)].astype(np.int32)
        used = int(np.sum(-(-lens.astype(np.int64) // BLOCK_SIZE)))
        return Spec(name, 4, "bf16", 64, 8, 128, lens, int(math.ceil(1.1 * used)), _inv_sqrt(128),
                    (1024,), outlier_frac=0.01, outlier_mult=20.0,
                    note="64 seqs: 48 of U[128, 4096], 16 of U[32768, 131072], shuffled; 64/8 heads; "
                         "1% of key rows x20")
    if name == "batch8_131k_gqa5":
        return Spec(name, 5, "bf16", 40, 8, 128, np.full(8, 131072, np.int32), 70000,
                    _inv_sqrt(128), (1024,),
                    note="8 seqs x 131072 tokens, 40/8 heads (GQA 5), 70000-block pool")
    raise KeyError(name)


CONFIG_NAMES = ("tiny_f32_2k", "long_100k_gqa8", "batch16_1k_32k", "batch64_mixed_outliers",
                "batch8_131k_gqa5")


def custom(name: str, seed: int, dtype: str, num_q_heads: int, num_kv_heads: int, head_dim: int,
           seq_lens, num_blocks: int | None = None, scale: float | None = None,
           partition_sizes=(512,), outlier_frac: float = 0.0, outlier_mult: float = 1.0) -> Spec:
    """A shrunk or edge-case batch with the same recipe."""
    lens = np.asarray(seq_lens, np.int32).reshape(-1)
    used = int(np.sum(-(-lens.astype(np.int64) // BLOCK_SIZE)))
    if num_blocks is None:
        num_blocks = max(1, used + used // 4 + 3)
    if scale is None:
        scale = _inv_sqrt(head_dim)
    return Spec(name, seed, dtype, num_q_heads, num_kv_heads, head_dim, lens, num_blocks, scale,
                tuple(partition_sizes), outlier_frac, outlier_mult)


@dataclass
class Batch:
    """A generated batch: torch CPU tensors in the paged layout."""
    spec: Spec
    query: torch.Tensor          # [S, Hq, D]
    key_cache: torch.Tensor      # [num_blocks, Hkv, D / x, 16, x]
    value_cache: torch.Tensor    # [num_blocks, Hkv, D, 16]
    block_tables: torch.Tensor   # int32 [S, max_blocks_per_seq]
    seq_lens: torch.Tensor       # int32 [S]
    extras: dict = field(default_factory=dict)

    def numpy(self):
        """(query, key_cache, value_cache, block_tables, seq_lens) as numpy arrays;
        bf16 tensors come out as uint16 bit patterns."""
        return (to_numpy(self.query), to_numpy(self.key_cache), to_numpy(self.value_cache),
                self.block_tables.numpy(), self.seq_lens.numpy())

    def numpy_logical(self):
        """As numpy(), but keys and values as logical [num_blocks, Hkv, 16, D] copies."""
        q, kc, vc, bt, sl = self.numpy()
        k, v = unpack_kv(kc, vc)
        return q, k, v, bt, sl


def torch_dtype(dtype: str) -> torch.dtype:
    return {"f32": torch.float32, "bf16": torch.bfloat16}[dtype]


def to_numpy(t: torch.Tensor) -> np.ndarray:
    """CPU tensor -> numpy without copying; bf16 becomes its uint16 bit pattern."""
    t = t.contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def _workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def generate(spec: Spec, poison: bool = True, threads: int | None = None) -> Batch:
    S, Hq, Hkv, D = spec.num_seqs, spec.num_q_heads, spec.num_kv_heads, spec.head_dim
    tdt = torch_dtype(spec.dtype)
    lens = spec.seq_lens.astype(np.int64)
    nblk = -(-lens // BLOCK_SIZE)
    total = int(nblk.sum())
    if total > spec.num_blocks:
        raise ValueError(f"{spec.name}: {total} blocks needed, pool has {spec.num_blocks}")
    mb = spec.max_blocks_per_seq

    perm = _rng(spec.seed, _STREAM_PERM).permutation(spec.num_blocks)[:total]
    tables = np.full((S, mb), -1, np.int32)
    starts = np.concatenate([[0], np.cumsum(nblk)])
    for s in range(S):
        tables[s, :nblk[s]] = perm[starts[s]:starts[s + 1]]

    q = _rng(spec.seed, _STREAM_Q).standard_normal((S, Hq, D), dtype=np.float32)
    query = torch.from_numpy(q).to(tdt)

    fill = float("nan") if poison else 0.0
    x = key_group(spec.elem_size)
    kc = torch.full((spec.num_blocks, Hkv, D // x, BLOCK_SIZE, x), fill, dtype=tdt)
    vc = torch.full((spec.num_blocks, Hkv, D, BLOCK_SIZE), fill, dtype=tdt)
    perm_t = torch.from_numpy(perm.astype(np.int64))

    def fill_chunk(ci: int):
        b0 = ci * _CHUNK_BLOCKS
        b1 = min(total, b0 + _CHUNK_BLOCKS)
        n = b1 - b0
        k = _rng(spec.seed, _STREAM_K, ci).standard_normal((n, Hkv, BLOCK_SIZE, D), dtype=np.float32)
        v = _rng(spec.seed, _STREAM_V, ci).standard_normal((n, Hkv, BLOCK_SIZE, D), dtype=np.float32)
        if spec.outlier_frac > 0:
            rows = _rng(spec.seed, _STREAM_OUTLIER, ci).random((n, Hkv, BLOCK_SIZE)) < spec.outlier_frac
            k[rows] *= np.float32(spec.outlier_mult)
        idx = perm_t[b0:b1]
        ks, vs = pack_kv(k, v, spec.elem_size)
        kc[idx] = torch.from_numpy(ks).to(tdt)
        vc[idx] = torch.from_numpy(vs).to(tdt)

    nchunks = -(-total // _CHUNK_BLOCKS)
    with ThreadPoolExecutor(threads or _workers()) as ex:
        list(ex.map(fill_chunk, range(nchunks)))

    if poison:
        for s in range(S):
            r = int(lens[s] % BLOCK_SIZE)
            if r:
                last = int(tables[s, nblk[s] - 1])
                kc[last, :, :, r:, :] = float("nan")
                vc[last, :, :, r:] = float("nan")

    return Batch(spec, query, kc, vc, torch.from_numpy(tables),
                 torch.from_numpy(spec.seq_lens.astype(np.int32).copy()))
