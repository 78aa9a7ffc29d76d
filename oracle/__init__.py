"""CPU reference ("oracle") for paged single-query decode attention.

TEST INFRASTRUCTURE ONLY: imported by the test suite, the smoke check and the
CPU-baseline leg of the benchmark, never by the product path.  It shares no
code with the HIP library (split_kv_paged_pa_amd): the arithmetic is in
pa_oracle.c, computed in float64; this module only marshals numpy arrays.

Functions
  decode    full-softmax attention (the plain definition; V1 and V2 are both
            schedules of it)
  decode_q  the same for q_len query tokens per sequence, causal over the cache
  partials  the pages' Phase 1 per-partition statistics (m_p, s_p, o_p)
  merge     the pages' Phase 2 log-sum-exp merge of those partials

Every array argument is a C-contiguous numpy array.  Floating-point inputs are
float32, or bfloat16 carried as uint16 bit patterns (dtype="bf16").
Sources: commit pages 900ae0b (vllm/_custom_ops.py), 490ff98 (paged_attn.py)
and 15ef28e (paged_attention_v2_pytorch.py) of project_6; the header of
pa_oracle.c cites the passages each step follows.
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libpa_oracle.so")
_DTYPES = {"f32": (0, np.float32), "bf16": (1, np.uint16)}


_default = None


def load(path=None):
    """Open an oracle library (default: the one built from pa_oracle.c here) and
    return a ctypes handle with its signatures declared."""
    path = path or _LIB_PATH
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run `python oracle/build.py`")
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    I = ctypes.c_int
    lib.pa_oracle_decode.argtypes = [P, P, P, P, I, P, P, I, I, I, I, I, I, ctypes.c_float, P, I, I]
    lib.pa_oracle_decode.restype = I
    lib.pa_oracle_partials.argtypes = [P, P, P, P, P, P, I, P, P, I, I, I, I, I, I, ctypes.c_float,
                                       I, I, I]
    lib.pa_oracle_partials.restype = I
    lib.pa_oracle_merge.argtypes = [P, P, P, P, P, I, I, I, I, I]
    lib.pa_oracle_merge.restype = I
    lib.pa_oracle_decode_q.argtypes = [P, P, P, P, I, P, P, I, I, I, I, I, I, I, ctypes.c_float, I]
    lib.pa_oracle_decode_q.restype = I
    return lib


def _load(lib=None):
    global _default
    if lib is not None:
        return lib
    if _default is None:
        _default = load()
    return _default


def _ptr(a):
    return ctypes.c_void_p(a.ctypes.data)


def _check(name, a, dtype, ndim):
    if not isinstance(a, np.ndarray):
        raise TypeError(f"{name} must be a numpy array")
    if a.dtype != dtype:
        raise TypeError(f"{name} must have dtype {np.dtype(dtype).name}, got {a.dtype}")
    if a.ndim != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got shape {a.shape}")
    if not a.flags["C_CONTIGUOUS"]:
        raise ValueError(f"{name} must be C-contiguous")


def _problem(query, key_cache, value_cache, block_tables, seq_lens, dtype):
    if dtype not in _DTYPES:
        raise ValueError(f"dtype must be one of {sorted(_DTYPES)}")
    code, npdt = _DTYPES[dtype]
    _check("query", query, npdt, 3)
    _check("key_cache", key_cache, npdt, 5)
    _check("value_cache", value_cache, npdt, 4)
    _check("block_tables", block_tables, np.int32, 2)
    _check("seq_lens", seq_lens, np.int32, 1)
    S, Hq, D = query.shape
    # keys [blocks][Hkv][D / x][16][x] with x = 16 bytes of values; values [blocks][Hkv][D][16]
    nb, Hkv, Dx, B, x = key_cache.shape
    if x * np.dtype(npdt).itemsize != 16 or Dx * x != D or value_cache.shape != (nb, Hkv, D, B):
        raise ValueError("key/value cache shapes disagree with the query or the split layout")
    if block_tables.shape[0] != S or seq_lens.shape[0] != S:
        raise ValueError("block_tables / seq_lens rows must equal num_seqs")
    mb = block_tables.shape[1]
    if np.any(seq_lens > mb * B):
        raise ValueError("a seq_len exceeds max_blocks_per_seq * block_size")
    return code, S, Hq, Hkv, D, B, mb


def decode(query, key_cache, value_cache, block_tables, seq_lens, scale, dtype="f32",
           rows=None, threads=0, lib=None):
    """fp64 attention output: [S, Hq, D], or [len(rows), D] for rows = [(s, h), ...]."""
    lib = _load(lib)
    code, S, Hq, Hkv, D, B, mb = _problem(query, key_cache, value_cache, block_tables, seq_lens,
                                          dtype)
    if rows is None:
        out = np.empty((S, Hq, D), np.float64)
        rp, nr = None, 0
    else:
        r = np.ascontiguousarray(np.asarray(rows, dtype=np.int32).reshape(-1, 2))
        out = np.empty((r.shape[0], D), np.float64)
        rp, nr = _ptr(r), r.shape[0]
    rc = lib.pa_oracle_decode(_ptr(out), _ptr(query), _ptr(key_cache), _ptr(value_cache), code,
                              _ptr(block_tables), _ptr(seq_lens), S, Hq, Hkv, D, B, mb,
                              float(scale), rp, nr, int(threads))
    if rc:
        raise RuntimeError(f"pa_oracle_decode failed with code {rc}")
    return out


def decode_q(query, key_cache, value_cache, block_tables, seq_lens, scale, dtype="f32",
             threads=0, lib=None):
    """fp64 output [S, q_len, Hq, D] of q_len query tokens per sequence ([S, q_len, Hq, D]
    query): token j attends to cache tokens 0 .. L - q_len + j (zero row if none)."""
    lib = _load(lib)
    if not isinstance(query, np.ndarray) or query.ndim != 4:
        raise ValueError("query must be a [S, q_len, Hq, D] numpy array")
    S, q_len, Hq, D = query.shape
    code, _, _, Hkv, _, B, mb = _problem(query.reshape(S, q_len * Hq, D), key_cache, value_cache,
                                         block_tables, seq_lens, dtype)
    if Hq % Hkv:
        raise ValueError("num_q_heads must be a multiple of num_kv_heads")
    out = np.empty((S, q_len, Hq, D), np.float64)
    rc = lib.pa_oracle_decode_q(_ptr(out), _ptr(query), _ptr(key_cache), _ptr(value_cache), code,
                                _ptr(block_tables), _ptr(seq_lens), S, q_len, Hq, Hkv, D, B, mb,
                                float(scale), int(threads))
    if rc:
        raise RuntimeError(f"pa_oracle_decode_q failed with code {rc}")
    return out


def num_partitions(seq_len, partition_size):
    """ceil(L / P): partitions covering L tokens (0 for L == 0)."""
    return -(-int(seq_len) // int(partition_size)) if seq_len > 0 else 0


def partials(query, key_cache, value_cache, block_tables, seq_lens, scale, partition_size,
             dtype="f32", max_partitions=None, threads=0, lib=None):
    """Phase-1 partials (tmp_out [S,Hq,Pmax,D], exp_sums [S,Hq,Pmax], max_logits [S,Hq,Pmax])
    in float64; entries of partitions beyond ceil(L/P) are NaN."""
    lib = _load(lib)
    code, S, Hq, Hkv, D, B, mb = _problem(query, key_cache, value_cache, block_tables, seq_lens,
                                          dtype)
    if max_partitions is None:
        max_partitions = max([num_partitions(L, partition_size) for L in seq_lens] + [0])
    tmp = np.empty((S, Hq, max_partitions, D), np.float64)
    es = np.empty((S, Hq, max_partitions), np.float64)
    ml = np.empty((S, Hq, max_partitions), np.float64)
    rc = lib.pa_oracle_partials(_ptr(tmp), _ptr(es), _ptr(ml), _ptr(query), _ptr(key_cache),
                                _ptr(value_cache), code, _ptr(block_tables), _ptr(seq_lens), S, Hq,
                                Hkv, D, B, mb, float(scale), int(partition_size),
                                int(max_partitions), int(threads))
    if rc:
        raise RuntimeError(f"pa_oracle_partials failed with code {rc}")
    return tmp, es, ml


def merge(tmp_out, exp_sums, max_logits, seq_lens, partition_size, lib=None):
    """Phase-2 merge of float64 partials -> [S, Hq, D] float64."""
    lib = _load(lib)
    _check("tmp_out", tmp_out, np.float64, 4)
    _check("exp_sums", exp_sums, np.float64, 3)
    _check("max_logits", max_logits, np.float64, 3)
    _check("seq_lens", seq_lens, np.int32, 1)
    S, Hq, Pm, D = tmp_out.shape
    if exp_sums.shape != (S, Hq, Pm) or max_logits.shape != (S, Hq, Pm) or seq_lens.shape != (S,):
        raise ValueError("partials shapes disagree")
    out = np.empty((S, Hq, D), np.float64)
    rc = lib.pa_oracle_merge(_ptr(out), _ptr(tmp_out), _ptr(exp_sums), _ptr(max_logits),
                             _ptr(seq_lens), S, Hq, D, int(partition_size), Pm)
    if rc:
        raise RuntimeError(f"pa_oracle_merge failed with code {rc}")
    return out
