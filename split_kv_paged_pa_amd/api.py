"""Python binding of libpa_decode.so (include/pa_decode.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI.  torch supplies device memory and streams.  There is
no fallback: if the library is missing or the tensors are not on a GPU, the
call raises.

Functions keep the C names: pa_decode_v1, pa_decode_v2, pa_decode,
pa_decode_v2_partials, pa_decode_v2_reduce, pa_decode_v2_groups,
pa_decode_v2_reduce_entries, pa_decode_v2_noalloc, pa_workspace_size,
pa_workspace_layout, pa_workspace_init, pa_select_partition_size, pa_select_v2, pa_select_v2_auto,
pa_decode_auto, pa_decode_v2_single, pa_decode_v1_q, pa_decode_v2_q, pa_prefill_v1,
pa_prefill_v2, pa_select_q_kernel, pa_status_string.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpa_decode.so")
BLOCK_SIZE = 16

PA_OK = 0
WORKSPACE_HEADER_BYTES = 16384  # PA_WORKSPACE_HEADER_BYTES
_DTYPE_CODE = {torch.float32: 0, torch.bfloat16: 1}
_lib = None


class PagedAttentionError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {pa_status_string(status)} (status {status})")
        self.status = status


def load_library():
    """Open libpa_decode.so (built by split_kv_paged_pa_amd/build.py); raises if absent."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build it with `python split_kv_paged_pa_amd/build.py` "
            "(there is no non-HIP fallback)")
    lib = ctypes.CDLL(LIB_PATH)
    P, I, F, Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    common = [P, P, P, P, P, I, I, I, I, I, I, I, I, F, I]
    lib.pa_status_string.argtypes = [I]
    lib.pa_status_string.restype = ctypes.c_char_p
    lib.pa_workspace_size.argtypes = [I, I, I, I, I]
    lib.pa_workspace_size.restype = Z
    lib.pa_workspace_layout.argtypes = [I, I, I, I, I, ctypes.POINTER(Z), ctypes.POINTER(Z),
                                        ctypes.POINTER(Z), ctypes.POINTER(I)]
    lib.pa_workspace_layout.restype = I
    lib.pa_workspace_init.argtypes = [P, Z, P]
    lib.pa_workspace_init.restype = I
    lib.pa_select_v2.argtypes = [I, I, I, I]
    lib.pa_select_v2.restype = I
    lib.pa_select_partition_size.argtypes = [I, I, I]
    lib.pa_select_partition_size.restype = I
    lib.pa_select_v2_auto.argtypes = [I, I, I, I]
    lib.pa_select_v2_auto.restype = I
    lib.pa_decode_auto.argtypes = [P] + common + [I, P, Z, P]
    lib.pa_decode_auto.restype = I
    lib.pa_decode_v1.argtypes = [P] + common + [P]
    lib.pa_decode_v1.restype = I
    common_q = common[:6] + [I] + common[6:]  # q_len after num_seqs
    lib.pa_decode_v1_q.argtypes = [P] + common_q + [P]
    lib.pa_decode_v1_q.restype = I
    lib.pa_decode_v2_q.argtypes = [P] + common_q + [I, P, Z, P]
    lib.pa_decode_v2_q.restype = I
    lib.pa_select_q_kernel.argtypes = [I, I, I, I, I, I, I, I]
    lib.pa_select_q_kernel.restype = I
    lib.pa_prefill_v1.argtypes = [P] + common_q + [I, P]
    lib.pa_prefill_v1.restype = I
    lib.pa_prefill_v2.argtypes = [P] + common_q + [I, P, Z, I, P]
    lib.pa_prefill_v2.restype = I
    lib.pa_decode_v2.argtypes = [P] + common + [I, P, Z, P]
    lib.pa_decode_v2.restype = I
    lib.pa_decode_v2_single.argtypes = [P] + common + [I, P, Z, P]
    lib.pa_decode_v2_single.restype = I
    lib.pa_decode.argtypes = [P] + common + [I, P, Z, P]
    lib.pa_decode.restype = I
    lib.pa_decode_v2_partials.argtypes = common + [I, P, Z, P]
    lib.pa_decode_v2_partials.restype = I
    lib.pa_decode_v2_reduce.argtypes = [P, P, I, I, I, I, I, I, P, Z, P]
    lib.pa_decode_v2_reduce.restype = I
    lib.pa_decode_v2_noalloc.argtypes = [P] + common + [I, P]
    lib.pa_decode_v2_noalloc.restype = I
    lib.pa_decode_v2_groups.argtypes = common + [I, P, Z, ctypes.POINTER(I), P]
    lib.pa_decode_v2_groups.restype = I
    lib.pa_decode_v2_reduce_entries.argtypes = [P, P, I, I, I, I, I, I, I, P, Z, P]
    lib.pa_decode_v2_reduce_entries.restype = I
    lib.pa_cache_from_token_major.argtypes = [P, P, P, P, I, I, I, I, I, P]
    lib.pa_cache_from_token_major.restype = I
    _lib = lib
    return lib


def pa_cache_from_token_major(key_out, value_out, key_in, value_in, stream=None):
    """Token-major caches [blocks, Hkv, 16, D] into the split layout the kernels
    read: key_out [blocks, Hkv, D/x, 16, x], value_out [blocks, Hkv, D, 16] (same
    dtype, x = key_group(dtype)).  Either (out, in) pair may be None to skip that
    cache.  Bit-exact data movement on the GPU."""
    ref = key_in if key_in is not None else value_in
    if ref is None:
        raise ValueError("at least one of key_in / value_in is needed")
    if ref.dtype not in _DTYPE_CODE or ref.dim() != 4 or ref.shape[2] != 16:
        raise ValueError("token-major caches [blocks, Hkv, 16, D] of float32 or bfloat16 expected")
    nb, Hkv, B, D = ref.shape
    x = key_group(ref.dtype)
    args = []
    for name, out, inp, shape in (("key", key_out, key_in, (nb, Hkv, D // x, B, x)),
                                  ("value", value_out, value_in, (nb, Hkv, D, B))):
        if (out is None) != (inp is None):
            raise ValueError(f"{name}_out and {name}_in go together")
        if inp is None:
            args.append((ctypes.c_void_p(0), ctypes.c_void_p(0)))
            continue
        if tuple(inp.shape) != (nb, Hkv, B, D) or tuple(out.shape) != shape:
            raise ValueError(f"{name}: token-major {(nb, Hkv, B, D)} in, split layout {shape} out expected")
        args.append((_dev(f"{name}_out", out, ref.dtype), _dev(f"{name}_in", inp, ref.dtype)))
    _check(load_library().pa_cache_from_token_major(args[0][0], args[1][0], args[0][1], args[1][1], nb,
                                                    Hkv, D, B, _DTYPE_CODE[ref.dtype], _stream(stream)),
           "pa_cache_from_token_major")


def split_layout(key_tm, value_tm, stream=None):
    """New key / value caches in the split layout from token-major ones."""
    nb, Hkv, B, D = key_tm.shape
    x = key_group(key_tm.dtype)
    k = torch.empty((nb, Hkv, D // x, B, x), dtype=key_tm.dtype, device=key_tm.device)
    v = torch.empty((nb, Hkv, D, B), dtype=value_tm.dtype, device=value_tm.device)
    pa_cache_from_token_major(k, v, key_tm, value_tm, stream)
    return k, v


def pa_status_string(status: int) -> str:
    return load_library().pa_status_string(int(status)).decode()


def pa_workspace_size(num_seqs: int, num_q_heads: int, head_dim: int, max_seq_len: int,
                      partition_size: int) -> int:
    return int(load_library().pa_workspace_size(num_seqs, num_q_heads, head_dim, max_seq_len,
                                                partition_size))


def pa_workspace_layout(num_seqs, num_q_heads, head_dim, max_seq_len, partition_size):
    """(tmp_output_offset, exp_sums_offset, max_logits_offset, max_partitions) in bytes / count."""
    t, e, m, n = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_int()
    st = load_library().pa_workspace_layout(num_seqs, num_q_heads, head_dim, max_seq_len,
                                            partition_size, ctypes.byref(t), ctypes.byref(e),
                                            ctypes.byref(m), ctypes.byref(n))
    if st != PA_OK:
        raise PagedAttentionError(st, "pa_workspace_layout")
    return int(t.value), int(e.value), int(m.value), int(n.value)


def pa_workspace_init(workspace, stream=None):
    """Zero the counter header of a workspace (needed once, before its first pa_decode_v2)."""
    wp, wb = _workspace(workspace)
    _check(load_library().pa_workspace_init(wp, wb, _stream(stream)), "pa_workspace_init")


def pa_select_partition_size(num_seqs: int, num_kv_heads: int, max_seq_len: int) -> int:
    """The partition size the split-KV entry points use for partition_size = 0."""
    return int(load_library().pa_select_partition_size(num_seqs, num_kv_heads, max_seq_len))


def pa_select_v2(max_seq_len: int, num_seqs: int, num_kv_heads: int, partition_size: int) -> bool:
    return bool(load_library().pa_select_v2(max_seq_len, num_seqs, num_kv_heads, partition_size))


def pa_select_v2_auto(max_seq_len: int, num_seqs: int, num_kv_heads: int,
                      partition_size: int) -> bool:
    return bool(load_library().pa_select_v2_auto(max_seq_len, num_seqs, num_kv_heads,
                                                 partition_size))


def _stream(stream):
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def _dev(name, t, dtype=None, ndim=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a GPU (the library has no CPU path)")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {tuple(t.shape)}")
    return ctypes.c_void_p(t.data_ptr())


def key_group(dtype: torch.dtype) -> int:
    """x of the key layout: values per 16-byte group (8 for bf16, 4 for float32)."""
    return 16 // torch.empty((), dtype=dtype).element_size()


def _problem(query, key_cache, value_cache, block_tables, seq_lens, scale, max_seq_len):
    if query.dtype not in _DTYPE_CODE:
        raise TypeError(f"query dtype must be float32 or bfloat16, got {query.dtype}")
    if query.dim() != 3 or key_cache.dim() != 5 or value_cache.dim() != 4:
        raise ValueError("query [S, Hq, D], key_cache [blocks, Hkv, D/x, 16, x] and "
                         "value_cache [blocks, Hkv, D, 16] expected")
    S, Hq, D = query.shape
    nb, Hkv, Dx, B, x = key_cache.shape
    if x != key_group(query.dtype) or Dx * x != D or tuple(value_cache.shape) != (nb, Hkv, D, B):
        raise ValueError(f"cache shapes {tuple(key_cache.shape)} / {tuple(value_cache.shape)} do "
                         f"not match the query {tuple(query.shape)} in the split layout")
    if block_tables.shape[0] != S or seq_lens.shape[0] != S:
        raise ValueError("block_tables and seq_lens need one row per sequence")
    args = [_dev("query", query, None, 3),
            _dev("key_cache", key_cache, query.dtype, 5),
            _dev("value_cache", value_cache, query.dtype, 4),
            _dev("block_tables", block_tables, torch.int32, 2),
            _dev("seq_lens", seq_lens, torch.int32, 1),
            S, Hq, Hkv, D, B, nb, block_tables.shape[1], int(max_seq_len), float(scale),
            _DTYPE_CODE[query.dtype]]
    return args


def _problem_q(query, key_cache, value_cache, block_tables, seq_lens, scale, max_seq_len):
    """Arguments of the q_len entry points: query [S, q_len, Hq, D]."""
    if query.dim() != 4:
        raise ValueError("query must be [S, q_len, Hq, D]")
    S, q_len, Hq, D = query.shape
    args = _problem(query.view(S, q_len * Hq, D), key_cache, value_cache, block_tables, seq_lens,
                    scale, max_seq_len)
    # replace the flattened head count by (q_len, Hq)
    return args[:5] + [S, q_len, Hq] + args[7:], q_len, Hq


def _check(st, where):
    if st != PA_OK:
        raise PagedAttentionError(st, where)


def _workspace(ws):
    if ws is None:
        return ctypes.c_void_p(0), 0
    _dev("workspace", ws)
    return ctypes.c_void_p(ws.data_ptr()), ws.numel() * ws.element_size()


def pa_decode_v1(out, query, key_cache, value_cache, block_tables, seq_lens, scale, max_seq_len,
                 stream=None):
    """V1 single-pass decode into out [S, Hq, D] (same dtype as query)."""
    args = _problem(query, key_cache, value_cache, block_tables, seq_lens, scale, max_seq_len)
    o = _dev("out", out, query.dtype)
    if out.shape != query.shape:
        raise ValueError("out must have the query's shape")
    _check(load_library().pa_decode_v1(o, *args, _stream(stream)), "pa_decode_v1")


def pa_decode_v2(out, query, key_cache, value_cache, block_tables, seq_lens, scale, max_seq_len,
                 partition_size, workspace, stream=None):
    """V2 split-KV decode: Phase 1 partials into workspace, Phase 2 merge into out."""
    args = _problem(query, key_cache, value_cache, block_tables, seq_lens, scale, max_seq_len)
    o = _dev("out", out, query.dtype)
    if out.shape != query.shape:
        raise ValueError("out must have the query's shape")
    wp, wb = _workspace(workspace)
    _check(load_library().pa_decode_v2(o, *args, int(partition_size), wp, wb, _stream(stream)),
           "pa_decode_v2")


NOALLOC_SCRATCH_BYTES = 64 << 20  # PA_NOALLOC_SCRATCH_BYTES


def pa_decode_v2_noalloc(out, query, key_cache, value_cache, block_tables, seq_lens, scale,
                         max_seq_len, partition_size, stream=None):
    """pa_decode_v2 with its workspace in the library's per-device scratch array (no
    allocation; problems whose workspace exceeds NOALLOC_SCRATCH_BYTES are refused)."""
    args = _problem(query, key_cache, value_cache, block_tables, seq_lens, scale, max_seq_len)
    o = _dev("out", out, query.dtype)
    if out.shape != query.shape:
        raise ValueError("out must have the query's shape")
    _check(load_library().pa_decode_v2_noalloc(o, *args, int(partition_size), _stream(stream)),
           "pa_decode_v2_noalloc")


def bind_decode_v2(out, query, key_cache, value_cache, block_tables, seq_lens, scale, max_seq_len,
                   partition_size, workspace, stream=None):
    """pa_decode_v2 with its arguments checked and marshalled once: returns a
    callable that enqueues the call again (for launch loops, where re-marshalling
    the tensors each time would cost more host time than the launch itself).  The
    library still checks every call; the tensors must stay alive and unmoved."""
    args = _problem(query, key_cache, value_cache, block_tables, seq_lens, scale, max_seq_len)
    o = _dev("out", out, query.dtype)
    if out.shape != query.shape:
        raise ValueError("out must have the query's shape")
    wp, wb = _workspace(workspace)
    full = (o, *args, int(partition_size), wp, wb, _stream(stream))
    fn = load_library().pa_decode_v2

    def call():
        st = fn(*full)
        if st != PA_OK:
            raise PagedAttentionError(st, "pa_decode_v2")
    return call


def pa_decode_v2_single(out, query, key_cache, value_cache, block_tables, seq_lens, scale,
                        max_seq_len, partition_size, workspace, stream=None):
    """V2 in one launch (the workspace header must be zero before the first call;
    new_workspace returns it zeroed).  Raises PagedAttentionError with
    PA_ERR_UNSUPPORTED when the problem does not fit the single-launch merge."""
    args = _problem(query, key_cache, value_cache, block_tables, seq_lens, scale, max_seq_len)
    o = _dev("out", out, query.dtype)
    if out.shape != query.shape:
        raise ValueError("out must have the query's shape")
    wp, wb = _workspace(workspace)
    _check(load_library().pa_decode_v2_single(o, *args, int(partition_size), wp, wb,
                                              _stream(stream)), "pa_decode_v2_single")


def pa_decode(out, query, key_cache, value_cache, block_tables, seq_lens, scale, max_seq_len,
              partition_size, workspace, stream=None):
    """V1 or V2 as pa_select_v2 decides."""
    args = _problem(query, key_cache, value_cache, block_tables, seq_lens, scale, max_seq_len)
    o = _dev("out", out, query.dtype)
    if out.shape != query.shape:
        raise ValueError("out must have the query's shape")
    wp, wb = _workspace(workspace)
    _check(load_library().pa_decode(o, *args, int(partition_size), wp, wb, _stream(stream)),
           "pa_decode")


def pa_decode_auto(out, query, key_cache, value_cache, block_tables, seq_lens, scale, max_seq_len,
                   partition_size, workspace, stream=None):
    """V1 or V2 as pa_select_v2_auto decides (the MI355X-measured rule)."""
    args = _problem(query, key_cache, value_cache, block_tables, seq_lens, scale, max_seq_len)
    o = _dev("out", out, query.dtype)
    if out.shape != query.shape:
        raise ValueError("out must have the query's shape")
    wp, wb = _workspace(workspace)
    _check(load_library().pa_decode_auto(o, *args, int(partition_size), wp, wb, _stream(stream)),
           "pa_decode_auto")


def pa_decode_v1_q(out, query, key_cache, value_cache, block_tables, seq_lens, scale, max_seq_len,
                   stream=None):
    """V1 for q_len query tokens per sequence: query and out [S, q_len, Hq, D]."""
    args, _, _ = _problem_q(query, key_cache, value_cache, block_tables, seq_lens, scale,
                            max_seq_len)
    o = _dev("out", out, query.dtype)
    if out.shape != query.shape:
        raise ValueError("out must have the query's shape")
    _check(load_library().pa_decode_v1_q(o, *args, _stream(stream)), "pa_decode_v1_q")


def pa_decode_v2_q(out, query, key_cache, value_cache, block_tables, seq_lens, scale, max_seq_len,
                   partition_size, workspace, stream=None):
    """V2 for q_len query tokens per sequence; the workspace is sized for S sequences
    of q_len * Hq heads (new_workspace(S, q_len * Hq, ...))."""
    args, _, _ = _problem_q(query, key_cache, value_cache, block_tables, seq_lens, scale,
                            max_seq_len)
    o = _dev("out", out, query.dtype)
    if out.shape != query.shape:
        raise ValueError("out must have the query's shape")
    wp, wb = _workspace(workspace)
    _check(load_library().pa_decode_v2_q(o, *args, int(partition_size), wp, wb, _stream(stream)),
           "pa_decode_v2_q")


def pa_select_q_kernel(single_pass, num_seqs, q_len, num_q_heads, num_kv_heads, dtype,
                       max_seq_len, partition_size=1024):
    """Kernel the q_len entry points use: 0 = decode kernel, 1 or 2 = prefill kernel tiles.
    dtype: torch.float32 / torch.bfloat16."""
    return int(load_library().pa_select_q_kernel(int(bool(single_pass)), int(num_seqs), int(q_len),
                                                 int(num_q_heads), int(num_kv_heads),
                                                 _DTYPE_CODE[dtype], int(max_seq_len),
                                                 int(partition_size)))


def pa_prefill_v1(out, query, key_cache, value_cache, block_tables, seq_lens, scale, max_seq_len,
                  column_tiles=0, stream=None):
    """Tiled prefill, one pass: query and out [S, q_len, Hq, D], bf16; column_tiles
    1, 2 or 4 tiles of 16 columns per wave (0: the library's choice)."""
    args, _, _ = _problem_q(query, key_cache, value_cache, block_tables, seq_lens, scale,
                            max_seq_len)
    o = _dev("out", out, query.dtype)
    if out.shape != query.shape:
        raise ValueError("out must have the query's shape")
    _check(load_library().pa_prefill_v1(o, *args, int(column_tiles), _stream(stream)),
           "pa_prefill_v1")


def pa_prefill_v2(out, query, key_cache, value_cache, block_tables, seq_lens, scale, max_seq_len,
                  partition_size, workspace, column_tiles=0, stream=None):
    """Tiled prefill, split-KV: as pa_decode_v2_q (same workspace) plus column_tiles."""
    args, _, _ = _problem_q(query, key_cache, value_cache, block_tables, seq_lens, scale,
                            max_seq_len)
    o = _dev("out", out, query.dtype)
    if out.shape != query.shape:
        raise ValueError("out must have the query's shape")
    wp, wb = _workspace(workspace)
    _check(load_library().pa_prefill_v2(o, *args, int(partition_size), wp, wb, int(column_tiles),
                                        _stream(stream)), "pa_prefill_v2")


def pa_decode_v2_partials(query, key_cache, value_cache, block_tables, seq_lens, scale,
                          max_seq_len, partition_size, workspace, stream=None):
    """V2 Phase 1 only: partials into workspace (see workspace_views)."""
    args = _problem(query, key_cache, value_cache, block_tables, seq_lens, scale, max_seq_len)
    wp, wb = _workspace(workspace)
    _check(load_library().pa_decode_v2_partials(*args, int(partition_size), wp, wb,
                                                _stream(stream)), "pa_decode_v2_partials")


def pa_decode_v2_reduce(out, seq_lens, max_seq_len, partition_size, workspace, stream=None):
    """V2 Phase 2 only: merge the workspace partials into out [S, Hq, D]."""
    S, Hq, D = out.shape
    o = _dev("out", out)
    if out.dtype not in _DTYPE_CODE:
        raise TypeError("out must be float32 or bfloat16")
    sl = _dev("seq_lens", seq_lens, torch.int32, 1)
    wp, wb = _workspace(workspace)
    _check(load_library().pa_decode_v2_reduce(o, sl, S, Hq, D, int(max_seq_len),
                                              _DTYPE_CODE[out.dtype], int(partition_size), wp, wb,
                                              _stream(stream)), "pa_decode_v2_reduce")


def pa_decode_v2_groups(query, key_cache, value_cache, block_tables, seq_lens, scale, max_seq_len,
                        partition_size, workspace, stream=None) -> int:
    """V2 Phase 1 as pa_decode_v2 runs it; returns the tokens behind each workspace entry."""
    args = _problem(query, key_cache, value_cache, block_tables, seq_lens, scale, max_seq_len)
    wp, wb = _workspace(workspace)
    n = ctypes.c_int(0)
    _check(load_library().pa_decode_v2_groups(*args, int(partition_size), wp, wb, ctypes.byref(n),
                                              _stream(stream)), "pa_decode_v2_groups")
    return int(n.value)


def pa_decode_v2_reduce_entries(out, seq_lens, max_seq_len, partition_size, entry_tokens,
                                workspace, stream=None):
    """V2 Phase 2 over workspace entries of entry_tokens tokens each."""
    S, Hq, D = out.shape
    o = _dev("out", out)
    if out.dtype not in _DTYPE_CODE:
        raise TypeError("out must be float32 or bfloat16")
    sl = _dev("seq_lens", seq_lens, torch.int32, 1)
    wp, wb = _workspace(workspace)
    _check(load_library().pa_decode_v2_reduce_entries(
        o, sl, S, Hq, D, int(max_seq_len), _DTYPE_CODE[out.dtype], int(partition_size),
        int(entry_tokens), wp, wb, _stream(stream)), "pa_decode_v2_reduce_entries")


def new_workspace(num_seqs, num_q_heads, head_dim, max_seq_len, partition_size, device="cuda"):
    """A zero-filled uint8 device tensor of pa_workspace_size bytes (at least the
    counter header), ready for every V2 entry point."""
    n = pa_workspace_size(num_seqs, num_q_heads, head_dim, max_seq_len, partition_size)
    return torch.zeros(max(n, WORKSPACE_HEADER_BYTES), dtype=torch.uint8, device=device)


def workspace_views(workspace, num_seqs, num_q_heads, head_dim, max_seq_len, partition_size):
    """(tmp_out [S,Hq,Pmax,D], exp_sums [S,Hq,Pmax], max_logits [S,Hq,Pmax]) float32 views."""
    t_off, e_off, m_off, n = pa_workspace_layout(num_seqs, num_q_heads, head_dim, max_seq_len,
                                                 partition_size)
    rows = num_seqs * num_q_heads * n
    f = workspace.view(torch.uint8)
    tmp = f[t_off:t_off + rows * head_dim * 4].view(torch.float32).view(num_seqs, num_q_heads, n,
                                                                        head_dim)
    es = f[e_off:e_off + rows * 4].view(torch.float32).view(num_seqs, num_q_heads, n)
    ml = f[m_off:m_off + rows * 4].view(torch.float32).view(num_seqs, num_q_heads, n)
    return tmp, es, ml
