"""split_kv_paged_pa_amd: paged single-query decode attention for AMD MI355X (gfx950).

The kernels and their C ABI live in libpa_decode.so (sources in csrc/, header
include/pa_decode.h at the repository root); `api` is the Python binding with
the same function names; `workloads` draws seeded synthetic decode batches.
"""
from .api import (PagedAttentionError, bind_decode_v2, load_library, new_workspace, pa_cache_from_token_major,
                  pa_decode, pa_decode_auto, split_layout,
                  pa_decode_v1, pa_decode_v1_q, pa_decode_v2, pa_decode_v2_partials,
                  pa_decode_v2_groups, pa_decode_v2_noalloc, pa_decode_v2_q, pa_decode_v2_reduce,
                  pa_decode_v2_reduce_entries,
                  pa_decode_v2_single, pa_prefill_v1, pa_prefill_v2, pa_select_partition_size,
                  pa_select_q_kernel, pa_select_v2, pa_select_v2_auto, pa_status_string,
                  pa_workspace_init, pa_workspace_layout, pa_workspace_size, workspace_views)

__all__ = ["PagedAttentionError", "bind_decode_v2", "load_library", "new_workspace", "pa_cache_from_token_major",
           "pa_decode", "pa_decode_auto", "split_layout",
           "pa_decode_v1", "pa_decode_v1_q", "pa_decode_v2", "pa_decode_v2_partials",
           "pa_decode_v2_groups", "pa_decode_v2_noalloc", "pa_decode_v2_q", "pa_decode_v2_reduce",
           "pa_decode_v2_reduce_entries",
           "pa_decode_v2_single", "pa_prefill_v1", "pa_prefill_v2", "pa_select_partition_size",
           "pa_select_q_kernel", "pa_select_v2", "pa_select_v2_auto", "pa_status_string",
           "pa_workspace_init", "pa_workspace_layout", "pa_workspace_size", "workspace_views"]
