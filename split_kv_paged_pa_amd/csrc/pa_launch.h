// pa_launch.h -- internal interface between the C-ABI layer (pa_api.cpp) and the
// HIP kernels (pa_kernels.hip).  Not installed, not part of the public ABI.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace pa {

enum class Dtype : int { F32 = 0, BF16 = 1 };

// One decode batch, already validated by the ABI layer.
struct Problem {
    const void *query;          // [S][qlen][Hq][D]
    const void *key_cache;      // [num_blocks][Hkv][D / x][16][x], x = 16 bytes of values
    const void *value_cache;    // [num_blocks][Hkv][D][16]
    const int32_t *block_tables;  // [S][max_blocks]
    const int32_t *seq_lens;    // [S]
    int num_seqs, num_q_heads, num_kv_heads, head_dim;
    int qlen;                   // query tokens per sequence (query/out are [S][qlen][Hq][D])
    int num_blocks, max_blocks, max_seq_len;
    float scale;
    Dtype dtype;
};

// Float32 partials of the split-KV form, carved out of the caller's workspace.
struct Partials {
    float *tmp_out;      // [S][Hq][max_parts][D]
    float *exp_sums;     // [S][Hq][max_parts]
    float *max_logits;   // [S][Hq][max_parts]
    uint32_t *tickets;   // [S][Hkv] arrival counters of the fused form (zero between calls)
    int partition_size;
    int max_parts;   // entries per row of the three arrays (the row stride)
    int per_group;   // consecutive partitions handled by one Phase-1 workgroup
    int span_blocks; // launch_grouped: blocks per workgroup (any partition boundaries inside)
    int span_count;  // launch_grouped: workgroups per (sequence, kv head, chunk)
    int entry_tokens;  // tokens behind each entry Phase 2 reads: partition_size after
                       // launch_partitions, 16 * span_blocks after launch_grouped
    int marked_entries;  // >= 0: Phase 1 wrote entries [0, marked_entries) of every row
                         // (launch_grouped: span_count; an empty span's max logit is -inf),
                         // so Phase 2 needs no seq_lens; -1: ceil(L_s / entry_tokens) entries
};

// V1: one workgroup per (kv head, sequence) over the whole sequence -> out.
hipError_t launch_single_pass(const Problem &pb, void *out, hipStream_t stream);
// V2 Phase 1: one workgroup per (partition, kv head, sequence) -> partials.
hipError_t launch_partitions(const Problem &pb, const Partials &parts, hipStream_t stream);
// V2 Phase 1 as equal spans: workgroup x of a (sequence, kv head, chunk) takes
// blocks [x * span_blocks, (x + 1) * span_blocks) as one partition and writes its
// partials to entry x of the row (max logit -inf when the span is past the
// sequence's end) -> Phase 2 then runs with entry_tokens = 16 * span_blocks and
// marked_entries = span_count.  Needs span_count <= max_parts and span_count *
// span_blocks >= ceil(max_seq_len / 16).
hipError_t launch_grouped(const Problem &pb, const Partials &parts, hipStream_t stream);
// V2 in one launch: the Phase-1 grid; each workgroup folds its partitions into a
// group partial, and the last workgroup of each (sequence, kv head) merges them -> out.
// Needs group * ceil(max_parts / per_group) <= fused_merge_capacity().
hipError_t launch_fused(const Problem &pb, const Partials &parts, void *out, hipStream_t stream);
int fused_merge_capacity();
// n uint32 zeros at p (a plain fill kernel).
hipError_t launch_zero_words(uint32_t *p, int n, hipStream_t stream);
// Many columns (G * qlen (query token, head) pairs per kv head), bf16 only: each
// wave holds nct tiles of 16 columns; a workgroup's 4 waves share one K/V stream
// staged through LDS.  parts == nullptr: one pass over each sequence -> out;
// otherwise one workgroup per partition -> partials (then launch_reduce).  nct is
// 1, 2 or 4.
hipError_t launch_prefill(const Problem &pb, const Partials *parts, void *out, int nct,
                          hipStream_t stream);
// Workgroups per kv head in grid y of launch_prefill.
int prefill_column_groups(int group, int qlen, int nct);
// Token-major caches [num_blocks][num_kv_heads][16][head_dim] into the split
// layout (keys [..][head_dim / x][16][x], values [..][head_dim][16]); either
// input / output pair may be null.  head_dim a multiple of 16 bytes' worth of
// elements, at most repack_max_dim().
hipError_t launch_repack(const void *key_in, const void *value_in, void *key_out, void *value_out,
                         int num_blocks, int num_kv_heads, int head_dim, Dtype dtype,
                         hipStream_t stream);
int repack_max_dim();
// V2 Phase 2: partials -> out.  Row r of sequence s holds ceil(L_s / entry_tokens)
// valid entries.
hipError_t launch_reduce(const int32_t *seq_lens, int num_seqs, int num_q_heads, int head_dim,
                         int max_seq_len, Dtype dtype, const Partials &parts, void *out,
                         hipStream_t stream);

}  // namespace pa
