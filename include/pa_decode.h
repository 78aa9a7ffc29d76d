/*
 * pa_decode.h -- C ABI of libpa_decode.so: paged single-query decode attention
 * on AMD MI355X (gfx950).
 *
 * The operation.  For every sequence s and query head h, attention of the one
 * decode-step query q[s][h] over the L = seq_lens[s] cached tokens of s, with
 * grouped-query heads: query head h reads kv head h / G, G = num_q_heads /
 * num_kv_heads.
 *   z_t = scale * (q . k_t),  out = sum_t softmax(z)_t * v_t,   t = 0 .. L-1
 * Token t of sequence s lives in slot t % 16 of physical block
 * block_tables[s][t / 16].
 *
 * Sources (project_6 commit pages):
 *   - paged cache read through a per-sequence block id list, 16-token blocks,
 *     GQA by broadcasting each kv head over its group: commit 15ef28e
 *     (paged_attention_v2_pytorch.py), message "[OPT] Vectorize
 *     paged_attention_v2";
 *   - V1 (one pass over the whole sequence per unit of work) and V2 (Phase 1
 *     per-partition max logit, exp-sum and partial output; Phase 2 merge with
 *     the global max and the rescale exp(m_p - M) * s_p): commit 15ef28e,
 *     message "[OPT] PagedAttention V2 implementation";
 *   - partition size as the tuning knob (512 vs 1024), and V2 only for
 *     max_seq_len above 8192: commit 900ae0b (vllm/_custom_ops.py), messages
 *     "Two changes based on CCCL source reading" and "THE SINGLE
 *     HIGHEST-IMPACT CODE CHANGE";
 *   - caller-owned, pre-allocated V2 intermediates: commit 490ff98
 *     (paged_attn.py), "Three changes", item 2.
 *
 * Deployment note: every call launches one or two short kernels whose first
 * instruction reads its arguments.  Run the process with the ROCm runtime
 * variable HIP_FORCE_DEV_KERNARG=1 (read when HIP starts) so that kernel
 * arguments live in device memory: measured on MI355X, a 100K-token V2 step
 * takes about 2 us less than with the default host-memory arguments.
 *
 * Layouts (row-major, contiguous, all in device memory):
 *   query, out      [num_seqs][num_q_heads][head_dim]                         dtype
 *   key_cache       [num_blocks][num_kv_heads][head_dim / x][block_size][x]    dtype
 *   value_cache     [num_blocks][num_kv_heads][head_dim][block_size]           dtype
 *   block_tables    [num_seqs][max_blocks_per_seq]                             int32
 *   seq_lens        [num_seqs]                                                 int32
 * with x = 16 bytes / element size (8 for bf16, 4 for float32): K[t][d] of
 * slot t of a block is at [..][d / x][t][d % x], V[t][d] at [..][d][t].  The
 * pages gather whole blocks by id and permute them into token order, leaving
 * the in-block order open; this is the split layout of paged caches, in
 * which every 16-byte key group and every value row of a block is contiguous
 * across its 16 tokens.
 * dtype (PA_DTYPE_F32 or PA_DTYPE_BF16) applies to query, caches and out.
 * Partials in the V2 workspace are always float32 (layout below).
 *
 * Alignment: query, key_cache, value_cache, out and the workspace must be
 * 16-byte aligned (else PA_ERR_INVALID_ARGUMENT).
 *
 * Ownership and threading.  Every pointer is caller-owned device memory (except
 * host-side size outputs).  The library never allocates, frees or synchronises,
 * and never reads device memory from the host.  It holds no state: calls from
 * several threads are safe as long as their outputs and workspaces differ.
 * `out` must not alias any input or the workspace.  All work is enqueued on
 * `stream` (a hipStream_t; NULL is the default stream) of the current device.
 *
 * Errors.  Every check that the host can make is made before anything is
 * enqueued; on failure nothing is launched and `out` / `workspace` are left
 * untouched.  PA_ERR_HIP reports a failed launch (hipGetLastError).  PA_OK
 * means "enqueued".
 *
 * Device-side contract (not checkable on the host, enforced defensively):
 *   - 0 <= seq_lens[s] <= max_seq_len; values outside are clamped into that
 *     range by the kernels;
 *   - the first ceil(seq_lens[s] / 16) entries of block_tables[s] are block ids
 *     in [0, num_blocks); an id outside that range is never dereferenced and
 *     the 16 tokens it stands for are left out of the softmax;
 *   - cache slots past the end of a sequence (the tail of its last block) are
 *     never used: any value there, NaN included, does not reach the output.
 *
 * Supported shapes: head_dim 64 or 128; block_size 16; num_q_heads a multiple
 * of num_kv_heads with group size G <= 16; partition_size a multiple of 16;
 * num_seqs <= 65535 and num_kv_heads * ceil(G * q_len / 16) <= 65535 (q_len = 1
 * for the plain entry points).  Anything else returns
 * PA_ERR_UNSUPPORTED or PA_ERR_INVALID_SHAPE.
 */
#ifndef PA_DECODE_H
#define PA_DECODE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes and dtypes are 32-bit integers with named values (not C enum
 * types), so that a caller passing any int -- a bad dtype included -- hands the
 * library a well-defined value to reject. */
typedef int32_t pa_status_t;
enum {
    PA_OK = 0,
    PA_ERR_NULL_POINTER = 1,       /* a required pointer is NULL */
    PA_ERR_INVALID_SHAPE = 2,      /* negative or inconsistent sizes */
    PA_ERR_UNSUPPORTED = 3,        /* valid, but outside the supported shapes */
    PA_ERR_WORKSPACE_TOO_SMALL = 4,
    PA_ERR_HIP = 5,                /* a HIP launch failed */
    PA_ERR_INVALID_ARGUMENT = 6    /* non-finite scale, bad dtype, misaligned pointer,
                                      column_tiles not 0, 1, 2 or 4 */
};

typedef int32_t pa_dtype_t;
enum { PA_DTYPE_F32 = 0, PA_DTYPE_BF16 = 1 };

/* Human-readable name of a status code (static storage; never NULL). */
const char *pa_status_string(pa_status_t status);

/* Bytes at the start of every V2 workspace that hold the arrival counters of
 * pa_decode_v2_single (one uint32 per (sequence, kv head), up to 4096). */
#define PA_WORKSPACE_HEADER_BYTES 16384

/*
 * Bytes of V2 workspace for this problem: the counter header, then three
 * float32 arrays, each starting on a 256-byte boundary, with
 * P_max = ceil(max_seq_len / partition_size):
 *   header      PA_WORKSPACE_HEADER_BYTES                  at offset 0
 *   tmp_output  [num_seqs][num_q_heads][P_max][head_dim]   at *tmp_output_offset
 *   exp_sums    [num_seqs][num_q_heads][P_max]             at *exp_sums_offset
 *   max_logits  [num_seqs][num_q_heads][P_max]             at *max_logits_offset
 * After pa_decode_v2_partials, max_logits holds the largest scaled logit of
 * each partition (natural-log units), exp_sums holds sum_t exp(z_t - max_logit)
 * over the partition, and tmp_output holds the partition's normalised output
 * sum_t exp(z_t - m) v_t / s.  (The pre-allocated intermediates of commit
 * 490ff98, "Three changes", item 2.)
 * The header must be zero before the workspace's first use by
 * pa_decode_v2_single (pa_workspace_init, or any zero fill of the buffer);
 * every call leaves it zero again, whatever the problem shape, so one
 * workspace serves calls of any shape that fits it.  The other entry points
 * neither read nor write the header.
 * Returns 0 when there is nothing to hold (num_seqs or max_seq_len is 0) or
 * when the arguments are invalid (negative sizes, partition_size not a
 * positive multiple of 16).
 */
size_t pa_workspace_size(int num_seqs, int num_q_heads, int head_dim, int max_seq_len,
                         int partition_size);

/* Offsets of the workspace arrays described at pa_workspace_size.  Any output
 * pointer may be NULL.  Returns PA_ERR_INVALID_SHAPE for invalid sizes. */
pa_status_t pa_workspace_layout(int num_seqs, int num_q_heads, int head_dim, int max_seq_len,
                                int partition_size, size_t *tmp_output_offset,
                                size_t *exp_sums_offset, size_t *max_logits_offset,
                                int *max_partitions);

/* Zeroes the counter header of a workspace (workspace_bytes >=
 * PA_WORKSPACE_HEADER_BYTES, 16-byte aligned), with a small fill kernel on
 * `stream`.  Needed once per workspace, before its first pa_decode_v2_single. */
pa_status_t pa_workspace_init(void *workspace, size_t workspace_bytes, void *stream);

/*
 * V1: single pass.  One workgroup per (sequence, kv head) walks all of the
 * sequence's blocks with an online-softmax accumulator {running max, running
 * exp-sum, running output}, merging with the factor exp(old max - new max)
 * (commit 490ff98, the summary_statistics message; commit 15ef28e, "[OPT]
 * PagedAttention V2 implementation", the V1 limitation).  Writes out directly.
 */
pa_status_t pa_decode_v1(void *out, const void *query, const void *key_cache,
                         const void *value_cache, const int32_t *block_tables,
                         const int32_t *seq_lens, int num_seqs, int num_q_heads, int num_kv_heads,
                         int head_dim, int block_size, int num_blocks, int max_blocks_per_seq,
                         int max_seq_len, float scale, pa_dtype_t dtype, void *stream);

/*
 * Partition size for the split-KV entry points when the caller passes
 * partition_size = 0.  The pages treat the partition size as the knob that
 * trades Phase-1 parallelism against Phase-2 cost (commit 900ae0b, "Two
 * changes based on CCCL source reading", item 1; commit 490ff98, "Three
 * changes", item 3); their 512 and 1024 were chosen for a 16-SM device.  This
 * rule is measured on MI355X: 2048 tokens, unless that gives fewer work units
 * (num_seqs * num_kv_heads * ceil(max_seq_len / 2048)) than the current
 * device has compute units; then the smallest multiple of 16 (at least 256)
 * that gives at most one partition per compute unit, i.e. about
 * max_seq_len * num_seqs * num_kv_heads / CUs (1568 for one 100000-token
 * sequence with 4 kv heads on 256 CUs).  Returns 2048 for invalid arguments.
 * Host-only; 256 compute units are assumed when no device is visible.  Size the
 * workspace with the value it returns: pa_workspace_size(..., 0) is invalid.
 */
int pa_select_partition_size(int num_seqs, int num_kv_heads, int max_seq_len);

/*
 * V2: split-KV.  Phase 1, one workgroup per (partition group, kv head,
 * sequence), computes each partition's partials; Phase 2, one workgroup per
 * (query head, sequence), merges them into out (commit 15ef28e, "[OPT]
 * PagedAttention V2 implementation", Phase 1 and Phase 2).  Two launches on
 * `stream`, no host synchronisation.  partition_size = 0 uses
 * pa_select_partition_size(num_seqs, num_kv_heads, max_seq_len).
 * workspace_bytes must be at least pa_workspace_size(num_seqs, num_q_heads,
 * head_dim, max_seq_len, partition_size) and the workspace 16-byte aligned; it
 * may be reused by later calls on the same stream, but two calls in flight at
 * once must not share it.  A sequence with L == 0 gets an all-zero output row.
 * When partitions are few, Phase 1 runs in equal spans of blocks, about one
 * per compute unit (see pa_decode_v2_groups): after pa_decode_v2 the workspace
 * holds Phase-2 entries, one per span, not necessarily one per partition
 * (pa_decode_v2_partials writes one per partition).
 */
pa_status_t pa_decode_v2(void *out, const void *query, const void *key_cache,
                         const void *value_cache, const int32_t *block_tables,
                         const int32_t *seq_lens, int num_seqs, int num_q_heads, int num_kv_heads,
                         int head_dim, int block_size, int num_blocks, int max_blocks_per_seq,
                         int max_seq_len, float scale, pa_dtype_t dtype, int partition_size,
                         void *workspace, size_t workspace_bytes, void *stream);

/*
 * V2 in a single launch: the same partitions, each computed as in Phase 1, but
 * every workgroup folds the partitions it computed into one partial with the
 * Phase-2 rescale, and the last workgroup of each (sequence, kv head) to
 * finish -- found with an arrival counter in the workspace header -- merges
 * those partials in a fixed order and writes out.  Commit 490ff98 (the
 * StableReductionOrder paragraph) sets a one-kernel atomic merge against a
 * two-kernel stable one; this is one kernel with a fixed merge order, so its
 * results are reproducible bit for bit (they differ from pa_decode_v2's only
 * in rounding order).  Same arguments and workspace as pa_decode_v2, whose
 * header must be zero before the first call (see pa_workspace_size).  Returns
 * PA_ERR_UNSUPPORTED, having launched nothing, when num_seqs * num_kv_heads >
 * 4096 or when (num_q_heads / num_kv_heads) times the number of workgroups per
 * (sequence, kv head) exceeds 2048.  On MI355X the two launches of
 * pa_decode_v2 measured faster; this form is for callers that need one launch.
 */
pa_status_t pa_decode_v2_single(void *out, const void *query, const void *key_cache,
                                const void *value_cache, const int32_t *block_tables,
                                const int32_t *seq_lens, int num_seqs, int num_q_heads,
                                int num_kv_heads, int head_dim, int block_size, int num_blocks,
                                int max_blocks_per_seq, int max_seq_len, float scale,
                                pa_dtype_t dtype, int partition_size, void *workspace,
                                size_t workspace_bytes, void *stream);

/*
 * Decode of q_len query tokens per sequence (q_len >= 1: several new tokens at
 * once, as in speculative decoding).  query and out are
 * [num_seqs][q_len][num_q_heads][head_dim].  The q_len tokens are the last
 * q_len positions of each sequence and are already in the cache.  Query token j
 * sits at position L - q_len + j and attends to tokens 0 .. L - q_len + j
 * (causal over the cache); a token that sees no token (L < q_len - j) gets a
 * zero row.  This extends the decode step along the q_len dimension that the
 * pages batch next to the GQA group (commit 490ff98, the summary_statistics
 * message).  Each (token, head) pair is one column of the kernels' 16-wide
 * tiles.  The decode kernel gives a workgroup 16 columns of a kv head, so up to
 * (num_q_heads / num_kv_heads) * q_len = 16 the keys and values are read once,
 * and beyond that once per 16 columns; for many columns (bf16) these entry
 * points switch to the tiled prefill kernel of pa_prefill_v1 / pa_prefill_v2,
 * as pa_select_q_kernel reports (results then agree to rounding, not bit for
 * bit, with the decode kernel's).  num_kv_heads * ceil(G * q_len / 16) must not
 * exceed 65535, else PA_ERR_UNSUPPORTED.
 * pa_decode_v1_q is the single pass.  pa_decode_v2_q is split-KV in two
 * launches; its workspace holds q_len * num_q_heads rows per sequence, i.e.
 * pa_workspace_size(num_seqs, q_len * num_q_heads, head_dim, max_seq_len,
 * partition_size) bytes; partition_size = 0 uses
 * pa_select_partition_size(num_seqs, num_kv_heads * ceil(G * q_len / 16),
 * max_seq_len).  With q_len = 1 they equal pa_decode_v1 and
 * pa_decode_v2 bit for bit.
 */
pa_status_t pa_decode_v1_q(void *out, const void *query, const void *key_cache,
                           const void *value_cache, const int32_t *block_tables,
                           const int32_t *seq_lens, int num_seqs, int q_len, int num_q_heads,
                           int num_kv_heads, int head_dim, int block_size, int num_blocks,
                           int max_blocks_per_seq, int max_seq_len, float scale,
                           pa_dtype_t dtype, void *stream);

pa_status_t pa_decode_v2_q(void *out, const void *query, const void *key_cache,
                           const void *value_cache, const int32_t *block_tables,
                           const int32_t *seq_lens, int num_seqs, int q_len, int num_q_heads,
                           int num_kv_heads, int head_dim, int block_size, int num_blocks,
                           int max_blocks_per_seq, int max_seq_len, float scale,
                           pa_dtype_t dtype, int partition_size, void *workspace,
                           size_t workspace_bytes, void *stream);

/*
 * Tiled prefill: the same computation as pa_decode_v1_q / pa_decode_v2_q (same
 * arguments, layouts, workspace and causal rule: query j of q_len sees cache
 * tokens 0 .. L - q_len + j), on a kernel built for many (query token, head)
 * columns per kv head, i.e. prefill-like q_len (the [kv_h, gqa, q_len, tile]
 * batching of commit 490ff98, paged_attn.py, taken to long q_len; partition
 * partials and their merge as in commit 15ef28e, "[OPT] PagedAttention V2
 * implementation").  Each wave holds column_tiles tiles of 16 columns and reads
 * every key/value block of its range once for all of them, so the cache is
 * re-read once per 64 * column_tiles columns instead of once per 16.
 *   column_tiles: 1, 2 or 4; 0 lets the library choose.  Other values give
 *                 PA_ERR_INVALID_ARGUMENT.
 *   dtype:        PA_DTYPE_BF16 only (PA_ERR_UNSUPPORTED for fp32).
 * pa_prefill_v1 makes one pass per sequence; pa_prefill_v2 writes one partial
 * per partition of partition_size tokens into the workspace (sized as for
 * pa_decode_v2_q) and merges them.  Results agree with the _q entry points to
 * rounding, not bit for bit: weights are taken against a running reference
 * max that moves in steps (kept below 2^8 relative to it), which changes the
 * rounding, not the value.
 */
pa_status_t pa_prefill_v1(void *out, const void *query, const void *key_cache,
                          const void *value_cache, const int32_t *block_tables,
                          const int32_t *seq_lens, int num_seqs, int q_len, int num_q_heads,
                          int num_kv_heads, int head_dim, int block_size, int num_blocks,
                          int max_blocks_per_seq, int max_seq_len, float scale, pa_dtype_t dtype,
                          int column_tiles, void *stream);

pa_status_t pa_prefill_v2(void *out, const void *query, const void *key_cache,
                          const void *value_cache, const int32_t *block_tables,
                          const int32_t *seq_lens, int num_seqs, int q_len, int num_q_heads,
                          int num_kv_heads, int head_dim, int block_size, int num_blocks,
                          int max_blocks_per_seq, int max_seq_len, float scale, pa_dtype_t dtype,
                          int partition_size, void *workspace, size_t workspace_bytes,
                          int column_tiles, void *stream);

/*
 * Kernel that pa_decode_v1_q (single_pass = 1) or pa_decode_v2_q (single_pass
 * = 0, partitions of partition_size tokens) runs for this shape: 0 = the decode
 * kernel (16 (query token, head) columns per workgroup, the blocks of a
 * partition split over its waves); 1 or 2 = the tiled prefill kernel of
 * pa_prefill_v1 / pa_prefill_v2 with that many 16-column tiles per wave.  The
 * prefill kernel is chosen for bf16 when a kv head has at least 64 (single
 * pass) or 128 (split) columns G * q_len and the grid keeps enough waves for
 * the device's compute units (two tiles at two or more waves per SIMD; one
 * tile otherwise, or -- single pass -- the decode kernel below one wave per
 * SIMD).  Invalid arguments give 0.  Host-only; 256 compute units are assumed
 * when no device is visible.
 */
int pa_select_q_kernel(int single_pass, int num_seqs, int q_len, int num_q_heads, int num_kv_heads,
                       pa_dtype_t dtype, int max_seq_len, int partition_size);

/* V2 Phase 1 alone: fills the workspace partials (layout at pa_workspace_size)
 * for partitions p < ceil(L / partition_size) of each sequence, one entry per
 * partition; other entries are not written.  Same arguments as pa_decode_v2,
 * without out (partition_size = 0 as there). */
pa_status_t pa_decode_v2_partials(const void *query, const void *key_cache,
                                  const void *value_cache, const int32_t *block_tables,
                                  const int32_t *seq_lens, int num_seqs, int num_q_heads,
                                  int num_kv_heads, int head_dim, int block_size, int num_blocks,
                                  int max_blocks_per_seq, int max_seq_len, float scale,
                                  pa_dtype_t dtype, int partition_size, void *workspace,
                                  size_t workspace_bytes, void *stream);

/* V2 Phase 1 alone, exactly as pa_decode_v2 runs it, and the tokens behind each
 * workspace entry it writes (*entry_tokens, may be NULL).  When partitions are
 * many, that is one entry per partition (entry_tokens = partition_size).  When
 * they are few (fewer than four per compute unit over all sequences and kv
 * heads), Phase 1 splits each (sequence, kv head) into equal spans of blocks,
 * about one span per compute unit, cutting the partitions wherever the spans
 * fall: a workgroup computes each partition piece in its span (merged across its
 * waves as in Phase 1), folds the pieces in order with the Phase-2 rescale, and
 * writes one entry per span -- the same layout and meaning as a partition's
 * entry, over the span's tokens (entry_tokens = the span, a multiple of 16, so
 * entry e of a row covers tokens [e * entry_tokens, (e + 1) * entry_tokens)).
 * Same arguments as pa_decode_v2, without out; partition_size = 0 as there.
 * pa_decode_v2 is this call followed by pa_decode_v2_reduce_entries, bit for
 * bit. */
pa_status_t pa_decode_v2_groups(const void *query, const void *key_cache,
                                const void *value_cache, const int32_t *block_tables,
                                const int32_t *seq_lens, int num_seqs, int num_q_heads,
                                int num_kv_heads, int head_dim, int block_size, int num_blocks,
                                int max_blocks_per_seq, int max_seq_len, float scale,
                                pa_dtype_t dtype, int partition_size, void *workspace,
                                size_t workspace_bytes, int *entry_tokens, void *stream);

/* V2 Phase 2 over workspace entries of entry_tokens tokens each (>= 1; else
 * PA_ERR_INVALID_ARGUMENT), as pa_decode_v2_groups writes them: reads the
 * ceil(L / entry_tokens) entries of each row.  partition_size gives the
 * workspace layout (pa_workspace_size); the entries of a row must fit it,
 * ceil(max_seq_len / entry_tokens) <= ceil(max_seq_len / partition_size), else
 * PA_ERR_INVALID_SHAPE. */
pa_status_t pa_decode_v2_reduce_entries(void *out, const int32_t *seq_lens, int num_seqs,
                                        int num_q_heads, int head_dim, int max_seq_len,
                                        pa_dtype_t dtype, int partition_size, int entry_tokens,
                                        const void *workspace, size_t workspace_bytes,
                                        void *stream);

/* Repack of token-major caches into the split layout above, for callers that
 * store K and V as [num_blocks][num_kv_heads][block_size][head_dim] (K[t][d]
 * and V[t][d] of slot t at [..][t][d]).  The pages gather a sequence's blocks
 * by id and permute each into token order, leaving the in-block order to the
 * storage layout (commit 15ef28e, "[OPT] Vectorize paged_attention_v2"); this
 * call moves a token-major cache into the order the kernels read, bit for bit.
 *   key_out, value_out  the key_cache / value_cache layouts above (written)
 *   key_in, value_in    token-major caches (read only)
 * Either pair may be NULL to skip that cache, not both; an output must not
 * overlap its input (PA_ERR_INVALID_ARGUMENT).  block_size must be 16,
 * head_dim a multiple of x and at most 512 (PA_ERR_UNSUPPORTED); dtype
 * PA_DTYPE_F32 or PA_DTYPE_BF16; pointers 16-byte aligned.  num_blocks == 0
 * enqueues nothing.  Every pointer is caller-owned device memory; the call
 * allocates nothing and is enqueued on `stream`. */
pa_status_t pa_cache_from_token_major(void *key_out, void *value_out, const void *key_in,
                                      const void *value_in, int num_blocks, int num_kv_heads,
                                      int head_dim, int block_size, pa_dtype_t dtype, void *stream);

/*
 * pa_decode_v2 for callers that cannot allocate: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc.  Same arguments as
 * pa_decode_v2 without the workspace, same results bit for bit.  The workspace
 * is a file-scope device array of PA_NOALLOC_SCRATCH_BYTES in the library (one
 * per device, held until the process ends; its device address is looked up
 * once per device, on the first call with that device current).  The call
 * allocates nothing -- no hipMalloc, no hipFree, no allocating library
 * routine -- and needs nothing in the array cleared: Phase 1 writes every
 * entry Phase 2 reads.  Returns PA_ERR_WORKSPACE_TOO_SMALL, having launched
 * nothing, when pa_workspace_size for the problem (with the partition size in
 * use; partition_size = 0 as in pa_decode_v2) exceeds PA_NOALLOC_SCRATCH_BYTES,
 * and PA_ERR_HIP if the array's address cannot be obtained.  Every call on one
 * device shares that device's array: calls that may overlap on one device (two
 * streams, or two host threads) race and must be ordered by the caller; calls
 * in order on one stream are safe.
 */
#define PA_NOALLOC_SCRATCH_BYTES (64u << 20)

pa_status_t pa_decode_v2_noalloc(void *out, const void *query, const void *key_cache,
                                 const void *value_cache, const int32_t *block_tables,
                                 const int32_t *seq_lens, int num_seqs, int num_q_heads,
                                 int num_kv_heads, int head_dim, int block_size, int num_blocks,
                                 int max_blocks_per_seq, int max_seq_len, float scale,
                                 pa_dtype_t dtype, int partition_size, void *stream);

/* V2 Phase 2 alone: merges the workspace partials into out with the
 * log-sum-exp rescale (commit 15ef28e, "[OPT] PagedAttention V2
 * implementation", Phase 2).  Reads only partitions p < ceil(L / partition_size)
 * of each sequence, one entry per partition as pa_decode_v2_partials writes
 * them.  partition_size must be the explicit size (0 is not accepted here). */
pa_status_t pa_decode_v2_reduce(void *out, const int32_t *seq_lens, int num_seqs, int num_q_heads,
                                int head_dim, int max_seq_len, pa_dtype_t dtype,
                                int partition_size, const void *workspace, size_t workspace_bytes,
                                void *stream);

/*
 * Dispatch rule between V1 and V2: returns 1 (use V2) iff max_seq_len > 8192,
 * the threshold of commit 900ae0b ("THE SINGLE HIGHEST-IMPACT CODE CHANGE")
 * and commit 490ff98 ("Three changes", item 1); 0 otherwise.  The other
 * arguments are accepted for future occupancy-aware rules and are not used.
 */
int pa_select_v2(int max_seq_len, int num_seqs, int num_kv_heads, int partition_size);

/* pa_decode_v1 or pa_decode_v2, chosen by pa_select_v2.  The workspace is only
 * required (and only checked) when V2 is chosen. */
pa_status_t pa_decode(void *out, const void *query, const void *key_cache, const void *value_cache,
                      const int32_t *block_tables, const int32_t *seq_lens, int num_seqs,
                      int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                      int num_blocks, int max_blocks_per_seq, int max_seq_len, float scale,
                      pa_dtype_t dtype, int partition_size, void *workspace,
                      size_t workspace_bytes, void *stream);

/*
 * Dispatch rule derived from measurements on MI355X (256 compute units), for the
 * same choice.  Returns 1 (V2) when max_seq_len > 8192, as pa_select_v2 does:
 * above that, V1 would leave one long sequence as a straggler, and the host
 * does not know the individual lengths.  Returns 0 (V1) when
 * max_seq_len <= 1024.  In between, returns 1 iff the V1 grid, one workgroup per
 * (sequence, kv head), would occupy fewer than half of the current device's
 * compute units (2 * num_seqs * num_kv_heads < CUs); there the pages' rule picks
 * V1, which measured up to 4x slower.  Falls back to pa_select_v2 when the
 * compute-unit count is unknown.  partition_size is not used.
 */
int pa_select_v2_auto(int max_seq_len, int num_seqs, int num_kv_heads, int partition_size);

/* pa_decode_v1 or pa_decode_v2, chosen by pa_select_v2_auto. */
pa_status_t pa_decode_auto(void *out, const void *query, const void *key_cache,
                           const void *value_cache, const int32_t *block_tables,
                           const int32_t *seq_lens, int num_seqs, int num_q_heads,
                           int num_kv_heads, int head_dim, int block_size, int num_blocks,
                           int max_blocks_per_seq, int max_seq_len, float scale, pa_dtype_t dtype,
                           int partition_size, void *workspace, size_t workspace_bytes,
                           void *stream);

#ifdef __cplusplus
}
#endif

#endif /* PA_DECODE_H */
