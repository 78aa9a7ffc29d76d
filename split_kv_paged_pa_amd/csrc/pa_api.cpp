// pa_api.cpp -- the C ABI of libpa_decode.so (declared in include/pa_decode.h):
// host-side argument checks, workspace carving, V1/V2 dispatch, launches.
// Every check happens before anything is enqueued; nothing here allocates,
// synchronises or reads device memory.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdint>
#include <mutex>

#include "../../include/pa_decode.h"
#include "pa_launch.h"

namespace {

constexpr int kBlockTokens = 16;
constexpr int kMaxGroup = 16;
constexpr int kMaxGridYZ = 65535;
// V2 is used above this many tokens: the threshold of commit 900ae0b
// ("THE SINGLE HIGHEST-IMPACT CODE CHANGE") and commit 490ff98 ("Three changes").
constexpr int kV2MinSeqLen = 8192;
// Measured on MI355X: V1 (one workgroup per (sequence, kv head)) already wins at
// or below this many tokens, whatever the batch.
constexpr int kV1ShortSeqLen = 1024;
constexpr size_t kAlign = 256;
// Arrival counters of the single-launch V2, one per (sequence, kv head), at the
// start of every workspace.
constexpr size_t kHeaderBytes = PA_WORKSPACE_HEADER_BYTES;
constexpr long long kTicketSlots = (long long)(kHeaderBytes / sizeof(uint32_t));

// Phase 1 groups consecutive partitions of one (sequence, kv head) into one
// workgroup when there are few partitions overall (at most kGroupFewUnits per
// compute unit): one long-running workgroup per compute unit streams faster on
// MI355X than two shorter ones sharing a unit.
constexpr int kGroupFewUnits = 4;
constexpr int kMaxDevices = 64;

// Partition size the library picks (partition_size = 0): measured on MI355X over
// the 100K-token sequence (32/4 heads), 16 ragged sequences up to 32K tokens, 64
// ragged sequences up to 131K tokens and 8 x 131K tokens (GQA 5), at P = 256 ..
// 16384: 2048 is within 2% of the best size on every batch (1024 ties, 4096
// loses up to 2x on the 64-sequence batch, 256 and 512 lose 3-20%); when
// (sequence, kv head) pairs are so few that 2048-token partitions give fewer
// work units than compute units, one partition per compute unit is faster (the
// 100K-token step at P = 1568: 39.4 us against 39.9 us at 2048 and 40.4 us at
// 1024).
constexpr int kAutoPartition = 2048;
constexpr int kAutoPartitionMin = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Compute units of the current device (cached per device; 0 if unknown).
int compute_units() {
    static std::atomic<int> cache[kMaxDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
    if (dev < kMaxDevices) {
        const int c = cache[dev].load(std::memory_order_relaxed);
        if (c > 0) return c;
    }
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) n = 0;
    if (n > 0 && dev < kMaxDevices) cache[dev].store(n, std::memory_order_relaxed);
    return n;
}

// Partitions per Phase-1 workgroup for S * Hkv * P_max units.
int partitions_per_group(long long units) {
    const int cus = compute_units();
    if (cus <= 0 || units <= cus || units > (long long)kGroupFewUnits * cus) return 1;
    return (int)((units + cus - 1) / cus);
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct Layout {
    int max_parts;
    size_t tmp_off, exp_off, max_off, total;
};

// Workspace layout; false if the sizes are invalid.
bool layout(int num_seqs, int num_q_heads, int head_dim, int max_seq_len, int partition_size,
            Layout *out) {
    if (num_seqs < 0 || num_q_heads <= 0 || head_dim <= 0 || max_seq_len < 0) return false;
    if (partition_size < kBlockTokens || partition_size % kBlockTokens != 0) return false;
    const long long parts = max_seq_len > 0
                                ? ((long long)max_seq_len + partition_size - 1) / partition_size
                                : 0;
    const unsigned long long rows = (unsigned long long)num_seqs * num_q_heads * parts;
    const unsigned long long tmp = rows * head_dim * sizeof(float);
    const unsigned long long vec = rows * sizeof(float);
    if (rows && (tmp / rows / sizeof(float) != (unsigned long long)head_dim)) return false;
    out->max_parts = (int)parts;
    out->tmp_off = kHeaderBytes;
    out->exp_off = out->tmp_off + align_up(tmp);
    out->max_off = out->exp_off + align_up(vec);
    out->total = rows ? out->max_off + align_up(vec) : 0;
    return true;
}

pa_status_t check_problem(const void *query, const void *key_cache, const void *value_cache,
                          const int32_t *block_tables, const int32_t *seq_lens, int num_seqs,
                          int q_len, int num_q_heads, int num_kv_heads, int head_dim,
                          int block_size, int num_blocks, int max_blocks_per_seq, int max_seq_len,
                          float scale, pa_dtype_t dtype) {
    if (num_seqs < 0 || q_len <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
        block_size <= 0 || num_blocks < 0 || max_blocks_per_seq < 0 || max_seq_len < 0)
        return PA_ERR_INVALID_SHAPE;
    if (num_q_heads % num_kv_heads != 0) return PA_ERR_INVALID_SHAPE;
    if ((long long)max_seq_len > (long long)max_blocks_per_seq * block_size)
        return PA_ERR_INVALID_SHAPE;
    if (dtype != PA_DTYPE_F32 && dtype != PA_DTYPE_BF16) return PA_ERR_INVALID_ARGUMENT;
    if (!std::isfinite(scale)) return PA_ERR_INVALID_ARGUMENT;
    if (head_dim != 64 && head_dim != 128) return PA_ERR_UNSUPPORTED;
    if (block_size != kBlockTokens) return PA_ERR_UNSUPPORTED;
    if (num_q_heads / num_kv_heads > kMaxGroup) return PA_ERR_UNSUPPORTED;
    // 16 (query token, head) columns per workgroup: kv heads * column chunks workgroups in y.
    const long long chunks = ((long long)(num_q_heads / num_kv_heads) * q_len + 15) / 16;
    if ((long long)num_kv_heads * chunks > kMaxGridYZ) return PA_ERR_UNSUPPORTED;
    if (num_seqs > kMaxGridYZ) return PA_ERR_UNSUPPORTED;
    if (num_seqs == 0) return PA_OK;
    if (!query || !key_cache || !value_cache || !block_tables || !seq_lens)
        return PA_ERR_NULL_POINTER;
    if (!aligned16(query) || !aligned16(key_cache) || !aligned16(value_cache))
        return PA_ERR_INVALID_ARGUMENT;
    return PA_OK;
}

pa::Problem make_problem(const void *query, const void *key_cache, const void *value_cache,
                         const int32_t *block_tables, const int32_t *seq_lens, int num_seqs,
                         int q_len, int num_q_heads, int num_kv_heads, int head_dim,
                         int num_blocks, int max_blocks_per_seq, int max_seq_len, float scale,
                         pa_dtype_t dtype) {
    pa::Problem pb;
    pb.qlen = q_len;
    pb.query = query;
    pb.key_cache = key_cache;
    pb.value_cache = value_cache;
    pb.block_tables = block_tables;
    pb.seq_lens = seq_lens;
    pb.num_seqs = num_seqs;
    pb.num_q_heads = num_q_heads;
    pb.num_kv_heads = num_kv_heads;
    pb.head_dim = head_dim;
    pb.num_blocks = num_blocks;
    pb.max_blocks = max_blocks_per_seq;
    pb.max_seq_len = max_seq_len;
    pb.scale = scale;
    pb.dtype = dtype == PA_DTYPE_BF16 ? pa::Dtype::BF16 : pa::Dtype::F32;
    return pb;
}

// Checks the V2 workspace and carves it.
pa_status_t carve(int num_seqs, int num_q_heads, int num_kv_heads, int head_dim, int max_seq_len,
                  int partition_size, void *workspace, size_t workspace_bytes,
                  pa::Partials *parts) {
    if (partition_size < kBlockTokens || partition_size % kBlockTokens != 0)
        return PA_ERR_UNSUPPORTED;
    if ((long long)max_seq_len + partition_size > 0x7fffffffLL) return PA_ERR_UNSUPPORTED;
    Layout lay;
    if (!layout(num_seqs, num_q_heads, head_dim, max_seq_len, partition_size, &lay))
        return PA_ERR_INVALID_SHAPE;
    if (workspace_bytes < lay.total) return PA_ERR_WORKSPACE_TOO_SMALL;
    if (lay.total > 0 && !workspace) return PA_ERR_NULL_POINTER;
    if (lay.total > 0 && !aligned16(workspace)) return PA_ERR_INVALID_ARGUMENT;
    // A problem with nothing to hold may come with a NULL workspace: carve only a real one.
    char *base = static_cast<char *>(workspace);
    parts->tickets = reinterpret_cast<uint32_t *>(base);
    parts->tmp_out = base ? reinterpret_cast<float *>(base + lay.tmp_off) : nullptr;
    parts->exp_sums = base ? reinterpret_cast<float *>(base + lay.exp_off) : nullptr;
    parts->max_logits = base ? reinterpret_cast<float *>(base + lay.max_off) : nullptr;
    parts->partition_size = partition_size;
    parts->max_parts = lay.max_parts;
    parts->per_group = partitions_per_group((long long)num_seqs * num_kv_heads * lay.max_parts);
    parts->span_blocks = 0;
    parts->span_count = 0;
    parts->entry_tokens = partition_size;
    parts->marked_entries = -1;
    return PA_OK;
}

pa_status_t from_hip(hipError_t e) { return e == hipSuccess ? PA_OK : PA_ERR_HIP; }

// Equal spans serve a batch whose partitions make at most kGroupFewUnits
// workgroups per compute unit, when each (sequence, kv head, column chunk) row
// gets at least two spans (ny rows per sequence).  Also when the partitions make
// exactly one workgroup per CU, as the library's own partition size does for a
// few long rows: the spans then cut the same blocks and Phase 2 skips its
// seq_lens round trip (measured on MI355X, the 100K-token step at P = 1568:
// 36.4 us per partition against 36.0 us for the spans at P = 512, same run).
bool use_spans(int num_seqs, int ny, int max_parts) {
    int cus = compute_units();
    if (cus <= 0) return false;
    const long long rows = (long long)num_seqs * ny;
    return rows * max_parts <= (long long)kGroupFewUnits * cus && 2 * rows <= cus &&
           max_parts >= 2;
}

// Phase-1 spans for the grouped form (few work units: use_spans).  Each
// of the ny (kv head, column chunk) rows of a sequence is split into W equal
// spans of blocks, W = CUs / (num_seqs * ny) -- one workgroup per compute unit --
// but at most max_parts (the entries a workspace row holds); each span is one
// partition of its workgroup, whatever boundaries of the caller's partition size
// fall inside it.  Measured on MI355X, one 100K-token sequence with 4 kv heads
// (64 spans of 98 blocks per kv head, 256 workgroups, against 196 workgroups of
// two whole 1024-token partitions each): the step 40.42 -> 40.12 us at P 1024
// and 40.92 -> 40.68 us at P 512 with the caller's partitions closed inside the
// spans, 36.9 us at both once the span is one partition.
void grouped_spans(int num_seqs, int ny, int max_seq_len, pa::Partials *parts) {
    const long long nblk = ((long long)max_seq_len + kBlockTokens - 1) / kBlockTokens;
    const int cus = compute_units();
    long long w = cus > 0 ? cus / ((long long)num_seqs * ny) : 1;
    if (w > parts->max_parts) w = parts->max_parts;
    if (w < 1) w = 1;
    const long long span = nblk > 0 ? (nblk + w - 1) / w : 1;
    parts->span_blocks = (int)span;  // <= nblk <= INT_MAX / 16
    parts->span_count = nblk > 0 ? (int)((nblk + span - 1) / span) : 1;
}

// Kernel selection of decode_v1 / decode_v2 (their tiles argument):
//   0          the decode kernel;
//   1, 2, 4    the prefill kernel with that many 16-column tiles per wave (bf16);
//   kAuto      the library's choice between the two (auto_tiles);
//   kAutoPrefill  the prefill kernel, tiles chosen by the library.
constexpr int kAuto = -1;
constexpr int kAutoPrefill = -2;

pa_status_t check_tiles(int tiles, pa_dtype_t dtype) {
    if (tiles == 0 || tiles == kAuto) return PA_OK;
    if (tiles != 1 && tiles != 2 && tiles != 4 && tiles != kAutoPrefill)
        return PA_ERR_INVALID_ARGUMENT;
    return dtype == PA_DTYPE_BF16 ? PA_OK : PA_ERR_UNSUPPORTED;
}

// Kernel for the q_len entry points (tiles argument of decode_v1 / decode_v2):
// 0 = the decode kernel (16 columns per workgroup, blocks split over its waves),
// 1 or 2 = the prefill kernel with that many 16-column tiles per wave.  The
// prefill kernel reads each key/value block once per 64 * tiles columns instead
// of once per 16, which pays once a kv head has many (query token, head)
// columns and the grid still has enough waves: two tiles when that leaves at
// least two waves per SIMD, one tile when it leaves one (single pass) or when
// the partitions make up the parallelism (split-KV).  Measured on MI355X
// (S 1, Hq 32, Hkv 4, D 128): q_len 512 / 8192 tokens 216 -> 185 us single pass,
// 321 -> 147 us split at P 1024; q_len 8 keeps the decode kernel.
// prefill_only: the caller asked for the prefill kernel; the answer is then
// 1 or 2, never 0.
int auto_tiles(bool single_pass, bool prefill_only, int num_seqs, int num_kv_heads, int group,
               int q_len, pa_dtype_t dtype, int max_parts) {
    if (dtype != PA_DTYPE_BF16) return 0;
    const long long cols = (long long)group * q_len;
    if (!prefill_only && cols < (single_pass ? 64 : 128)) return 0;
    int cus = compute_units();
    if (cus <= 0) cus = 256;
    const long long units = (long long)num_seqs * num_kv_heads * (single_pass ? 1 : max(max_parts, 1));
    if (units * ((cols + 31) / 32) >= 8LL * cus) return 2;
    if (!single_pass || prefill_only) return 1;
    return units * ((cols + 15) / 16) >= 4LL * cus ? 1 : 0;
}

// The single launch applies when every (sequence, kv head) has a counter slot
// and the last workgroup's merge fits its weight table.
bool fused_fits(int num_seqs, int num_q_heads, int num_kv_heads, const pa::Partials &parts) {
    if (parts.max_parts <= 0) return false;
    if ((long long)num_seqs * num_kv_heads > kTicketSlots) return false;
    const long long groups = (parts.max_parts + parts.per_group - 1) / parts.per_group;
    return (long long)(num_q_heads / num_kv_heads) * groups <= pa::fused_merge_capacity();
}

}  // namespace

extern "C" {

const char *pa_status_string(pa_status_t status) {
    switch (status) {
        case PA_OK: return "PA_OK";
        case PA_ERR_NULL_POINTER: return "PA_ERR_NULL_POINTER: a required pointer is NULL";
        case PA_ERR_INVALID_SHAPE: return "PA_ERR_INVALID_SHAPE: negative or inconsistent sizes";
        case PA_ERR_UNSUPPORTED: return "PA_ERR_UNSUPPORTED: shape outside the supported set";
        case PA_ERR_WORKSPACE_TOO_SMALL: return "PA_ERR_WORKSPACE_TOO_SMALL";
        case PA_ERR_HIP: return "PA_ERR_HIP: a HIP launch failed";
        case PA_ERR_INVALID_ARGUMENT:
            return "PA_ERR_INVALID_ARGUMENT: bad dtype, non-finite scale or misaligned pointer";
    }
    return "unknown pa_status_t";
}

size_t pa_workspace_size(int num_seqs, int num_q_heads, int head_dim, int max_seq_len,
                         int partition_size) {
    Layout lay;
    if (!layout(num_seqs, num_q_heads, head_dim, max_seq_len, partition_size, &lay)) return 0;
    return lay.total;
}

pa_status_t pa_workspace_layout(int num_seqs, int num_q_heads, int head_dim, int max_seq_len,
                                int partition_size, size_t *tmp_output_offset,
                                size_t *exp_sums_offset, size_t *max_logits_offset,
                                int *max_partitions) {
    Layout lay;
    if (!layout(num_seqs, num_q_heads, head_dim, max_seq_len, partition_size, &lay))
        return PA_ERR_INVALID_SHAPE;
    if (tmp_output_offset) *tmp_output_offset = lay.tmp_off;
    if (exp_sums_offset) *exp_sums_offset = lay.exp_off;
    if (max_logits_offset) *max_logits_offset = lay.max_off;
    if (max_partitions) *max_partitions = lay.max_parts;
    return PA_OK;
}

pa_status_t pa_workspace_init(void *workspace, size_t workspace_bytes, void *stream) {
    if (!workspace) return PA_ERR_NULL_POINTER;
    if (workspace_bytes < kHeaderBytes) return PA_ERR_WORKSPACE_TOO_SMALL;
    if (!aligned16(workspace)) return PA_ERR_INVALID_ARGUMENT;
    return from_hip(pa::launch_zero_words(static_cast<uint32_t *>(workspace),
                                          (int)(kHeaderBytes / sizeof(uint32_t)),
                                          static_cast<hipStream_t>(stream)));
}

pa_status_t pa_cache_from_token_major(void *key_out, void *value_out, const void *key_in,
                                      const void *value_in, int num_blocks, int num_kv_heads,
                                      int head_dim, int block_size, pa_dtype_t dtype, void *stream) {
    if (num_blocks < 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0)
        return PA_ERR_INVALID_SHAPE;
    if (dtype != PA_DTYPE_F32 && dtype != PA_DTYPE_BF16) return PA_ERR_INVALID_ARGUMENT;
    const int es = dtype == PA_DTYPE_BF16 ? 2 : 4;
    if (block_size != kBlockTokens || head_dim % (16 / es) != 0 || head_dim > pa::repack_max_dim())
        return PA_ERR_UNSUPPORTED;
    if ((key_in == nullptr) != (key_out == nullptr) || (value_in == nullptr) != (value_out == nullptr) ||
        (key_in == nullptr && value_in == nullptr))
        return PA_ERR_NULL_POINTER;
    const size_t bytes = (size_t)num_blocks * num_kv_heads * kBlockTokens * head_dim * es;
    auto overlaps = [bytes](const void *a, const void *b) {
        const char *x = static_cast<const char *>(a), *y = static_cast<const char *>(b);
        return x < y + bytes && y < x + bytes;
    };
    for (const void *p : {static_cast<const void *>(key_out), static_cast<const void *>(value_out), key_in, value_in})
        if (p != nullptr && !aligned16(p)) return PA_ERR_INVALID_ARGUMENT;
    if (key_in && (overlaps(key_out, key_in) || (value_in && overlaps(key_out, value_in))))
        return PA_ERR_INVALID_ARGUMENT;
    if (value_in && (overlaps(value_out, value_in) || (key_in && overlaps(value_out, key_in))))
        return PA_ERR_INVALID_ARGUMENT;
    if (key_in && value_in && overlaps(key_out, value_out)) return PA_ERR_INVALID_ARGUMENT;
    if (num_blocks == 0) return PA_OK;
    return from_hip(pa::launch_repack(key_in, value_in, key_out, value_out, num_blocks, num_kv_heads,
                                      head_dim, dtype == PA_DTYPE_BF16 ? pa::Dtype::BF16 : pa::Dtype::F32,
                                      static_cast<hipStream_t>(stream)));
}

int pa_select_partition_size(int num_seqs, int num_kv_heads, int max_seq_len) {
    if (num_seqs <= 0 || num_kv_heads <= 0 || max_seq_len <= 0) return kAutoPartition;
    int cus = compute_units();
    if (cus <= 0) cus = 256;
    const long long pairs = (long long)num_seqs * num_kv_heads;
    const long long units = pairs * (((long long)max_seq_len + kAutoPartition - 1) / kAutoPartition);
    if (units >= cus) return kAutoPartition;
    // pairs < cus here: k partitions per pair make at most one unit per compute unit.
    const long long k = cus / pairs;
    long long p = ((long long)max_seq_len + k - 1) / k;
    p = (p + kBlockTokens - 1) / kBlockTokens * kBlockTokens;
    if (p < kAutoPartitionMin) p = kAutoPartitionMin;
    if (p > kAutoPartition) p = kAutoPartition;
    return (int)p;
}

int pa_select_v2(int max_seq_len, int num_seqs, int num_kv_heads, int partition_size) {
    (void)num_seqs;
    (void)num_kv_heads;
    (void)partition_size;
    return max_seq_len > kV2MinSeqLen ? 1 : 0;
}

}  // extern "C"

namespace {

pa_status_t decode_v1(void *out, const void *query, const void *key_cache,
                      const void *value_cache, const int32_t *block_tables,
                      const int32_t *seq_lens, int num_seqs, int q_len, int num_q_heads,
                      int num_kv_heads, int head_dim, int block_size, int num_blocks,
                      int max_blocks_per_seq, int max_seq_len, float scale, pa_dtype_t dtype,
                      int tiles, void *stream) {
    pa_status_t st = check_problem(query, key_cache, value_cache, block_tables, seq_lens, num_seqs,
                                   q_len, num_q_heads, num_kv_heads, head_dim, block_size,
                                   num_blocks, max_blocks_per_seq, max_seq_len, scale, dtype);
    if (st != PA_OK) return st;
    st = check_tiles(tiles, dtype);
    if (st != PA_OK || num_seqs == 0) return st;
    if (tiles < 0)
        tiles = auto_tiles(true, tiles == kAutoPrefill, num_seqs, num_kv_heads,
                           num_q_heads / num_kv_heads, q_len, dtype, 1);
    if (!out) return PA_ERR_NULL_POINTER;
    if (!aligned16(out)) return PA_ERR_INVALID_ARGUMENT;
    pa::Problem pb = make_problem(query, key_cache, value_cache, block_tables, seq_lens, num_seqs,
                                  q_len, num_q_heads, num_kv_heads, head_dim, num_blocks,
                                  max_blocks_per_seq, max_seq_len, scale, dtype);
    hipStream_t hs = static_cast<hipStream_t>(stream);
    if (tiles > 0) return from_hip(pa::launch_prefill(pb, nullptr, out, tiles, hs));
    return from_hip(pa::launch_single_pass(pb, out, hs));
}

// What decode_v2 runs: both phases; Phase 1 alone with one workspace entry per
// partition; or Phase 1 alone as the two-phase form runs it (entries of equal
// block spans when partitions are few), reporting the tokens per entry.
enum class V2Run { kBoth, kPartitions, kEntries };

// V2 Phase 1 (+ Phase 2 for kBoth).  With q_len query tokens per sequence the
// partials have q_len * num_q_heads rows per sequence.  tiles > 0: Phase 1 on
// the prefill kernel with that many column tiles per wave.
pa_status_t decode_v2(void *out, V2Run run, int *entry_tokens_out, const void *query,
                      const void *key_cache,
                      const void *value_cache, const int32_t *block_tables,
                      const int32_t *seq_lens, int num_seqs, int q_len, int num_q_heads,
                      int num_kv_heads, int head_dim, int block_size, int num_blocks,
                      int max_blocks_per_seq, int max_seq_len, float scale, pa_dtype_t dtype,
                      int partition_size, void *workspace, size_t workspace_bytes, int tiles,
                      void *stream) {
    pa_status_t st = check_problem(query, key_cache, value_cache, block_tables, seq_lens, num_seqs,
                                   q_len, num_q_heads, num_kv_heads, head_dim, block_size,
                                   num_blocks, max_blocks_per_seq, max_seq_len, scale, dtype);
    if (st != PA_OK) return st;
    st = check_tiles(tiles, dtype);
    if (st != PA_OK) return st;
    const long long rows_per_seq = (long long)q_len * num_q_heads;
    if (rows_per_seq > 0x7fffffffLL) return PA_ERR_UNSUPPORTED;
    // Workgroups per (sequence, partition group): kv heads times column chunks.
    const int chunks = (int)(((long long)(num_q_heads / num_kv_heads) * q_len + 15) / 16);
    if (partition_size == 0)
        partition_size = pa_select_partition_size(num_seqs, num_kv_heads * chunks, max_seq_len);
    pa::Partials parts;
    st = carve(num_seqs, (int)rows_per_seq, num_kv_heads * chunks, head_dim, max_seq_len,
               partition_size, workspace, workspace_bytes, &parts);
    if (st != PA_OK) return st;
    if (tiles < 0)
        tiles = auto_tiles(false, tiles == kAutoPrefill, num_seqs, num_kv_heads,
                           num_q_heads / num_kv_heads, q_len, dtype, parts.max_parts);
    // Few partitions: Phase 1 in equal spans, one entry per span (not on the
    // prefill kernel, and not when the per-partition partials were asked for).
    const bool grouped = run != V2Run::kPartitions && tiles <= 0 &&
                         use_spans(num_seqs, num_kv_heads * chunks, parts.max_parts);
    if (grouped) {
        grouped_spans(num_seqs, num_kv_heads * chunks, max_seq_len, &parts);
    }
    if (entry_tokens_out)
        *entry_tokens_out = grouped ? parts.span_blocks * kBlockTokens : partition_size;
    if (num_seqs == 0) return PA_OK;
    const bool want_out = run == V2Run::kBoth;
    if (want_out && !out) return PA_ERR_NULL_POINTER;
    if (want_out && !aligned16(out)) return PA_ERR_INVALID_ARGUMENT;
    hipStream_t hs = static_cast<hipStream_t>(stream);
    pa::Problem pb = make_problem(query, key_cache, value_cache, block_tables, seq_lens, num_seqs,
                                  q_len, num_q_heads, num_kv_heads, head_dim, num_blocks,
                                  max_blocks_per_seq, max_seq_len, scale, dtype);
    if (parts.max_parts > 0) {
        if (tiles > 0) {
            st = from_hip(pa::launch_prefill(pb, &parts, nullptr, tiles, hs));
        } else if (grouped) {
            // Workgroups with several partitions fold them and write one group
            // partial each; Phase 2 merges those.
            st = from_hip(pa::launch_grouped(pb, parts, hs));
            parts.entry_tokens = parts.span_blocks * kBlockTokens;
            parts.marked_entries = parts.span_count;  // every entry of the grid written
        } else {
            st = from_hip(pa::launch_partitions(pb, parts, hs));
        }
        if (st != PA_OK || !want_out) return st;
    }
    if (!want_out) return PA_OK;
    return from_hip(pa::launch_reduce(seq_lens, num_seqs, (int)rows_per_seq, head_dim,
                                      max_seq_len, pb.dtype, parts, out, hs));
}

}  // namespace

extern "C" {

pa_status_t pa_decode_v1(void *out, const void *query, const void *key_cache,
                         const void *value_cache, const int32_t *block_tables,
                         const int32_t *seq_lens, int num_seqs, int num_q_heads, int num_kv_heads,
                         int head_dim, int block_size, int num_blocks, int max_blocks_per_seq,
                         int max_seq_len, float scale, pa_dtype_t dtype, void *stream) {
    return decode_v1(out, query, key_cache, value_cache, block_tables, seq_lens, num_seqs, 1,
                     num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                     max_blocks_per_seq, max_seq_len, scale, dtype, 0, stream);
}

pa_status_t pa_decode_v1_q(void *out, const void *query, const void *key_cache,
                           const void *value_cache, const int32_t *block_tables,
                           const int32_t *seq_lens, int num_seqs, int q_len, int num_q_heads,
                           int num_kv_heads, int head_dim, int block_size, int num_blocks,
                           int max_blocks_per_seq, int max_seq_len, float scale,
                           pa_dtype_t dtype, void *stream) {
    return decode_v1(out, query, key_cache, value_cache, block_tables, seq_lens, num_seqs, q_len,
                     num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                     max_blocks_per_seq, max_seq_len, scale, dtype, kAuto, stream);
}

pa_status_t pa_decode_v2_partials(const void *query, const void *key_cache,
                                  const void *value_cache, const int32_t *block_tables,
                                  const int32_t *seq_lens, int num_seqs, int num_q_heads,
                                  int num_kv_heads, int head_dim, int block_size, int num_blocks,
                                  int max_blocks_per_seq, int max_seq_len, float scale,
                                  pa_dtype_t dtype, int partition_size, void *workspace,
                                  size_t workspace_bytes, void *stream) {
    return decode_v2(nullptr, V2Run::kPartitions, nullptr, query, key_cache, value_cache,
                     block_tables, seq_lens,
                     num_seqs, 1, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                     max_blocks_per_seq, max_seq_len, scale, dtype, partition_size, workspace,
                     workspace_bytes, 0, stream);
}

pa_status_t pa_decode_v2_groups(const void *query, const void *key_cache,
                                const void *value_cache, const int32_t *block_tables,
                                const int32_t *seq_lens, int num_seqs, int num_q_heads,
                                int num_kv_heads, int head_dim, int block_size, int num_blocks,
                                int max_blocks_per_seq, int max_seq_len, float scale,
                                pa_dtype_t dtype, int partition_size, void *workspace,
                                size_t workspace_bytes, int *entry_tokens, void *stream) {
    return decode_v2(nullptr, V2Run::kEntries, entry_tokens, query, key_cache, value_cache,
                     block_tables, seq_lens, num_seqs, 1, num_q_heads, num_kv_heads, head_dim,
                     block_size, num_blocks, max_blocks_per_seq, max_seq_len, scale, dtype,
                     partition_size, workspace, workspace_bytes, 0, stream);
}

pa_status_t pa_decode_v2_reduce_entries(void *out, const int32_t *seq_lens, int num_seqs,
                                        int num_q_heads, int head_dim, int max_seq_len,
                                        pa_dtype_t dtype, int partition_size, int entry_tokens,
                                        const void *workspace, size_t workspace_bytes,
                                        void *stream) {
    if (num_seqs < 0 || num_q_heads <= 0 || head_dim <= 0 || max_seq_len < 0)
        return PA_ERR_INVALID_SHAPE;
    if (dtype != PA_DTYPE_F32 && dtype != PA_DTYPE_BF16) return PA_ERR_INVALID_ARGUMENT;
    if (head_dim != 64 && head_dim != 128) return PA_ERR_UNSUPPORTED;
    if (num_seqs > kMaxGridYZ) return PA_ERR_UNSUPPORTED;
    pa::Partials parts;
    pa_status_t st = carve(num_seqs, num_q_heads, 1, head_dim, max_seq_len, partition_size,
                           const_cast<void *>(workspace), workspace_bytes, &parts);
    if (st != PA_OK) return st;
    if (entry_tokens < 1) return PA_ERR_INVALID_ARGUMENT;
    if (num_seqs == 0) return PA_OK;
    if (!out || !seq_lens) return PA_ERR_NULL_POINTER;
    if (!aligned16(out)) return PA_ERR_INVALID_ARGUMENT;
    // The entries of a row must fit the row the workspace holds.
    if (max_seq_len > 0 && ((long long)max_seq_len + entry_tokens - 1) / entry_tokens > parts.max_parts)
        return PA_ERR_INVALID_SHAPE;
    parts.entry_tokens = entry_tokens;
    return from_hip(pa::launch_reduce(seq_lens, num_seqs, num_q_heads, head_dim, max_seq_len,
                                      dtype == PA_DTYPE_BF16 ? pa::Dtype::BF16 : pa::Dtype::F32,
                                      parts, out, static_cast<hipStream_t>(stream)));
}

pa_status_t pa_decode_v2_reduce(void *out, const int32_t *seq_lens, int num_seqs, int num_q_heads,
                                int head_dim, int max_seq_len, pa_dtype_t dtype,
                                int partition_size, const void *workspace, size_t workspace_bytes,
                                void *stream) {
    return pa_decode_v2_reduce_entries(out, seq_lens, num_seqs, num_q_heads, head_dim, max_seq_len,
                                       dtype, partition_size, partition_size, workspace,
                                       workspace_bytes, stream);
}

pa_status_t pa_decode_v2(void *out, const void *query, const void *key_cache,
                         const void *value_cache, const int32_t *block_tables,
                         const int32_t *seq_lens, int num_seqs, int num_q_heads, int num_kv_heads,
                         int head_dim, int block_size, int num_blocks, int max_blocks_per_seq,
                         int max_seq_len, float scale, pa_dtype_t dtype, int partition_size,
                         void *workspace, size_t workspace_bytes, void *stream) {
    return decode_v2(out, V2Run::kBoth, nullptr, query, key_cache, value_cache, block_tables,
                     seq_lens, num_seqs,
                     1, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                     max_blocks_per_seq, max_seq_len, scale, dtype, partition_size, workspace,
                     workspace_bytes, 0, stream);
}

pa_status_t pa_decode_v2_q(void *out, const void *query, const void *key_cache,
                           const void *value_cache, const int32_t *block_tables,
                           const int32_t *seq_lens, int num_seqs, int q_len, int num_q_heads,
                           int num_kv_heads, int head_dim, int block_size, int num_blocks,
                           int max_blocks_per_seq, int max_seq_len, float scale,
                           pa_dtype_t dtype, int partition_size, void *workspace,
                           size_t workspace_bytes, void *stream) {
    return decode_v2(out, V2Run::kBoth, nullptr, query, key_cache, value_cache, block_tables,
                     seq_lens, num_seqs,
                     q_len, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                     max_blocks_per_seq, max_seq_len, scale, dtype, partition_size, workspace,
                     workspace_bytes, kAuto, stream);
}

pa_status_t pa_decode_v2_single(void *out, const void *query, const void *key_cache,
                                const void *value_cache, const int32_t *block_tables,
                                const int32_t *seq_lens, int num_seqs, int num_q_heads,
                                int num_kv_heads, int head_dim, int block_size, int num_blocks,
                                int max_blocks_per_seq, int max_seq_len, float scale,
                                pa_dtype_t dtype, int partition_size, void *workspace,
                                size_t workspace_bytes, void *stream) {
    pa_status_t st = check_problem(query, key_cache, value_cache, block_tables, seq_lens, num_seqs,
                                   1, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                                   max_blocks_per_seq, max_seq_len, scale, dtype);
    if (st != PA_OK) return st;
    if (partition_size == 0)
        partition_size = pa_select_partition_size(num_seqs, num_kv_heads, max_seq_len);
    pa::Partials parts;
    st = carve(num_seqs, num_q_heads, num_kv_heads, head_dim, max_seq_len, partition_size,
               workspace, workspace_bytes, &parts);
    if (st != PA_OK || num_seqs == 0) return st;
    if (!out) return PA_ERR_NULL_POINTER;
    if (!aligned16(out)) return PA_ERR_INVALID_ARGUMENT;
    hipStream_t hs = static_cast<hipStream_t>(stream);
    pa::Problem pb = make_problem(query, key_cache, value_cache, block_tables, seq_lens, num_seqs,
                                  1, num_q_heads, num_kv_heads, head_dim, num_blocks,
                                  max_blocks_per_seq, max_seq_len, scale, dtype);
    if (parts.max_parts == 0)  // no tokens anywhere: the reduce alone writes the zero rows
        return from_hip(pa::launch_reduce(seq_lens, num_seqs, num_q_heads, head_dim, max_seq_len,
                                          pb.dtype, parts, out, hs));
    if (!fused_fits(num_seqs, num_q_heads, num_kv_heads, parts)) return PA_ERR_UNSUPPORTED;
    return from_hip(pa::launch_fused(pb, parts, out, hs));
}

pa_status_t pa_prefill_v1(void *out, const void *query, const void *key_cache,
                          const void *value_cache, const int32_t *block_tables,
                          const int32_t *seq_lens, int num_seqs, int q_len, int num_q_heads,
                          int num_kv_heads, int head_dim, int block_size, int num_blocks,
                          int max_blocks_per_seq, int max_seq_len, float scale, pa_dtype_t dtype,
                          int column_tiles, void *stream) {
    if (column_tiles == 0) column_tiles = kAutoPrefill;
    else if (column_tiles < 0) return PA_ERR_INVALID_ARGUMENT;
    return decode_v1(out, query, key_cache, value_cache, block_tables, seq_lens, num_seqs, q_len,
                     num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                     max_blocks_per_seq, max_seq_len, scale, dtype, column_tiles, stream);
}

pa_status_t pa_prefill_v2(void *out, const void *query, const void *key_cache,
                          const void *value_cache, const int32_t *block_tables,
                          const int32_t *seq_lens, int num_seqs, int q_len, int num_q_heads,
                          int num_kv_heads, int head_dim, int block_size, int num_blocks,
                          int max_blocks_per_seq, int max_seq_len, float scale, pa_dtype_t dtype,
                          int partition_size, void *workspace, size_t workspace_bytes,
                          int column_tiles, void *stream) {
    if (column_tiles == 0) column_tiles = kAutoPrefill;
    else if (column_tiles < 0) return PA_ERR_INVALID_ARGUMENT;
    return decode_v2(out, V2Run::kBoth, nullptr, query, key_cache, value_cache, block_tables,
                     seq_lens, num_seqs,
                     q_len, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                     max_blocks_per_seq, max_seq_len, scale, dtype, partition_size, workspace,
                     workspace_bytes, column_tiles, stream);
}

int pa_select_q_kernel(int single_pass, int num_seqs, int q_len, int num_q_heads, int num_kv_heads,
                       pa_dtype_t dtype, int max_seq_len, int partition_size) {
    if (num_seqs <= 0 || q_len <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 ||
        num_q_heads % num_kv_heads != 0 || max_seq_len < 0)
        return 0;
    int parts = 1;
    if (!single_pass) {
        if (partition_size < kBlockTokens || partition_size % kBlockTokens != 0) return 0;
        parts = (int)(((long long)max_seq_len + partition_size - 1) / partition_size);
    }
    return auto_tiles(single_pass != 0, false, num_seqs, num_kv_heads, num_q_heads / num_kv_heads,
                      q_len, dtype, parts);
}

int pa_select_v2_auto(int max_seq_len, int num_seqs, int num_kv_heads, int partition_size) {
    (void)partition_size;
    if (max_seq_len > kV2MinSeqLen) return 1;
    if (max_seq_len <= kV1ShortSeqLen) return 0;
    const int cus = compute_units();
    if (cus <= 0) return 0;  // unknown device: the pages' rule
    return 2LL * num_seqs * num_kv_heads < cus ? 1 : 0;
}

pa_status_t pa_decode_auto(void *out, const void *query, const void *key_cache,
                           const void *value_cache, const int32_t *block_tables,
                           const int32_t *seq_lens, int num_seqs, int num_q_heads,
                           int num_kv_heads, int head_dim, int block_size, int num_blocks,
                           int max_blocks_per_seq, int max_seq_len, float scale, pa_dtype_t dtype,
                           int partition_size, void *workspace, size_t workspace_bytes,
                           void *stream) {
    if (pa_select_v2_auto(max_seq_len, num_seqs, num_kv_heads, partition_size)) {
        return pa_decode_v2(out, query, key_cache, value_cache, block_tables, seq_lens, num_seqs,
                            num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                            max_blocks_per_seq, max_seq_len, scale, dtype, partition_size,
                            workspace, workspace_bytes, stream);
    }
    return pa_decode_v1(out, query, key_cache, value_cache, block_tables, seq_lens, num_seqs,
                        num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                        max_blocks_per_seq, max_seq_len, scale, dtype, stream);
}

pa_status_t pa_decode(void *out, const void *query, const void *key_cache, const void *value_cache,
                      const int32_t *block_tables, const int32_t *seq_lens, int num_seqs,
                      int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                      int num_blocks, int max_blocks_per_seq, int max_seq_len, float scale,
                      pa_dtype_t dtype, int partition_size, void *workspace,
                      size_t workspace_bytes, void *stream) {
    if (pa_select_v2(max_seq_len, num_seqs, num_kv_heads, partition_size)) {
        return pa_decode_v2(out, query, key_cache, value_cache, block_tables, seq_lens, num_seqs,
                            num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                            max_blocks_per_seq, max_seq_len, scale, dtype, partition_size,
                            workspace, workspace_bytes, stream);
    }
    return pa_decode_v1(out, query, key_cache, value_cache, block_tables, seq_lens, num_seqs,
                        num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                        max_blocks_per_seq, max_seq_len, scale, dtype, stream);
}

// ---------------------------------------------------------------------------
// Allocation-free V2.  The workspace of pa_decode_v2_noalloc lives in this
// file-scope device array: each device the library runs on holds its own copy
// until the process ends.  Host code never uses the array's name as an
// address (on the host it is only a stand-in for the symbol): the device
// address comes from hipGetSymbolAddress, resolved once per device with that
// device current, and only that address is passed to kernels.
// ---------------------------------------------------------------------------
}  // extern "C"

namespace {

static __device__ __align__(256) unsigned char scratch[PA_NOALLOC_SCRATCH_BYTES];

std::mutex g_scratch_mutex;
std::atomic<void *> g_scratch_ptr[kMaxDevices];

// Device address of this device's scratch array (nullptr if it cannot be had).
void *device_scratch() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    void *p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (p) return p;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (p) return p;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
        (void)hipGetLastError();  // leave no sticky error for the caller's next call
        return nullptr;
    }
    g_scratch_ptr[dev].store(p, std::memory_order_release);
    return p;
}

}  // namespace

extern "C" {

pa_status_t pa_decode_v2_noalloc(void *out, const void *query, const void *key_cache,
                                 const void *value_cache, const int32_t *block_tables,
                                 const int32_t *seq_lens, int num_seqs, int num_q_heads,
                                 int num_kv_heads, int head_dim, int block_size, int num_blocks,
                                 int max_blocks_per_seq, int max_seq_len, float scale,
                                 pa_dtype_t dtype, int partition_size, void *stream) {
    // Argument checks first, with no workspace yet: every problem error is reported
    // as pa_decode_v2 would report it, before the size check below.
    pa_status_t st = check_problem(query, key_cache, value_cache, block_tables, seq_lens, num_seqs,
                                   1, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                                   max_blocks_per_seq, max_seq_len, scale, dtype);
    if (st != PA_OK) return st;
    if (partition_size == 0)
        partition_size = pa_select_partition_size(num_seqs, num_kv_heads, max_seq_len);
    Layout lay;
    if (partition_size < kBlockTokens || partition_size % kBlockTokens != 0)
        return PA_ERR_UNSUPPORTED;
    if (!layout(num_seqs, num_q_heads, head_dim, max_seq_len, partition_size, &lay))
        return PA_ERR_INVALID_SHAPE;
    if (lay.total > PA_NOALLOC_SCRATCH_BYTES) return PA_ERR_WORKSPACE_TOO_SMALL;
    if (num_seqs == 0) return PA_OK;
    void *ws = device_scratch();
    if (!ws) return PA_ERR_HIP;
    return decode_v2(out, V2Run::kBoth, nullptr, query, key_cache, value_cache, block_tables,
                     seq_lens, num_seqs, 1, num_q_heads, num_kv_heads, head_dim, block_size,
                     num_blocks, max_blocks_per_seq, max_seq_len, scale, dtype, partition_size, ws,
                     PA_NOALLOC_SCRATCH_BYTES, 0, stream);
}

}  // extern "C"
