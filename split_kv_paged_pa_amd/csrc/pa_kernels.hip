// pa_kernels.hip -- gfx950 (CDNA4) kernels for paged decode attention (one query
// token per sequence, or a few: q_len).
//
// Method (project_6 commit pages):
//   - commit 15ef28e (paged_attention_v2_pytorch.py), "[OPT] PagedAttention V2
//     implementation": Phase 1 computes, per (sequence, head, partition), the
//     logits, their softmax statistics and the value-weighted sum, and stores
//     the partition output, exp-sum and max logit; Phase 2 takes the global max
//     over partitions, rescales each partition by exp(m_p - M) * s_p and sums
//     the partition outputs with those weights over their total.  V1 walks the
//     whole sequence in one unit of work.
//   - commit 490ff98 (paged_attn.py), the summary_statistics message: the
//     running state {max, exp-sum, output} of online softmax and its merge
//     with the factor exp(old max - new max); kv heads are independent and the
//     query heads of one group (and the q_len query tokens) are processed
//     together.
//   - commit 15ef28e, "[OPT] Vectorize paged_attention_v2": keys and values are
//     fetched through the per-sequence block id list, 16 tokens per block, and
//     each kv head is broadcast over its query-head group.
//
// Design for gfx950 (what differs from the pages' PyTorch design):
//   - One workgroup of NW wave64s per (partition group, kv head, sequence).  The
//     G query heads of the group -- times the q_len query tokens -- are the N
//     dimension (columns) of 16x16 MFMA tiles, so every key/value block is read
//     from HBM once for all of them; past 16 columns, grid y also counts column
//     chunks of 16.  When partitions are few, one workgroup takes several
//     consecutive partitions and streams across their boundaries.
//   - A wave owns whole 16-token blocks (blocks j = first + w, first + w + NW, ...).
//     The caches use the split layout (keys [D/x][16][x], values [D][16] per
//     block and kv head, x = 16 bytes of values), so every load instruction of
//     a wave reads contiguous memory: key chunk c of lane l is the 16 bytes at
//     1024*c + 16*l of the slab (token l % 16, d group 4c + l / 16), and value
//     tile T of lane (i, grp) is the 4 tokens 4*grp .. 4*grp+3 of row d = 16T + i.
//     Loads run ahead of the math in a ring of register slots with exact waits.
//   - QK^T: MFMA with A = keys (rows = tokens), B = Q^T (cols = heads).  The
//     result tile holds, in lane (g, grp) register i, the logit of token
//     4*grp + i for column g -- exactly the B-operand layout P^T needs for PV,
//     so the softmax weights never leave their lane.
//   - PV as O^T = V^T P^T: the value registers as loaded are the A operand (row
//     d, four consecutive tokens per lane), so no transpose is needed and the
//     block loop touches no LDS.
//   - Masked tokens (past the sequence end, or past a column's causal limit
//     when q_len > 1) get logit -inf; value slots past the sequence end are
//     zeroed before any MFMA touches them, so stale or NaN cache slots cannot
//     leak through 0 * NaN.
//   - Exponentials: exp(x) = 2^(x log2 e) on v_exp_f32.
//   - Waves merge their {max, exp-sum, output} states once per partition,
//     through LDS, in a fixed order, and Phase 2 merges partitions in a fixed
//     order: results are bitwise reproducible run to run.  The single-launch
//     form adds one atomic ticket per (sequence, kv head) to find the workgroup
//     that merges, which then merges in a fixed order too.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <type_traits>

#include "pa_device.h"
#include "pa_launch.h"
#include "pa_timeline.h"

namespace pa {
namespace {

// ---------------------------------------------------------------------------
// Element-type specific MFMA steps.
//   Keys: a lane holds "chunk c" of its token row: E consecutive d values
//   starting at d = (4c + grp) * E (grp = lane / 16), i.e. 16 bytes.
//   Values: a lane (i, grp) holds, for d tile T, the four tokens 4*grp .. 4*grp+3
//   of dimension d = 16T + i (one VU).
// ---------------------------------------------------------------------------
template <typename T> struct Mma;

// bf16 storage (uint16 bit patterns): v_mfma_f32_16x16x16_bf16, 4 values per lane.
template <> struct Mma<uint16_t> {
    static constexpr int E = 8;  // elements per 16-byte key chunk
    typedef u32x2 VU;            // four bf16 tokens of one d

    // S[t][g] += sum over the chunk's d of K[t][d] Q[g][d].
    static __device__ __forceinline__ void qk(f32x4 &s, uint4 k, uint4 q) {
        s = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(lo_half(k), lo_half(q), s, 0, 0, 0);
        s = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(hi_half(k), hi_half(q), s, 0, 0, 0);
    }

    struct Probs { s16x4 p; };
    static __device__ __forceinline__ Probs probs(const float *p) {
        return {pack_bf16(p[0], p[1], p[2], p[3])};
    }

    // acc (lane (g, grp), register r) += sum_t V[16T + 4*grp + r][t] P[g][t]:
    // O^T = V^T P^T, with v already in the A-operand layout (row d, 4 tokens).
    static __device__ __forceinline__ void pv(f32x4 &acc, VU v, const Probs &pr) {
        acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, v), pr.p, acc, 0, 0, 0);
    }

    // Zero the tokens 4*grp + e >= valid of v (e = 0..3).
    static __device__ __forceinline__ VU mask(VU v, int keep) {
        const uint32_t m0 = keep >= 2 ? 0xffffffffu : (keep == 1 ? 0x0000ffffu : 0u);
        const uint32_t m1 = keep >= 4 ? 0xffffffffu : (keep == 3 ? 0x0000ffffu : 0u);
        return VU{v[0] & m0, v[1] & m1};
    }

    static __device__ __forceinline__ float to_float(uint16_t x) {
        return __uint_as_float((uint32_t)x << 16);
    }
    static __device__ __forceinline__ uint16_t from_float(float x) {
        return __builtin_bit_cast(uint16_t, (__bf16)x);
    }
};

// float32 storage: v_mfma_f32_16x16x4_f32, one value per lane per MFMA.
template <> struct Mma<float> {
    static constexpr int E = 4;
    typedef uint4 VU;  // four fp32 tokens of one d

    static __device__ __forceinline__ void qk(f32x4 &s, uint4 k, uint4 q) {
        s = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(k.x), __uint_as_float(q.x), s, 0, 0, 0);
        s = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(k.y), __uint_as_float(q.y), s, 0, 0, 0);
        s = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(k.z), __uint_as_float(q.z), s, 0, 0, 0);
        s = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(k.w), __uint_as_float(q.w), s, 0, 0, 0);
    }

    struct Probs { float p[4]; };
    static __device__ __forceinline__ Probs probs(const float *p) { return {{p[0], p[1], p[2], p[3]}}; }

    // MFMA m reduces over the tokens 4*grp + m: lane (i, grp) gives V[d][4*grp + m]
    // (component m of v), lane (g, grp) gives P[g][4*grp + m] (register m of P^T).
    static __device__ __forceinline__ void pv(f32x4 &acc, VU v, const Probs &pr) {
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(v.x), pr.p[0], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(v.y), pr.p[1], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(v.z), pr.p[2], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(v.w), pr.p[3], acc, 0, 0, 0);
    }

    static __device__ __forceinline__ VU mask(VU v, int keep) {
        return make_uint4(keep > 0 ? v.x : 0u, keep > 1 ? v.y : 0u, keep > 2 ? v.z : 0u,
                          keep > 3 ? v.w : 0u);
    }

    static __device__ __forceinline__ float to_float(float x) { return x; }
    static __device__ __forceinline__ float from_float(float x) { return x; }
};

constexpr int kMergeCap = 2048;  // group partials (heads x groups) one fused merge can weigh


// ---------------------------------------------------------------------------
// Fused-V2 final merge, run by the last workgroup of a (sequence, kv head):
// for each of its G query heads, the n group partials {m_i, s_i, o_i} are merged
// as in Phase 2 -- M = max_i m_i, w_i = exp(m_i - M) s_i, out = sum_i w_i o_i /
// sum_i w_i -- in increasing i, so the result does not depend on which
// workgroup ran last.  G * n <= kMergeCap.
// ---------------------------------------------------------------------------
template <typename T, int D, int NW>
__device__ __forceinline__ void merge_groups(const float *__restrict__ tmp_out,
                                             const float *__restrict__ exp_sums,
                                             const float *__restrict__ max_logits, size_t head0,
                                             int group, int n, int max_parts, T *__restrict__ orow) {
    using M = Mma<T>;
    constexpr int NTH = NW * 64;
    constexpr int kPer = kMergeCap / NTH;  // entries per thread
    __shared__ float sm_w[kMergeCap];
    __shared__ float sm_hm[16];
    __shared__ float sm_hw[16];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int total = group * n;
    // Entry e = g * n + i: max logit and exp-sum of group partial i of head g.
    float es_r[kPer];
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
        const int e = tid + k * NTH;
        es_r[k] = 0.f;
        if (e < total) {
            const int gg = e / n;
            const size_t row = (head0 + gg) * max_parts + (e - gg * n);
            sm_w[e] = max_logits[row];
            es_r[k] = exp_sums[row];
        }
    }
    __syncthreads();
    for (int gg = w; gg < group; gg += NW) {
        float mx = -INFINITY;
        for (int i = lane; i < n; i += 64) mx = fmaxf(mx, sm_w[gg * n + i]);
        mx = wave_max(mx);
        if (lane == 0) sm_hm[gg] = mx;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
        const int e = tid + k * NTH;
        if (e < total) {
            const float m = sm_w[e];
            const float mx = sm_hm[e / n];
            sm_w[e] = m == -INFINITY ? 0.f : exp_e(m - mx) * es_r[k];
        }
    }
    __syncthreads();
    for (int gg = w; gg < group; gg += NW) {
        // Fixed-order sum: lane partials over i = lane, lane + 64, ..., then lanes in order.
        float sum = 0.f;
        for (int i = lane; i < n; i += 64) sum += sm_w[gg * n + i];
        for (int off = 32; off >= 1; off >>= 1) sum += __shfl_xor(sum, off);
        if (lane == 0) sm_hw[gg] = sum;
    }
    __syncthreads();
    // out[g][4c .. 4c+3] = sum_i w_i o_i[4c ..] / W_g, i in increasing order.
    constexpr int C4 = D / 4;
    for (int q = tid; q < group * C4; q += NTH) {
        const int gg = q / C4;
        const int c = q - gg * C4;
        const float *src = tmp_out + (head0 + gg) * (size_t)max_parts * D + 4 * c;
        const float *wt = sm_w + gg * n;
        f32x4 a = {0.f, 0.f, 0.f, 0.f};
        int i = 0;
        for (; i + 8 <= n; i += 8) {
            f32x4 v[8];
#pragma unroll
            for (int r = 0; r < 8; ++r) v[r] = *reinterpret_cast<const f32x4 *>(src + (size_t)(i + r) * D);
#pragma unroll
            for (int r = 0; r < 8; ++r) a += wt[i + r] * v[r];
        }
        for (; i < n; ++i) a += wt[i] * *reinterpret_cast<const f32x4 *>(src + (size_t)i * D);
        const float W = sm_hw[gg];
        const float inv = W > 0.f ? 1.f / W : 0.f;
#pragma unroll
        for (int r = 0; r < 4; ++r) orow[gg * D + 4 * c + r] = M::from_float(a[r] * inv);
    }
}

// ---------------------------------------------------------------------------
// Four schedules of one kernel (MODE):
//   kPartials (V2 Phase 1): workgroup (pg, kv head, sequence) handles the
//     partitions p in [pg * ppw, min((pg + 1) * ppw, ceil(L / P))) of that
//     sequence and kv head, one after the other, and writes each one's partials.
//   kFused (V2 in one launch): the same partitions, each computed exactly as in
//     kPartials, but folded into one group partial {max, exp-sum, output} per
//     head with the Phase-2 rescale; the workgroup writes that, takes a ticket
//     for its (sequence, kv head), and the last one to arrive merges the group
//     partials of all workgroups of that (sequence, kv head) in a fixed order
//     and writes the output.
//   kSinglePass (V1): workgroup (0, kv head, sequence) covers the whole sequence
//     as a single partition and writes the output.
//   kGrouped (V2 Phase 1 when partitions are few): workgroup (x, kv head,
//     sequence) takes the equal span of blocks [x * span, (x + 1) * span) of the
//     row as its one partition, whatever partition boundaries of the caller's
//     size fall inside it, and writes that span's partials to entry x; Phase 2
//     merges the entries as partitions of 16 * span tokens.  An empty span
//     (past the end of a shorter sequence) writes max logit -inf to its entry,
//     so Phase 2 can take every entry of the grid without reading seq_lens.
//     Closing the caller's partitions inside a span (each wave depositing its
//     state at every boundary, all merged at the end) measured 0.6-1.0 us per
//     100K-token step slower, for results that differ only in rounding.
// ---------------------------------------------------------------------------
enum Mode { kSinglePass = 0, kPartials = 1, kFused = 2, kGrouped = 3 };

// Argument order: what the first key/value loads depend on comes first -- the
// block table and seq_lens, the table stride, the workgroup's block stride, the
// caches and what forms their addresses (14 dwords) -- so that with kernel-
// argument preloading (the first 14 dwords arrive in SGPRs at wave launch) the
// first memory round trip is the block ids, not the argument buffer.
template <typename T, int D, int NW, int U, int MODE>
__global__ __launch_bounds__(NW * 64) void attend_kernel(
    const int32_t *__restrict__ block_tables, const int32_t *__restrict__ seq_lens,
    const T *__restrict__ key_cache, const T *__restrict__ value_cache, int max_blocks,
    int wg_blocks, int num_kv_heads, int num_blocks, int group, int qlen,
    const T *__restrict__ query, int num_q_heads, int max_seq_len, float scale,
    int partition_size, int ppw, int max_parts, float *__restrict__ tmp_out,
    float *__restrict__ exp_sums, float *__restrict__ max_logits, uint32_t *__restrict__ tickets,
    T *__restrict__ out) {
    // wg_blocks: blocks per workgroup (grid x): the span (kGrouped), ppw partitions
    // (kPartials, kFused); unused by kSinglePass.
    PA_TL_BEGIN_SLOT();  // diagnostic timeline build only
    constexpr bool kFinal = MODE == kSinglePass;
    // kFused folds each partition into the workgroup's group partial at its close.
    constexpr bool kFold = MODE == kFused;
    constexpr int KP = 1;
    using M = Mma<T>;
    constexpr int E = M::E;
    using VU = typename M::VU;
    constexpr int NC = D / (4 * E);          // key chunks (16 bytes) per lane per block
    constexpr int NT = D / 16;               // d tiles: value units and accumulator tiles
    constexpr int LDS_STRIDE = D + 4;

    // Per (wave, column) states: max, exp-sum, merge factor, output (33 KiB at D = 128).
    __shared__ float sm_m[KP][NW][16];
    __shared__ float sm_l[KP][NW][16];
    __shared__ float sm_f[KP][NW][16];
    __shared__ __attribute__((aligned(16))) float sm_o[KP][NW][16][LDS_STRIDE];  // rows 16-byte aligned
    // kFused: the group partial {max, exp-sum, unnormalised output} per head.
    constexpr int GA = kFold ? 16 : 1;
    __shared__ float sm_gm[GA];
    __shared__ float sm_gw[GA];
    __shared__ float sm_gs[GA];  // rescale of sm_ga for the partition being folded in
    __shared__ __attribute__((aligned(16))) float sm_ga[GA][kFold ? D : 1];
    __shared__ uint32_t sm_ticket;

    const int lane = threadIdx.x & 63;
    // Wave index, made provably uniform so that everything derived from it (the
    // block ids in particular) lives in scalar registers and is read with scalar
    // loads, which do not wait on the vector-memory counter of the K/V loads.
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int l16 = lane & 15;
    const int grp = lane >> 4;
    // blockIdx.y = kv head * column chunks + chunk: the G * qlen (query token, head)
    // columns of a kv head are taken 16 at a time (one chunk unless G * qlen > 16).
    const int nchunk = (group * qlen + 15) / 16;
    const int kvh = blockIdx.y / nchunk;
    const int c0 = (blockIdx.y - kvh * nchunk) * 16;  // first column of this chunk
    const int s = blockIdx.z;
    // Partition (group) of this workgroup.  kPartials rotates it by the grid row
    // (kv head, chunk, sequence): workgroups go to the XCDs in turn by linear
    // id, and when the row length is a multiple of 8 the unrotated index would
    // send partition p of every row to the same XCD -- with many single-partition
    // sequences, one XCD then holds most of the work (measured on MI355X, 64
    // ragged sequences at P = 4096: 1779 us per step against 869 us rotated;
    // P = 1024 and 2048 unchanged within 1%).
    const int pg = MODE == kPartials
                       ? (int)((blockIdx.x + blockIdx.y + (unsigned long long)gridDim.y * blockIdx.z) %
                               gridDim.x)
                       : (int)blockIdx.x;

    // The first block this wave will read does not depend on the sequence length:
    // its table entry is requested together with seq_lens[s] (index clamped into
    // the row), so the two scalar loads share one memory latency.
    const int32_t *bt = block_tables + (size_t)s * max_blocks;
    const int j_first = (kFinal ? 0
                                : pg * wg_blocks) + w;
    const int id_first = max_blocks > 0 ? bt[min(j_first, max_blocks - 1)] : 0;
    const int L = min(max(seq_lens[s], 0), max_seq_len);
    const int nblk = (L + kBlockTokens - 1) / kBlockTokens;
    // Partitions of this workgroup, in blocks of bp each.
    // The workgroup's blocks [b_lo, b_hi) fall in partitions p_begin .. p_end - 1;
    // piece p of them is [max(p * bp, b_lo), min((p + 1) * bp, b_hi)).  kGrouped
    // takes wg_blocks blocks from pg * wg_blocks as one piece (the span is this
    // workgroup's partition); the other modes take ppw whole partitions.
    int bp, p_begin, p_end, b_lo, b_hi;
    if (kFinal) {
        bp = max(nblk, 1);
        p_begin = 0;
        p_end = 1;
        b_lo = 0;
        b_hi = nblk;
    } else if (MODE == kGrouped) {
        bp = wg_blocks;
        b_lo = pg * wg_blocks;
        b_hi = min(b_lo + wg_blocks, nblk);
        if (b_lo >= b_hi) {  // uniform: past the sequence's last block
            // Mark the entry empty (max logit -inf): Phase 2 then takes every
            // entry of the grid without reading seq_lens first.
            const int nc = min(16, group * qlen - c0);
            if ((int)threadIdx.x < nc) {
                const int c = c0 + (int)threadIdx.x;
                const size_t row =
                    ((size_t)s * qlen + c / group) * num_q_heads + (size_t)kvh * group + c % group;
                store_through(max_logits + row * max_parts + pg, -INFINITY);
            }
            return;
        }
        p_begin = pg;
        p_end = pg + 1;
    } else {
        bp = partition_size / kBlockTokens;
        const int parts = (nblk + bp - 1) / bp;
        p_begin = pg * ppw;
        p_end = min(p_begin + ppw, parts);
        b_lo = p_begin * bp;
        b_hi = min(p_end * bp, nblk);
        if (p_begin >= p_end) {  // uniform over the workgroup
            if (MODE == kFused && parts == 0 && blockIdx.x == 0) {
                // No workgroup of this (sequence, kv head) has work: L == 0 gives zeros.
                T *orow = out + ((size_t)s * num_q_heads + (size_t)kvh * group) * D;
                for (int idx = threadIdx.x; idx < group * D; idx += NW * 64)
                    orow[idx] = M::from_float(0.f);
            }
            return;
        }
    }
    if (kFold) {
        for (int idx = threadIdx.x; idx < 16 * D; idx += NW * 64) sm_ga[idx / D][idx % D] = 0.f;
        if (threadIdx.x < 16) {
            sm_gm[threadIdx.x] = -INFINITY;
            sm_gw[threadIdx.x] = 0.f;
        }
    }

    // Columns: column g of the MFMA tiles is global column c = c0 + g, i.e. (query
    // token c / G, head kvh*G + c % G) of this sequence, for c < G * qlen (qlen query
    // tokens per sequence; 1 for plain decode).  Query and output rows are
    // [S][qlen][Hq][D]; the row of column gg is qrow_of(gg).
    const int g = l16;
    const int ncol = min(16, group * qlen - c0);
    auto qrow_of = [&](int gg) {
        const int c = c0 + gg;
        return ((size_t)s * qlen + c / group) * num_q_heads + (size_t)kvh * group + c % group;
    };
    // Q^T operand: lane (g, grp) holds chunk c of column g's query (zero for g >= ncol).
    uint4 qv[NC];
    if (g < ncol) {
        const uint4 *qrow = reinterpret_cast<const uint4 *>(query + qrow_of(g) * D);
#pragma unroll
        for (int c = 0; c < NC; ++c) qv[c] = qrow[c * 4 + grp];
    } else {
#pragma unroll
        for (int c = 0; c < NC; ++c) qv[c] = make_uint4(0, 0, 0, 0);
    }

    float m_run = -INFINITY;  // running max logit of column g
    float l_run = 0.f;        // this lane's share of the running exp-sum
    f32x4 acc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

    const size_t slab = (size_t)kBlockTokens * D;        // elements of one (block, kv head) slab
    // Byte offsets inside a (block, kv head) slab.  Keys, [D/E][16][E]: chunk c of
    // lane l is the 16 bytes at 1024*c + 16*l, so each load instruction reads 1 KiB
    // of contiguous memory.  Values, [D][16]: tile T of lane (i, grp) is the
    // 4 tokens at row d = 16T + i, byte 4*grp*sizeof(T); one instruction reads the
    // contiguous 16 rows of a tile.
    constexpr int kRowBytes = kBlockTokens * (int)sizeof(T);  // one value row (d)
    constexpr int kKStep = 1024;
    constexpr int kVStep = 16 * kRowBytes;
    const int k_lane = 16 * lane;
    const int v_lane = kRowBytes * l16 + 4 * (int)sizeof(T) * grp;
    const char *dummy = reinterpret_cast<const char *>(query + qrow_of(0) * D);
    // Last token column g may see: token j of qlen sits at L - qlen + j (causal
    // over the cache); unused columns take L - 1.
    const int lim = g < ncol ? L - qlen + (c0 + g) / group : L - 1;
    const int lim_min = L - qlen + c0 / group;  // smallest limit over this chunk's columns

    // ---- issue side: wave w takes blocks b_lo + w, b_lo + w + NW, ... of the
    // workgroup's whole range, so the waves' shares differ by at most one block
    // however the partitions cut it (restarting the stride at every piece left up
    // to one block per piece of imbalance); the piece of a block is the partition
    // it falls in.  Loads run U-1 blocks ahead of the math in a ring of register
    // slots, across piece boundaries.  The next block id is read one issue ahead
    // with a scalar load.
    int i_p = p_begin;     // piece of the next block to issue (p_end: done)
    int i_j = b_lo + w;    // next block to issue
    auto settle = [&]() { i_p = i_j < b_hi ? (kFinal ? 0 : i_j / bp) : p_end; };
    settle();
    int id_next = i_p < p_end ? (i_j == j_first ? id_first : bt[i_j]) : 0;

    // Every issue emits the same loads in the same order -- past the end, or for
    // a block id outside [0, num_blocks), they read the (cached) query row and the
    // block is not attended -- so the compiler keeps exactly the younger ring
    // slots outstanding at each wait.
    auto issue = [&](uint4 (&kr)[NC], VU (&vr)[NT], int &part, int &blk) -> bool {
        part = i_p;
        blk = i_j;
        const int phys = id_next;
        const bool ok = i_p < p_end && (unsigned)phys < (unsigned)num_blocks;
        if (i_p < p_end) {
            i_j += NW;
            settle();
            id_next = i_p < p_end ? bt[i_j] : 0;
        }
        // A dummy issue reads the same 16 bytes of the query row in every load.
        // Keys and values are read once per step: non-temporal loads, which keep
        // the stream out of the L2 and last-level cache (measured: the 100K-token
        // step 43.9 -> 40.1 us).
        const size_t base = ok ? ((size_t)phys * num_kv_heads + kvh) * slab : 0;
        const char *kp = ok ? reinterpret_cast<const char *>(key_cache + base) + k_lane : dummy;
        const char *vp = ok ? reinterpret_cast<const char *>(value_cache + base) + v_lane : dummy;
        const int ks = ok ? kKStep : 0;
        const int vs = ok ? kVStep : 0;
#pragma unroll
        for (int c = 0; c < NC; ++c) kr[c] = load_nt(reinterpret_cast<const uint4 *>(kp + c * ks));
#pragma unroll
        for (int t = 0; t < NT; ++t) vr[t] = load_nt(reinterpret_cast<const VU *>(vp + t * vs));
        return ok;
    };

    // One block: logits, running-max update, weights, PV.  kTail: the block
    // holds the end of the sequence, so some of its slots are masked.
    auto attend = [&](auto tail, int j, const uint4 (&kr)[NC], VU (&vr)[NT]) {
        constexpr bool kTail = decltype(tail)::value;
        const int valid = L - j * kBlockTokens;  // tokens of the block in range (>= 1)
        // Two independent MFMA chains (even / odd chunks) halve the dependent latency.
        f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < NC; c += 2) {
            M::qk(s0, kr[c], qv[c]);
            if (c + 1 < NC) M::qk(s1, kr[c + 1], qv[c + 1]);
        }
        const f32x4 sacc = s0 + s1;

        float z[4];
#pragma unroll
        for (int r = 0; r < 4; ++r)
            z[r] = (!kTail || j * kBlockTokens + 4 * grp + r <= lim) ? sacc[r] * scale : -INFINITY;
        const float bm = column_max(fmaxf(fmaxf(z[0], z[1]), fmaxf(z[2], z[3])));
        // Rescale only when some column's max grew: otherwise the factor is
        // exactly 1 and skipping it changes no bit.
        if (__builtin_amdgcn_ballot_w64(bm > m_run) != 0) {
            const float m_new = fmaxf(m_run, bm);
            // A column that has seen nothing yet keeps m = -inf (only in tail blocks with
            // several query tokens); its factor is 0, not exp(-inf + inf).
            const float alpha = m_run == -INFINITY ? 0.f : exp_e(m_run - m_new);
            l_run *= alpha;
            m_run = m_new;
#pragma unroll
            for (int t = 0; t < NT; ++t) acc[t] *= alpha;
        }
        float pr[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) pr[r] = (kTail && z[r] == -INFINITY) ? 0.f : exp_e(z[r] - m_run);
        l_run += (pr[0] + pr[1]) + (pr[2] + pr[3]);

        if (kTail) {
            const int keep = valid - 4 * grp;  // tokens of this lane's four still in range
#pragma unroll
            for (int t = 0; t < NT; ++t) vr[t] = M::mask(vr[t], keep);
        }
        const typename M::Probs pb = M::probs(pr);
#pragma unroll
        for (int t = 0; t < NT; ++t) M::pv(acc[t], vr[t], pb);
    };
    auto step = [&](int j, const uint4 (&kr)[NC], VU (&vr)[NT]) {
        if ((j + 1) * kBlockTokens <= lim_min + 1)  // every token visible to every column
            attend(std::false_type{}, j, kr, vr);
        else
            attend(std::true_type{}, j, kr, vr);
    };

    // One 16-byte write-through store (buffer_store_dwordx4 ... sc1) per thread of
    // o at float d of row row_of(gg): whole cache lines, a quarter of the store
    // instructions of one float per thread, and no dirty L2 lines at the end of
    // the kernel.  A buffer store takes a wave-uniform base, so the lanes' rows
    // are taken one at a time (two per wave at D = 128, four at D = 64); the
    // descriptor spans one row.  Measured on MI355X against one float per thread:
    // the 100K-token step -0.16 to -0.6 us, batches unchanged; plain 16-byte
    // stores cost a batch with 42 MB of partials 4.6% at the kernel's end, and 4-
    // or 8-byte stores in this mapping, which cover part of every line they
    // touch, cost a 64-sequence batch 9%.
    auto store_row4 = [&](auto row_of, int gg, int d, f32x4 o) {
        typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
        for (bool pending = true; pending;) {
            const int g0 = __builtin_amdgcn_readfirstlane(gg);
            if (gg == g0) {
                __builtin_amdgcn_raw_buffer_store_b128(
                    __builtin_bit_cast(u32x4v, o),
                    __builtin_amdgcn_make_buffer_rsrc(row_of(g0), 0, D * (int)sizeof(float),
                                                      kBufferWord3),
                    4 * d, 0, kCachePolicySc1);
                pending = false;
            }
        }
    };

    // End of piece p: merge the waves' states (fixed order) and write them (or,
    // kFold, fold them into the group partial).
    auto finish = [&](int p) {
        const float l_col = column_sum(l_run);
        if (p != p_begin) __syncthreads();  // the previous partition's readers are done
        // acc[t] of lane (g, grp) holds d = 16t + 4*grp + [0, 4) of column g.
        if (grp == 0) {
            sm_m[0][w][g] = m_run;
            sm_l[0][w][g] = l_col;
        }
#pragma unroll
        for (int t = 0; t < NT; ++t)
            *reinterpret_cast<f32x4 *>(&sm_o[0][w][g][16 * t + 4 * grp]) = acc[t];
        m_run = -INFINITY;
        l_run = 0.f;
#pragma unroll
        for (int t = 0; t < NT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
        __syncthreads();
        constexpr int C4 = D / 4;
        if (!kFold) {
            // Merge factors per (wave, column): f = exp(m_w - M) / (sum_w exp(m_w - M)
            // l_w), taken by every thread of the column from the deposited states (the
            // same arithmetic in each, so one barrier per close; sharing them through
            // LDS took a second barrier and round trip).  Each thread merges 4
            // consecutive d of one column; a partition's output goes out with
            // store_row4, then its exp-sum and max logit (no barrier follows them: a
            // barrier's release fence waits until the wave's global stores have
            // completed, a write-through round trip to memory, ~1 us).
            for (int idx = threadIdx.x; idx < ncol * C4; idx += NW * 64) {
                const int gg = idx / C4;
                const int d = (idx - gg * C4) * 4;
                float mw[NW], lw[NW];
#pragma unroll
                for (int ww = 0; ww < NW; ++ww) {
                    mw[ww] = sm_m[0][ww][gg];
                    lw[ww] = sm_l[0][ww][gg];
                }
                float mx = -INFINITY;
#pragma unroll
                for (int ww = 0; ww < NW; ++ww) mx = fmaxf(mx, mw[ww]);
                float f[NW];
                float total = 0.f;
#pragma unroll
                for (int ww = 0; ww < NW; ++ww) {
                    f[ww] = (mx == -INFINITY) ? 0.f : exp_e(mw[ww] - mx);
                    total += f[ww] * lw[ww];
                }
                const float inv = total > 0.f ? 1.f / total : 0.f;
                f32x4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ww = 0; ww < NW; ++ww)
                    o += (f[ww] * inv) * *reinterpret_cast<const f32x4 *>(&sm_o[0][ww][gg][d]);
                if (kFinal) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) out[qrow_of(gg) * D + d + r] = M::from_float(o[r]);
                } else {
                    store_row4([&](int g0) { return tmp_out + (qrow_of(g0) * max_parts + p) * D; },
                               gg, d, o);
                    if (d == 0) {
                        const size_t row = qrow_of(gg) * max_parts + p;
                        store_through(exp_sums + row, total);
                        store_through(max_logits + row, mx);
                    }
                }
            }
            return;
        }
        // kFold: thread g < 16 folds column g's merge into the group partial.
        if (threadIdx.x < 16) {
            const int gg = threadIdx.x;
            float mx = -INFINITY;
#pragma unroll
            for (int ww = 0; ww < NW; ++ww) mx = fmaxf(mx, sm_m[0][ww][gg]);
            float f[NW];
            float total = 0.f;
#pragma unroll
            for (int ww = 0; ww < NW; ++ww) {
                f[ww] = (mx == -INFINITY) ? 0.f : exp_e(sm_m[0][ww][gg] - mx);
                total += f[ww] * sm_l[0][ww][gg];
            }
            {
                // Fold (mx, total, sum_w f_w o_w) into the group partial with the
                // Phase-2 rescale: weights exp(m - M') against the new group max M'.
                const float gm = sm_gm[gg];
                const float gm_new = fmaxf(gm, mx);
                const float a = gm == -INFINITY ? 0.f : exp_e(gm - gm_new);
                const float b = mx == -INFINITY ? 0.f : exp_e(mx - gm_new);
                sm_gm[gg] = gm_new;
                sm_gw[gg] = sm_gw[gg] * a + total * b;
                sm_gs[gg] = a;
#pragma unroll
                for (int ww = 0; ww < NW; ++ww) sm_f[0][ww][gg] = f[ww] * b;
            }
        }
        __syncthreads();
        for (int idx = threadIdx.x; idx < ncol * C4; idx += NW * 64) {
            const int gg = idx / C4;
            const int d = (idx - gg * C4) * 4;
            f32x4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ww = 0; ww < NW; ++ww)
                o += sm_f[0][ww][gg] * *reinterpret_cast<const f32x4 *>(&sm_o[0][ww][gg][d]);
            f32x4 &ga = *reinterpret_cast<f32x4 *>(&sm_ga[gg][d]);
            ga = ga * sm_gs[gg] + o;  // same thread owns (gg, d .. d+3) every time
        }
    };

    // ---- attend side: consume the ring in order; close each partition when the
    // next block belongs to a later one.  Every wave closes every partition once,
    // so the barriers inside finish() line up across the waves.
    int a_p = p_begin;
    uint4 kb[U][NC];
    VU vb[U][NT];
    int sp[U], sj[U];
    bool live[U];
#pragma unroll
    for (int u = 0; u < U - 1; ++u) live[u] = issue(kb[u], vb[u], sp[u], sj[u]);
    bool done = false;
    for (;;) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            constexpr int kAhead = U - 1;
            const int slot = (u + kAhead) % U;
            live[slot] = issue(kb[slot], vb[slot], sp[slot], sj[slot]);  // unconditional
            if (!done) {
                if (sp[u] >= p_end) {
                    done = true;
                } else {
                    while (a_p < sp[u]) finish(a_p++);
                    if (live[u]) step(sj[u], kb[u], vb[u]);
                }
            }
        }
        if (done) break;
    }
    PA_TL_MARK(pa_tl_mid);
    while (a_p < p_end) finish(a_p++);
    PA_TL_RECORD(1, pa_tl_mid);

    if (MODE != kFused) return;

    // ---- kFused epilogue.  Group partial g of this workgroup goes to entry gi =
    // blockIdx.x of the workspace partials (normalised like a partition partial).
    const size_t head0 = (size_t)s * num_q_heads + (size_t)kvh * group;
    const int gi = blockIdx.x;
    __syncthreads();
    // Publication: the group partial is stored with device-scope atomic stores
    // (written through to the device's point of coherence), each wave waits until
    // its stores have completed, the workgroup barrier orders them before thread
    // 0's ticket, and the ticket is an acquire-release read-modify-write at device
    // scope: the last workgroup's acquire then synchronises with every earlier
    // workgroup's release, so the merge reads complete group partials under the
    // memory model, not only on this hardware's store ordering.
    if (threadIdx.x < group) {
        const size_t row = (head0 + threadIdx.x) * max_parts + gi;
        __hip_atomic_store(exp_sums + row, sm_gw[threadIdx.x], __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(max_logits + row, sm_gm[threadIdx.x], __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    }
    for (int idx = threadIdx.x; idx < group * D; idx += NW * 64) {
        const int gg = idx / D;
        const int d = idx - gg * D;
        const float W = sm_gw[gg];
        __hip_atomic_store(tmp_out + ((head0 + gg) * max_parts + gi) * D + d,
                           W > 0.f ? sm_ga[gg][d] / W : 0.f, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    }
    __builtin_amdgcn_s_waitcnt(0);  // this wave's stores have completed
    __syncthreads();
    uint32_t *ticket = tickets + (size_t)s * num_kv_heads + kvh;
    if (threadIdx.x == 0)
        sm_ticket = __hip_atomic_fetch_add(ticket, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    const int parts = (nblk + bp - 1) / bp;
    const int n = (parts + ppw - 1) / ppw;  // workgroups of this (sequence, kv head) with work
    if ((int)sm_ticket != n - 1) return;    // uniform: not the last to arrive
    // Acquire: drop this device's cached copies of lines other workgroups wrote.
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    merge_groups<T, D, NW>(tmp_out, exp_sums, max_logits, head0, group, n, max_parts,
                           out + head0 * D);
    if (threadIdx.x == 0)  // leave the counter zero for the next call
        __hip_atomic_store(ticket, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------------------
// Phase 2: one workgroup of NW waves per (query head, sequence).  Wave w takes
// partitions p = w, w + NW, ..., R at a time: it loads their max logits, exp-sums
// and partial outputs together (lane l holds d = l*DPL .. l*DPL + DPL - 1), and
// folds them into a wave-local {max, weight sum, weighted output} with the
// same rescale as Phase 1.  The waves then merge through LDS in a fixed order,
// so the result is reproducible bit for bit.  For up to NW * R partitions this
// is a single round of global loads.
//
// The R loads of a round are straight-line code into distinct registers: an
// index past the last partition is clamped to it (a row the wave has just
// requested, so no extra memory traffic) and its values are masked after the
// loads, so no branch separates the loads and all R are in flight together.
// (With a branch per partition the compiler waited for each load before issuing
// the next: one memory round trip per partition.)
// ---------------------------------------------------------------------------
// Entries of sequence s that Phase 2 merges.  marked >= 0: Phase 1 wrote every
// entry below marked -- an empty one with max logit -inf, which the merge skips --
// so the count needs no seq_lens load (one memory round trip less before the
// partials can be requested); else ceil(L_s / entry_tokens).
__device__ __forceinline__ int row_entries(const int32_t *__restrict__ seq_lens, int s,
                                           int max_seq_len, int entry_tokens, int marked) {
    if (marked >= 0) return marked;
    const int L = min(max(seq_lens[s], 0), max_seq_len);
    return L > 0 ? (int)(((long long)L + entry_tokens - 1) / entry_tokens) : 0;
}

template <int DPL> struct RowPiece;
template <> struct RowPiece<1> { typedef float type; };
template <> struct RowPiece<2> { typedef float type __attribute__((ext_vector_type(2))); };

template <typename T, int D, int NW>
__global__ __launch_bounds__(NW * 64) void reduce_kernel(
    const float *__restrict__ tmp_out, const float *__restrict__ exp_sums,
    const float *__restrict__ max_logits, const int32_t *__restrict__ seq_lens, int num_q_heads,
    int max_seq_len, int partition_size, int max_parts, int marked, T *__restrict__ out) {
    using M = Mma<T>;
    constexpr int NT = NW * 64;
    constexpr int DPL = D / 64;
    typedef typename RowPiece<DPL>::type Piece;
    constexpr int R = 8;  // partitions in flight per wave
    __shared__ float sm_m[NW];
    __shared__ float sm_w[NW];
    __shared__ float sm_acc[NW][D];

    const int h = blockIdx.x;
    const int s = blockIdx.y;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const size_t head = (size_t)s * num_q_heads + h;
    T *orow = out + head * D;

    const int parts = row_entries(seq_lens, s, max_seq_len, partition_size, marked);
    const float *ml = max_logits + head * max_parts;
    const float *es = exp_sums + head * max_parts;
    const Piece *po = reinterpret_cast<const Piece *>(tmp_out + head * max_parts * D) + lane;

    float m_w = -INFINITY;  // wave-local running max
    float wsum = 0.f;       // wave-local sum of exp(m_p - m_w) * s_p
    float acc[DPL];
#pragma unroll
    for (int k = 0; k < DPL; ++k) acc[k] = 0.f;
    for (int p0 = w; p0 < parts; p0 += R * NW) {
        float pm[R], ps[R];
        Piece pv[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int p = min(p0 + r * NW, parts - 1);
            pm[r] = ml[p];
            ps[r] = es[p];
            // Partial outputs are read once: non-temporal loads.
            pv[r] = __builtin_nontemporal_load(po + (size_t)p * (D / DPL));
        }
        // Keep every load of the round ahead of the fold (the compiler would
        // otherwise sink loads into the branches that use them).
#pragma unroll
        for (int r = 0; r < R; ++r) asm volatile("" ::"s"(pm[r]), "s"(ps[r]), "v"(pv[r]));
#pragma unroll
        for (int r = 0; r < R; ++r) {
            if (p0 + r * NW >= parts) pm[r] = -INFINITY;  // a clamped repeat
        }
        float cm = pm[0];
#pragma unroll
        for (int r = 1; r < R; ++r) cm = fmaxf(cm, pm[r]);
        if (cm > m_w) {  // wave-uniform
            const float alpha = m_w == -INFINITY ? 0.f : exp_e(m_w - cm);
            wsum *= alpha;
#pragma unroll
            for (int k = 0; k < DPL; ++k) acc[k] *= alpha;
            m_w = cm;
        }
        if (m_w == -INFINITY) continue;  // nothing valid yet (only without valid block ids)
#pragma unroll
        for (int r = 0; r < R; ++r) {
            if (pm[r] != -INFINITY) {
                const float wt = exp_e(pm[r] - m_w) * ps[r];
                wsum += wt;
                const float *v = reinterpret_cast<const float *>(&pv[r]);
#pragma unroll
                for (int k = 0; k < DPL; ++k) acc[k] += wt * v[k];
            }
        }
    }
    if (lane == 0) {
        sm_m[w] = m_w;
        sm_w[w] = wsum;
    }
#pragma unroll
    for (int k = 0; k < DPL; ++k) sm_acc[w][lane * DPL + k] = acc[k];
    __syncthreads();
    float mx = -INFINITY;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) mx = fmaxf(mx, sm_m[ww]);
    float f[NW];
    float total = 0.f;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) {
        f[ww] = mx == -INFINITY ? 0.f : exp_e(sm_m[ww] - mx);
        total += f[ww] * sm_w[ww];
    }
    // total == 0 only for L == 0 or when no block id of the sequence was valid.
    const float inv = total > 0.f ? 1.f / total : 0.f;
    for (int d = tid; d < D; d += NT) {
        float o = 0.f;
#pragma unroll
        for (int ww = 0; ww < NW; ++ww) o += f[ww] * sm_acc[ww][d];
        orow[d] = M::from_float(o * inv);
    }
}

// ---------------------------------------------------------------------------
// Phase 2 split over the output: workgroup (h * D/32 + x, s) of four waves
// computes out[s][h][32x .. 32x+31] (rows and slices share grid x, whose limit
// is 2^31 - 1: the q_len entry points give Phase 2 q_len * Hq rows).  Lane
// (j, c) of wave w -- j = lane / 8, c = lane % 8 -- takes d = 32x + 4c .. 4c+3
// of partitions p = 8w + j + 32k, K per round (32 K partitions per round: K = 4,
// or 8 for more than 128 partitions).
// Every wave first takes the global max M = max_p m_p over all the row's
// partitions (so no lane ever rescales), then each lane sums
// w_p = exp(m_p - M) s_p and w_p o_p[d .. d+3] over its partitions; the sums
// are folded over j with a fixed butterfly, then over the four waves in order
// through LDS, and out = sum / W.  Spreading a row over D/32 workgroups on
// different CUs keeps each CU's load queue short: with one 16-wave workgroup
// per row, the row's partials all pass one CU, and its fourth wave per SIMD
// received them 0.75 us after its first.
// ---------------------------------------------------------------------------
constexpr int kSplitCols = 32;  // output floats per workgroup

template <typename T, int D, int K>
__global__ __launch_bounds__(256) void reduce_split_kernel(
    const float *__restrict__ tmp_out, const float *__restrict__ exp_sums,
    const float *__restrict__ max_logits, const int32_t *__restrict__ seq_lens, int num_q_heads,
    int max_seq_len, int partition_size, int max_parts, int marked, T *__restrict__ out) {
    PA_TL_BEGIN();  // diagnostic timeline build only
    __shared__ __attribute__((aligned(16))) f32x4 sm_acc[4][8];
    __shared__ float sm_w[4];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int j = lane >> 3;
    const int c = lane & 7;
    constexpr int kSlices = D / kSplitCols;
    const int h = blockIdx.x / kSlices;
    const int x = blockIdx.x - h * kSlices;
    const int s = blockIdx.y;
    const size_t head = (size_t)s * num_q_heads + h;
    const int d0 = x * kSplitCols + 4 * c;

    const int parts = row_entries(seq_lens, s, max_seq_len, partition_size, marked);
    const float *ml = max_logits + head * max_parts;
    const float *es = exp_sums + head * max_parts;
    const float *po = tmp_out + head * max_parts * D + d0;

    // The first round's partials are requested together with the max logits of
    // the global max: one memory round trip for up to 128 partitions.
    float pm[K], ps[K];
    f32x4 pv[K];
    auto load_round = [&](int b) {
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const int p = min(b + 8 * w + j + 32 * k, parts - 1);  // clamped repeats are masked
            pm[k] = ml[p];
            ps[k] = es[p];
            pv[k] = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(po + (size_t)p * D));
        }
    };
    if (parts > 0) load_round(0);
    // Global max over the row's partitions, four loads per lane per round.
    float mx = -INFINITY;
    for (int p0 = 0; p0 < parts; p0 += 4 * 64) {
        float m4[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) m4[i] = ml[min(p0 + lane + 64 * i, parts - 1)];
#pragma unroll
        for (int i = 0; i < 4; ++i) mx = fmaxf(mx, m4[i]);  // clamped repeats change no max
    }
    const float mg = wave_max(mx);

    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    float wsum = 0.f;
    for (int b = 0; b < parts; b += 32 * K) {
        if (b > 0) load_round(b);
        // Keep the round's loads ahead of the fold (no load sunk into its branch).
#pragma unroll
        for (int k = 0; k < K; ++k) asm volatile("" ::"v"(pm[k]), "v"(ps[k]), "v"(pv[k]));
        const int p0 = b + 8 * w + j;
#pragma unroll
        for (int k = 0; k < K; ++k) {
            if (p0 + 32 * k < parts && pm[k] != -INFINITY) {
                const float wt = exp_e(pm[k] - mg) * ps[k];
                wsum += wt;
                acc += wt * pv[k];
            }
        }
    }
    PA_TL_MARK(pa_tl_mid);
    // Fold the eight partition slots of each d chunk: lanes c, c + 8, ..., c + 56.
#pragma unroll
    for (int off = 8; off < 64; off <<= 1) {
        wsum += __shfl_xor(wsum, off);
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[r] += __shfl_xor(acc[r], off);
    }
    if (j == 0) sm_acc[w][c] = acc;
    if (lane == 0) sm_w[w] = wsum;
    __syncthreads();
    if (w == 0 && lane < 8) {
        const f32x4 a = ((sm_acc[0][lane] + sm_acc[1][lane]) + sm_acc[2][lane]) + sm_acc[3][lane];
        const float W = ((sm_w[0] + sm_w[1]) + sm_w[2]) + sm_w[3];
        // W == 0 only for L == 0 or when no block id of the sequence was valid.
        const float inv = W > 0.f ? 1.f / W : 0.f;
        store_out4(out + head * D + x * kSplitCols, kSplitCols, lane, a[0] * inv, a[1] * inv,
                   a[2] * inv, a[3] * inv);
    }
    PA_TL_RECORD_LATE(2, pa_tl_mid);
}

// ---------------------------------------------------------------------------
// Phase 2 for many rows with few partitions (q_len * Hq rows of a prefill-like
// batch): one wave per (row, sequence), four rows per workgroup.  The wave takes
// the row's partitions R at a time in increasing order -- max logits and
// exp-sums through scalar loads, lane l holding d = l*DPL .. l*DPL + DPL - 1 of
// each partial output -- and folds them with the Phase-2 rescale: M = max m_p,
// w_p = exp(m_p - M) s_p, out = sum_p w_p o_p / sum_p w_p.
// ---------------------------------------------------------------------------
constexpr int kRowsPerGroup = 4;

template <typename T, int D, int R>
__global__ __launch_bounds__(kRowsPerGroup * 64) void reduce_rows_kernel(
    const float *__restrict__ tmp_out, const float *__restrict__ exp_sums,
    const float *__restrict__ max_logits, const int32_t *__restrict__ seq_lens, int num_rows,
    int max_seq_len, int partition_size, int max_parts, int marked, T *__restrict__ out) {
    using M = Mma<T>;
    constexpr int DPL = D / 64;
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int h = blockIdx.x * kRowsPerGroup + w;
    if (h >= num_rows) return;  // no barrier in this kernel
    const int s = blockIdx.y;
    const size_t row = (size_t)s * num_rows + h;
    const int parts = row_entries(seq_lens, s, max_seq_len, partition_size, marked);
    const float *ml = max_logits + row * max_parts;
    const float *es = exp_sums + row * max_parts;
    typedef typename RowPiece<DPL>::type Piece;
    const Piece *po = reinterpret_cast<const Piece *>(tmp_out + row * max_parts * D) + lane;

    float m_w = -INFINITY;  // running max
    float wsum = 0.f;       // sum of exp(m_p - m_w) * s_p
    float acc[DPL];
#pragma unroll
    for (int k = 0; k < DPL; ++k) acc[k] = 0.f;
    for (int p0 = 0; p0 < parts; p0 += R) {
        float pm[R], ps[R];
        Piece pv[R];
        // As in reduce_kernel: straight-line loads, an index past the last
        // partition clamped to it, its values masked after the loads.
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int p = min(p0 + r, parts - 1);
            pm[r] = ml[p];
            ps[r] = es[p];
            // Partial outputs are read once: non-temporal loads.
            pv[r] = __builtin_nontemporal_load(po + (size_t)p * (D / DPL));
        }
#pragma unroll
        for (int r = 0; r < R; ++r) asm volatile("" ::"s"(pm[r]), "s"(ps[r]), "v"(pv[r]));
#pragma unroll
        for (int r = 0; r < R; ++r) {
            if (p0 + r >= parts) pm[r] = -INFINITY;  // a clamped repeat
        }
        float cm = pm[0];
#pragma unroll
        for (int r = 1; r < R; ++r) cm = fmaxf(cm, pm[r]);
        if (cm > m_w) {  // wave-uniform
            const float alpha = m_w == -INFINITY ? 0.f : exp_e(m_w - cm);
            wsum *= alpha;
#pragma unroll
            for (int k = 0; k < DPL; ++k) acc[k] *= alpha;
            m_w = cm;
        }
        if (m_w == -INFINITY) continue;  // nothing valid yet
#pragma unroll
        for (int r = 0; r < R; ++r) {
            if (pm[r] != -INFINITY) {
                const float wt = exp_e(pm[r] - m_w) * ps[r];
                wsum += wt;
                const float *v = reinterpret_cast<const float *>(&pv[r]);
#pragma unroll
                for (int k = 0; k < DPL; ++k) acc[k] += wt * v[k];
            }
        }
    }
    const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
    T *orow = out + row * D + lane * DPL;
#pragma unroll
    for (int k = 0; k < DPL; ++k) orow[k] = M::from_float(acc[k] * inv);
}

// Phase 2 uses one wave per row when a row has few partitions (up to 16: one or
// two rounds of loads), or when there are so many rows that one wave each still
// fills the device and the partitions take a few rounds (up to 64); otherwise,
// for fewer than kSplitMaxRows rows, D/32 four-wave workgroups per row
// (reduce_split_kernel), and for more, a workgroup of 16 waves per row whose
// waves load the partitions in parallel.
constexpr int kRowReduceMaxParts = 16;
// Below this many rows Phase 2 splits each row over D/32 workgroups (measured on
// MI355X: the 100K-token step -0.4 to -1.0 us, 320-512 rows unchanged; at 4096
// rows with 128 partitions the per-row workgroup is 0.9% faster).
constexpr long long kSplitMaxRows = 2048;
constexpr long long kRowReduceManyRows = 8192;
constexpr int kRowReduceManyRowsMaxParts = 64;

__global__ void zero_words_kernel(uint32_t *__restrict__ p, int n) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0u;
}

constexpr int kWaves = 4;
constexpr int kReduceWaves = 16;

// Ring slots per wave: the block being attended and the next one in flight.
// (Three slots -- two blocks ahead -- measured 0.5-1.4% slower on MI355X: at
// 194 VGPRs against 162 they leave two waves per SIMD instead of three, and a
// CU streaming one workgroup gains nothing from the deeper ring.)
template <typename T, int D> constexpr int prefetch_depth() { return 2; }

template <typename T, int D, int MODE>
hipError_t launch_attend(const Problem &pb, const Partials *parts, void *out, hipStream_t stream) {
    constexpr bool kFinal = MODE == kSinglePass;
    const int group = pb.num_q_heads / pb.num_kv_heads;
    const int ppw = kFinal ? 1 : parts->per_group;
    const int nchunk = (group * pb.qlen + 15) / 16;  // 16 (query token, head) columns per workgroup
    const int gx = kFinal ? 1 : MODE == kGrouped ? parts->span_count
                                                : (parts->max_parts + ppw - 1) / ppw;
    dim3 grid(gx, pb.num_kv_heads * nchunk, pb.num_seqs);
    const int wg_blocks = kFinal ? 0
                          : MODE == kGrouped ? parts->span_blocks
                                             : ppw * (parts->partition_size / kBlockTokens);
    attend_kernel<T, D, kWaves, prefetch_depth<T, D>(), MODE><<<grid, kWaves * 64, 0, stream>>>(
        pb.block_tables, pb.seq_lens, static_cast<const T *>(pb.key_cache),
        static_cast<const T *>(pb.value_cache), pb.max_blocks, wg_blocks, pb.num_kv_heads,
        pb.num_blocks, group, pb.qlen, static_cast<const T *>(pb.query), pb.num_q_heads,
        pb.max_seq_len, pb.scale, kFinal ? kBlockTokens : parts->partition_size, ppw,
        kFinal ? 0 : parts->max_parts, kFinal ? nullptr : parts->tmp_out,
        kFinal ? nullptr : parts->exp_sums, kFinal ? nullptr : parts->max_logits,
        MODE == kFused ? parts->tickets : nullptr, static_cast<T *>(out));
    return hipGetLastError();
}

template <int MODE>
hipError_t dispatch_attend(const Problem &pb, const Partials *parts, void *out, hipStream_t stream) {
    if (pb.dtype == Dtype::BF16) {
        return pb.head_dim == 64 ? launch_attend<uint16_t, 64, MODE>(pb, parts, out, stream)
                                 : launch_attend<uint16_t, 128, MODE>(pb, parts, out, stream);
    }
    return pb.head_dim == 64 ? launch_attend<float, 64, MODE>(pb, parts, out, stream)
                             : launch_attend<float, 128, MODE>(pb, parts, out, stream);
}

template <typename T, int D>
hipError_t launch_reduce_t(const int32_t *seq_lens, int num_seqs, int num_q_heads, int max_seq_len,
                           const Partials &in, void *out, hipStream_t stream) {
    const long long rows = (long long)num_seqs * num_q_heads;
    // Entries of a row stand for entry_tokens tokens each: the kernels count
    // ceil(L / entry_tokens) of them (they take entry_tokens as their partition size).
    Partials parts = in;
    parts.partition_size = in.entry_tokens;
    const int entries = max_seq_len > 0
                            ? (int)(((long long)max_seq_len + in.entry_tokens - 1) / in.entry_tokens)
                            : 0;  // most entries a row holds
    if (entries <= kRowReduceMaxParts ||
        (rows >= kRowReduceManyRows && entries <= kRowReduceManyRowsMaxParts)) {
        dim3 grid((num_q_heads + kRowsPerGroup - 1) / kRowsPerGroup, num_seqs);
        reduce_rows_kernel<T, D, 8><<<grid, kRowsPerGroup * 64, 0, stream>>>(
            parts.tmp_out, parts.exp_sums, parts.max_logits, seq_lens, num_q_heads, max_seq_len,
            parts.partition_size, parts.max_parts, parts.marked_entries, static_cast<T *>(out));
        return hipGetLastError();
    }
    constexpr int kSlices = D / kSplitCols;
    if (rows < kSplitMaxRows && (long long)num_q_heads * kSlices <= 0x7fffffffLL) {
        // D/32 four-wave workgroups per row, on different CUs.
        dim3 grid((unsigned)num_q_heads * kSlices, num_seqs);
        if (entries <= 128)
            reduce_split_kernel<T, D, 4><<<grid, 256, 0, stream>>>(
                parts.tmp_out, parts.exp_sums, parts.max_logits, seq_lens, num_q_heads,
                max_seq_len, parts.partition_size, parts.max_parts, parts.marked_entries,
                static_cast<T *>(out));
        else  // one round of loads for up to 256 partitions
            reduce_split_kernel<T, D, 8><<<grid, 256, 0, stream>>>(
                parts.tmp_out, parts.exp_sums, parts.max_logits, seq_lens, num_q_heads,
                max_seq_len, parts.partition_size, parts.max_parts, parts.marked_entries,
                static_cast<T *>(out));
    } else {  // many rows: one 16-wave workgroup per row already spreads over the CUs
        dim3 grid(num_q_heads, num_seqs);
        reduce_kernel<T, D, kReduceWaves><<<grid, kReduceWaves * 64, 0, stream>>>(
            parts.tmp_out, parts.exp_sums, parts.max_logits, seq_lens, num_q_heads, max_seq_len,
            parts.partition_size, parts.max_parts, parts.marked_entries, static_cast<T *>(out));
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_single_pass(const Problem &pb, void *out, hipStream_t stream) {
    return dispatch_attend<kSinglePass>(pb, nullptr, out, stream);
}

hipError_t launch_partitions(const Problem &pb, const Partials &parts, hipStream_t stream) {
    return dispatch_attend<kPartials>(pb, &parts, nullptr, stream);
}

hipError_t launch_grouped(const Problem &pb, const Partials &parts, hipStream_t stream) {
    // Entry x of a row is written by span x: the spans must fit the workspace
    // rows and cover the longest sequence.
    const long long nblk = ((long long)pb.max_seq_len + kBlockTokens - 1) / kBlockTokens;
    if (parts.span_blocks < 1 || parts.span_count < 1 || parts.span_count > parts.max_parts ||
        (long long)parts.span_blocks * parts.span_count < nblk)
        return hipErrorInvalidValue;
    return dispatch_attend<kGrouped>(pb, &parts, nullptr, stream);
}

hipError_t launch_fused(const Problem &pb, const Partials &parts, void *out, hipStream_t stream) {
    return dispatch_attend<kFused>(pb, &parts, out, stream);
}

int fused_merge_capacity() { return kMergeCap; }

hipError_t launch_zero_words(uint32_t *p, int n, hipStream_t stream) {
    zero_words_kernel<<<(n + 255) / 256, 256, 0, stream>>>(p, n);
    return hipGetLastError();
}

hipError_t launch_reduce(const int32_t *seq_lens, int num_seqs, int num_q_heads, int head_dim,
                         int max_seq_len, Dtype dtype, const Partials &parts, void *out,
                         hipStream_t stream) {
    if (dtype == Dtype::BF16) {
        return head_dim == 64
                   ? launch_reduce_t<uint16_t, 64>(seq_lens, num_seqs, num_q_heads, max_seq_len, parts, out, stream)
                   : launch_reduce_t<uint16_t, 128>(seq_lens, num_seqs, num_q_heads, max_seq_len, parts, out, stream);
    }
    return head_dim == 64
               ? launch_reduce_t<float, 64>(seq_lens, num_seqs, num_q_heads, max_seq_len, parts, out, stream)
               : launch_reduce_t<float, 128>(seq_lens, num_seqs, num_q_heads, max_seq_len, parts, out, stream);
}

}  // namespace pa

#ifdef PA_TIMELINE
// Diagnostic timeline build: copies the records written so far (at most
// max_records of 4 x uint64) to host memory dst, then clears them and the
// counter.  Returns the number of records the counter reached (holes left by
// workgroups that had no work are all-zero), or a negative value if a HIP call
// failed.  Synchronises the device.
extern "C" int pa_timeline_fetch(void *dst, int max_records) {
    void *buf = nullptr, *cnt = nullptr;
    if (hipGetSymbolAddress(&buf, HIP_SYMBOL(pa::g_timeline)) != hipSuccess ||
        hipGetSymbolAddress(&cnt, HIP_SYMBOL(pa::g_timeline_count)) != hipSuccess)
        return -1;
    if (hipDeviceSynchronize() != hipSuccess) return -2;
    unsigned n = 0;
    if (hipMemcpy(&n, cnt, sizeof(n), hipMemcpyDeviceToHost) != hipSuccess) return -3;
    unsigned m = n < pa::kTimelineRecords ? n : pa::kTimelineRecords;
    if (max_records >= 0 && m > (unsigned)max_records) m = (unsigned)max_records;
    if (dst && m && hipMemcpy(dst, buf, (size_t)m * 32, hipMemcpyDeviceToHost) != hipSuccess)
        return -4;
    if (hipMemset(buf, 0, (size_t)pa::kTimelineRecords * 32) != hipSuccess ||
        hipMemset(cnt, 0, sizeof(n)) != hipSuccess || hipDeviceSynchronize() != hipSuccess)
        return -5;
    return (int)n;
}
#endif
