// pa_prefill.hip -- gfx950 (CDNA4) kernel for many query columns per kv head:
// q_len query tokens per sequence against the paged cache (prefill-like), bf16.
//
// Method (project_6 commit pages): the same attention as the decode kernels --
// per (sequence, query head, query token) the softmax over the visible cache
// tokens of scale * q.k, applied to the values; kv heads are independent and
// the G query heads of a group, times the q_len query tokens, share one key /
// value stream (commit 490ff98, paged_attn.py, the [kv_h, gqa, q_len, tile]
// batching); the running {max, exp-sum, output} state of online softmax and its
// rescale by exp(old max - new max) (same message).  Split-KV (commit 15ef28e,
// "[OPT] PagedAttention V2 implementation"): each partition of P cache tokens
// writes {normalised output, exp-sum, max logit} and the reduce kernel merges
// the partitions.  Query j of q_len sees cache tokens 0 .. L - q_len + j.
//
// Design for gfx950:
//   - The decode kernel gives a wave 16 (query token, head) columns and splits
//     the blocks of a partition over the waves; with many columns that makes
//     every wave fetch a whole K/V block for only 16 columns of MFMA work, and
//     the per-CU vector cache bandwidth, not the matrix cores, sets the speed.
//     Here a wave owns NCT tiles of 16 columns (Q^T held in registers) and
//     computes every block of its partition for them: each K/V operand it
//     reads feeds NCT tiles.  The 4 waves of a workgroup take consecutive
//     column groups of the same kv head and partition and share one K/V
//     stream: each step of 32 tokens is fetched once by the whole workgroup
//     (16 bytes x 4 per thread at D = 128), two steps ahead, straight into a
//     3-stage LDS ring, from which every wave reads its operands.  Key
//     positions are permuted at 16-byte granularity so that every operand read
//     is free of LDS bank conflicts (the rule is stated at the loads).
//   - MFMA v_mfma_f32_16x16x32_bf16 over steps of 32 tokens (two blocks).
//     QK^T: A = keys (16 token rows x 32 d), B = Q^T (32 d x 16 columns).  The
//     two 16-token tiles of a step take the tokens in an interleaved order --
//     tile T row r is token 16*(r/8) + 8*((r/4)%2) + 4T + r%4 of the step -- so
//     that lane (n, q) ends up holding the logits of tokens 8q .. 8q+7 of column
//     n: exactly the B operand P^T of the PV MFMA (k slot 8q+e = token 8q+e).
//   - PV as O^T = V^T P^T: with values stored [D][16] per block, the A operand
//     of lane (n, q) -- row d = 16t + n, tokens 8q .. 8q+7 -- is one contiguous
//     16-byte read; keys, stored [D/8][16][8], are 16-byte reads as well.
//   - Online softmax in base 2 with a lazy reference: the weights are
//     2^(z log2 e - m) with m the column's reference max, which moves only when
//     a logit exceeds it by more than 2^8 (then the output and exp-sum are
//     rescaled); weights stay below 256, the ratio output / exp-sum is what is
//     kept, and the true max is tracked on the side for the partials.  The
//     exp-sums come out of the PV step too: one more MFMA per tile with an
//     all-ones A operand sums each column's bf16 weights.
//   - A step issues its logits MFMAs, one (rarely taken) masking branch, one
//     rescale branch for all tiles, then per tile the weights and their PV
//     MFMAs: the common step is straight-line code.  Loop bounds and block ids
//     stay in scalar registers, and MFMA results stay in VGPRs (no AGPR
//     copies around the softmax code).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "pa_device.h"
#include "pa_launch.h"

namespace pa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kPrefillWaves = 4;
// A column's reference max moves when a logit exceeds it by more than this (log2 units).
constexpr float kLazyLog2 = 8.f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ f32x4 mfma_bf16_32(uint4 a, uint4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// max(a, b, c) in one v_max3_f32, max(a, b) in one v_max_f32.  The operands
// here are fma results, -inf, or results of these (never signalling NaNs), so
// the NaN-quieting the compiler puts before each operand of fmaxf in IEEE mode
// is not needed.
__device__ __forceinline__ float max3f(float a, float b, float c) {
    float r;
    asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    return r;
}
__device__ __forceinline__ float max2f(float a, float b) {
    float r;
    asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
    return r;
}

// 16 bytes per lane from `slab` (bytes in range) at byte `voffset` into LDS at
// `dst` + 16 * lane (dst wave-uniform): a buffer load with the lds flag, which
// writes LDS itself and counts in vmcnt.  (A __device__ function, not a lambda:
// the host pass of a kernel's lambdas must not see this builtin.)
__device__ __forceinline__ void load_lds16(const char *slab, int bytes, int voffset, char *dst) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        __builtin_amdgcn_make_buffer_rsrc(const_cast<char *>(slab), 0, bytes, kBufferWord3), dst, 16, voffset, 0,
        0, 0);
}

// The first `keep` (0..8) bf16 values of v, the rest zeroed.
__device__ __forceinline__ uint4 keep_first(uint4 v, int keep) {
    auto word = [&](uint32_t x, int k) -> uint32_t {
        return keep >= k + 2 ? x : (keep == k + 1 ? (x & 0x0000ffffu) : 0u);
    };
    return make_uint4(word(v.x, 0), word(v.y, 2), word(v.z, 4), word(v.w, 6));
}

// Grid: x = partition (0 for the single pass), y = kv head * column groups of
// kPrefillWaves * 16 * NCT columns, z = sequence.  Wave w of a workgroup owns
// columns cw .. cw + 16*NCT - 1; column c is (query token c / G, head kvh*G + c % G).
// kFinal: one pass over the whole sequence, output written.  Otherwise partition
// blockIdx.x of P tokens, partials written: tmp_out[row][p][D] (normalised
// output), exp_sums[row][p] (sum of exp(z - max)), max_logits[row][p] (max of z),
// with row = (s * q_len + token) * Hq + head and z = scale * q.k; a column that
// sees no token of the partition writes {0, 0, -inf}.
template <int D, int NCT, bool kFinal>
__global__ __launch_bounds__(kPrefillWaves * 64) void prefill_kernel(
    const uint16_t *__restrict__ query, const uint16_t *__restrict__ key_cache,
    const uint16_t *__restrict__ value_cache, const int32_t *__restrict__ block_tables,
    const int32_t *__restrict__ seq_lens, int num_q_heads, int num_kv_heads, int group, int qlen,
    int num_blocks, int max_blocks, int max_seq_len, float scale, int partition_size,
    int max_parts, float *__restrict__ tmp_out, float *__restrict__ exp_sums,
    float *__restrict__ max_logits, uint16_t *__restrict__ out) {
    constexpr int KS = D / 32;       // 32-wide steps over d (QK^T)
    constexpr int DT = D / 16;       // 16-row d tiles of the output
    constexpr int WCOLS = 16 * NCT;  // columns per wave
    constexpr int NW = kPrefillWaves;
    constexpr int kSlab = kBlockTokens * D * 2;  // bytes of one (block, kv head) slab
    constexpr int kPieces = kSlab / 16;          // 16-byte pieces per slab
    constexpr int kLoads = 4 * kPieces / (NW * 64);  // pieces per thread per step
    // LDS ring: kStages stages of four regions (keys of the step's two blocks,
    // then their values).  Regions are kSlab + 128 bytes apart: the two key
    // regions start half a 256-byte bank line apart (see the reads below).
    constexpr int kRegion = kSlab + 128;
    constexpr int kStage = 4 * kRegion;
    constexpr int kStages = 3;
    // One array per stage: the compiler tracks the loads that write LDS per
    // array, so reading one stage waits only for the loads into that stage
    // (with one array it would wait for every load in flight).
    static_assert(kStages == 3, "the step loop is unrolled by the stage count");
    __shared__ __attribute__((aligned(16))) char lds0[kStage];
    __shared__ __attribute__((aligned(16))) char lds1[kStage];
    __shared__ __attribute__((aligned(16))) char lds2[kStage];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = lane & 15;  // column of a tile; row of the A operands
    const int q = lane >> 4;  // lane group: k slots 8q .. 8q+7, result rows 4q .. 4q+3

    const int ncols = group * qlen;
    const int ygroups = (ncols + NW * WCOLS - 1) / (NW * WCOLS);
    const int kvh = blockIdx.y / ygroups;
    // Single pass: causal limits make a workgroup's work grow with its column
    // group (later query tokens see more of the cache).  The upper half of the kv
    // heads takes its column groups in reverse order, so workgroups y and
    // y + gridDim.y / 2 -- which share a CU when the grid fills two workgroups
    // per CU -- pair a heavy group with a light one.  Measured on MI355X (S 1,
    // Hq 32, Hkv 4, 8192 tokens; same-run A/B on two boxes): q_len 2048 -6.5 to
    // -7.6%, q_len 1024 -2.2 to -2.6%, q_len 512 unchanged.  Any order is correct: it is a permutation of the
    // column groups within each kv head.
    const int cg_index = blockIdx.y - kvh * ygroups;
    const bool reversed = kFinal && 2 * kvh >= num_kv_heads;
    const int cg = (reversed ? ygroups - 1 - cg_index : cg_index) * NW * WCOLS;  // first column
    const int cw = cg + w * WCOLS;                              // first column of this wave
    const bool has_cols = cw < ncols;  // a wave without columns still loads and waits
    const int s = blockIdx.z;
    const int L = min(max(seq_lens[s], 0), max_seq_len);
    const int nblk = (L + kBlockTokens - 1) / kBlockTokens;
    int p = 0, jb = 0, je = nblk;  // blocks [jb, je) of this partition
    if (!kFinal) {
        const int bp = partition_size / kBlockTokens;
        p = blockIdx.x;
        if (p >= (nblk + bp - 1) / bp) return;  // uniform: past the sequence, never read
        jb = p * bp;
        je = min(jb + bp, nblk);
    }

    // Columns of this lane: cw + 16 ct + n.  lim: the last cache token the column
    // sees (L - 1 for a column past the end, whose results are never stored).
    auto qrow_of = [&](int c) {  // query / output row of column c
        const int tok = c / group;
        return ((size_t)s * qlen + tok) * num_q_heads + (size_t)kvh * group + (c - tok * group);
    };
    // The maxima are taken over the raw products q.k and scaled afterwards, which
    // needs a positive factor: a negative scale flips the sign bits of the bf16
    // query instead (exact), and a zero scale becomes a tiny positive one (all
    // weights still round to 1).
    const uint32_t qsign = scale < 0.f ? 0x80008000u : 0u;
    const float c2 = fmaxf(fabsf(scale) * kLog2e, 1e-30f);  // |q.k| -> logit in log2 units
    int lim[NCT];
    uint4 qv[NCT][KS];  // Q^T operand: d = 32 ks + 8q .. +7 of the column's query row
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
        const int c = cw + 16 * ct + n;
        lim[ct] = c < ncols ? L - qlen + c / group : L - 1;
        const uint4 *src = reinterpret_cast<const uint4 *>(query + qrow_of(min(c, ncols - 1)) * D) + q;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const uint4 v = c < ncols ? src[4 * ks] : make_uint4(0, 0, 0, 0);
            qv[ct][ks] = make_uint4(v.x ^ qsign, v.y ^ qsign, v.z ^ qsign, v.w ^ qsign);
        }
    }
    // Causal range: the wave computes up to its own last column's limit, the
    // workgroup loads up to the last limit of all its columns.  These are uniform
    // (over the wave, the workgroup); readfirstlane keeps them in scalar
    // registers, so the loop control and the block ids stay scalar.
    const int lim_lo = __builtin_amdgcn_readfirstlane(L - qlen + cw / group);  // smallest of the wave
    const int lim_hi = __builtin_amdgcn_readfirstlane(
        has_cols ? L - qlen + (min(cw + WCOLS, ncols) - 1) / group : -1);
    const int lim_wg = L - qlen + (min(cg + NW * WCOLS, ncols) - 1) / group;
    const int je_g = __builtin_amdgcn_readfirstlane(
        lim_wg < 0 ? jb : max(jb, min(je, lim_wg / kBlockTokens + 1)));
    // Steps of two blocks; none without any cache block (every id would be skipped).
    const int nsteps = num_blocks > 0 ? (je_g - jb + 1) / 2 : 0;

    // m: the column's reference max; mt: this lane's part of the true max (log2
    // units), the maximum over the lane's own tokens, reduced over the column's
    // four lanes after the last step.
    float m[NCT], mt[NCT];
    f32x4 acc[NCT][DT];
    // Exp-sums: one more PV MFMA per tile against an all-ones A operand leaves
    // the column's sum of the (bf16) weights in every register of lane (n, q),
    // so the sums cost no VALU additions and use the very weights the output
    // does.
    f32x4 accl[NCT];
    uint4 ones = make_uint4(0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u);  // bf16 1.0
    // Opaque to the compiler, so the operand stays in four VGPRs instead of being
    // rebuilt from scalar registers (two v_mov_b64) in every step; measured on
    // MI355X, same-box A/B: q_len 2048 -0.4 to -0.8%, bitwise-identical.
    asm volatile("" : "+v"(ones.x), "+v"(ones.y), "+v"(ones.z), "+v"(ones.w));
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
        m[ct] = -INFINITY;
        mt[ct] = -INFINITY;
        accl[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < DT; ++t) acc[ct][t] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    const int32_t *bt = block_tables + (size_t)s * max_blocks;
    const char *kbase = reinterpret_cast<const char *>(key_cache) + (size_t)kvh * kSlab;
    const char *vbase = reinterpret_cast<const char *>(value_cache) + (size_t)kvh * kSlab;
    const size_t blk_stride = (size_t)num_kv_heads * kSlab;

    // Block ids of the step at block j (blocks j, j + 1); -1: not attended.
    auto ids = [&](int j, int &id0, int &id1) {
        id0 = j < je_g ? bt[j] : -1;
        id1 = j + 1 < je_g ? bt[j + 1] : -1;
        if ((unsigned)id0 >= (unsigned)num_blocks) id0 = -1;
        if ((unsigned)id1 >= (unsigned)num_blocks) id1 = -1;
    };
    // A step's 4 slabs (keys of blocks j, j + 1, then their values) go straight
    // from global memory into an LDS stage (buffer loads with the lds flag: the
    // data is written to LDS by the load itself, with no register staging and no
    // LDS store instruction in the wave).  Such a load writes 16 bytes per lane
    // at consecutive positions: lane l of wave w, load i, fills position
    // p = (256 i + 64 w + l) % kPieces of region r = (256 i + 64 w + l) / kPieces
    // (D = 128: region i; D = 64: region 2i + w / 2).  A 128-bit LDS read is
    // served 16 lanes per clock, 16 bytes each from the 16 slots of a 256-byte
    // bank line; the lanes served together share lane bit 5 and the parity of
    // lane bits 2..4 (lanes 0-3, 12-15, 20-23, 24-27 form one group; measured
    // on MI355X with the LDS bank-conflict counter), and a read is free of
    // conflicts when every group touches 16 distinct slots.  Key positions are
    // permuted to meet that; values are stored in slab order, which meets it
    // as is.  Position p of a key region holds piece swz(p) of its slab (swz
    // is its own inverse): piece (chunk c, token t) at 16c + (t ^ 4 * (t / 8)).
    // A block that is not attended is replaced by block 0 of the same kv head
    // (valid memory; its tokens are masked), so every step issues the same loads.
    int dma_lds[kLoads], dma_src[kLoads];  // LDS byte offset of the wave's run, lane's source byte
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
        const int k = tid + NW * 64 * i;
        const int r = k / kPieces;
        const int pos = k - r * kPieces;
        const int pc = r < 2 ? (pos ^ (((pos >> 3) & 1) << 2)) : pos;
        dma_lds[i] = __builtin_amdgcn_readfirstlane(r * kRegion + (pos - lane) * 16);
        dma_src[i] = pc * 16;  // byte offset inside the slab
    }
    auto dma = [&](char *stage, int id0, int id1) {
        const size_t o0 = (size_t)max(id0, 0) * blk_stride, o1 = (size_t)max(id1, 0) * blk_stride;
        const char *base[4] = {kbase + o0, kbase + o1, vbase + o0, vbase + o1};  // uniform
#pragma unroll
        for (int i = 0; i < kLoads; ++i) {
            const int r = (kLoads == 4) ? i : 2 * i + (w >> 1);  // uniform
            load_lds16(base[r], kSlab, dma_src[i], stage + dma_lds[i]);
        }
    };
    // LDS offsets of the operands.  Keys [D/8][16][8]: A row n of tile T is token
    // t = 8b + 4T + n%4 (b = (n/4)%2) of block n/8, d chunk 4 ks + q, stored at
    // token slot t ^ 4b = 8b + 4(T ^ b) + n%4.  Values [D][16]: lane (n, q) reads
    // row d = 16t + n, tokens 8*(q%2) .. +7 of block q/2.
    const int kb_ = (n >> 2) & 1;
    const int k_lds0 = (n >> 3) * kRegion + q * 256 + (8 * kb_ + 4 * kb_ + (n & 3)) * 16;        // T = 0
    const int k_lds1 = (n >> 3) * kRegion + q * 256 + (8 * kb_ + 4 * (1 - kb_) + (n & 3)) * 16;  // T = 1
    // Value piece x = 32t + 2n + q%2 of d tile t: one lane offset plus 512t.
    const int v_lds = (2 + (q >> 1)) * kRegion + (2 * n + (q & 1)) * 16;

    // One step of 32 tokens from an LDS stage: logits, reference update,
    // weights, PV.
    auto step = [&](int j, const char *stage, bool ok0, bool ok1) {
        const char *sk0 = stage + k_lds0;
        const char *sk1 = stage + k_lds1;
        const char *sv = stage + v_lds;  // + 512 t for d tile t
        const int t0 = j * kBlockTokens + 8 * q;  // lane's first token: t0 + 4T + i
        // Every token of the step attended and visible to every column of the wave.
        const bool full = ok0 && ok1 && j * kBlockTokens + 31 <= lim_lo;
        const bool okb = (q >> 1) ? ok1 : ok0;  // block of this lane's tokens
        uint4 kr[2][KS];
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                kr[t][ks] = *reinterpret_cast<const uint4 *>((t ? sk1 : sk0) + ks * 1024);
        // Logits of every tile first, so that the MFMAs run back to back.
        f32x4 sa[NCT][2];
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) a = mfma_bf16_32(kr[t][ks], qv[ct][ks], a);
                sa[ct][t] = a;
            }
        // The stretch from the logits to the exponentials (exponents, lane maxima,
        // growth test: a chain of dependent vector instructions) runs at raised
        // wave priority, so that it is not held up behind the MFMAs of the other
        // wave on the SIMD; the exponentials and PV MFMAs run at the normal one.
        // Measured on MI355X (q_len 2048 over 8192 tokens, same-box A/B): -6.5%;
        // priority 1 -5%, 3 the same as 2; raised over the MFMAs instead -2 to
        // -6%; raised over the exponentials too: no gain.
        __builtin_amdgcn_s_setprio(2);
        // Exponents of the weights against each column's reference: e = z log2 e - m
        // (z = scale q.k), taken before the column maxima so that the maxima run on
        // fma results, which need no NaN-quieting before each v_max.  A token the
        // column does not see gets e = -inf.
        auto masked = [&](int ct, int t, int i) { return !okb || t0 + 4 * t + i > lim[ct]; };
        float e[NCT][2][4];
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int i = 0; i < 4; ++i) e[ct][t][i] = fmaf(sa[ct][t][i], c2, -m[ct]);
        if (!full) {
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
                for (int t = 0; t < 2; ++t)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        if (masked(ct, t, i)) e[ct][t][i] = -INFINITY;
        }
        // The reference moves when some e of the column exceeds kLazyLog2, which
        // includes a column's first visible token (m = -inf gives e = +inf).  The
        // test runs on each lane's own maximum; only a step where some lane
        // passes it (rare after the first) takes the column maxima across the
        // four lanes, in one wave-uniform branch for all tiles.
        auto lane_max8 = [](const float (&v)[2][4]) {
            return max2f(max3f(max3f(max3f(v[0][0], v[0][1], v[0][2]), v[0][3], v[1][0]), v[1][1], v[1][2]),
                         v[1][3]);
        };
        auto col_max8 = [](const float (&v)[2][4]) {
            return column_max(fmaxf(fmaxf(fmaxf(v[0][0], v[0][1]), fmaxf(v[0][2], v[0][3])),
                                    fmaxf(fmaxf(v[1][0], v[1][1]), fmaxf(v[1][2], v[1][3]))));
        };
        float mxe[NCT];  // this lane's largest e
        float mx_all = -INFINITY;
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
            mxe[ct] = lane_max8(e[ct]);
            mx_all = ct == 0 ? mxe[0] : max2f(mx_all, mxe[ct]);
        }
        if (__builtin_amdgcn_ballot_w64(mx_all > kLazyLog2) != 0) {
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) {
                const float cmx = column_max(mxe[ct]);  // the column's largest e
                if (cmx > kLazyLog2) {  // the same for the four lanes of a column
                    // New reference: the step's largest scaled logit, i.e. m + max e,
                    // or -- for a column that had seen nothing -- the max over the
                    // visible raw products, scaled.
                    float m_new = m[ct] + cmx;
                    if (m[ct] == -INFINITY) {
                        float raw[2][4];
#pragma unroll
                        for (int t = 0; t < 2; ++t)
#pragma unroll
                            for (int i = 0; i < 4; ++i)
                                raw[t][i] = (!full && masked(ct, t, i)) ? -INFINITY : sa[ct][t][i];
                        m_new = col_max8(raw) * c2;
                    }
                    const float alpha = m[ct] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m[ct] - m_new);
                    m[ct] = m_new;
                    mxe[ct] = 0.f;  // the step's max, against the new reference
                    accl[ct] *= alpha;
#pragma unroll
                    for (int t = 0; t < DT; ++t) acc[ct][t] *= alpha;
#pragma unroll
                    for (int t = 0; t < 2; ++t)
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            e[ct][t][i] = (!full && masked(ct, t, i)) ? -INFINITY
                                                                      : fmaf(sa[ct][t][i], c2, -m_new);
                }
            }
        }
        // True max of the scaled logits (log2 units), for the partials: a lane
        // that saw nothing in this step has mxe = -inf and keeps mt.  (Rounding
        // of m + x is monotonic in x, so the column's maximum over its lanes
        // equals m + the column's largest e.)
        if constexpr (!kFinal) {
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) mt[ct] = fmaxf(mt[ct], m[ct] + mxe[ct]);
        }
        // Values first (one masking branch), then per tile: weights, then its PV
        // MFMAs, so the exponentials of tile ct + 1 can run while the matrix
        // cores work on tile ct.
        uint4 vv[DT];
#pragma unroll
        for (int t = 0; t < DT; ++t) vv[t] = *reinterpret_cast<const uint4 *>(sv + 512 * t);
        if (!full) {
            // Value slots past the sequence end (or of a block not attended) are
            // zeroed: their weights are 0, and 0 * NaN must not reach the sums.
            const int keep = okb ? min(max(L - t0, 0), 8) : 0;
#pragma unroll
            for (int t = 0; t < DT; ++t) vv[t] = keep_first(vv[t], keep);
        }
        __builtin_amdgcn_s_setprio(0);
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
            float pr[2][4];
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int i = 0; i < 4; ++i) pr[t][i] = __builtin_amdgcn_exp2f(e[ct][t][i]);  // 2^-inf = 0
            const uint4 pb = make_uint4(pack2_bf16(pr[0][0], pr[0][1]), pack2_bf16(pr[0][2], pr[0][3]),
                                        pack2_bf16(pr[1][0], pr[1][1]), pack2_bf16(pr[1][2], pr[1][3]));
#pragma unroll
            for (int t = 0; t < DT; ++t) acc[ct][t] = mfma_bf16_32(vv[t], pb, acc[ct][t]);
            accl[ct] = mfma_bf16_32(ones, pb, accl[ct]);
        }
    };

    // Pipeline: the loads of step i + 2 are issued into stage (i + 2) % 3 when
    // step i starts, so global latency has two steps to hide.  That stage held
    // step i - 1, which every wave finished before the barrier that opened step
    // i.  Before the barrier that opens step i + 1, each wave waits for its own
    // loads of step i + 1 (only those of step i + 2, issued later, may still be
    // in flight); after it, every wave's loads of step i + 1 are in LDS.  The
    // waits are explicit and the barrier is s_barrier alone: __syncthreads()
    // would also wait for the loads of step i + 2.  The empty asm statements with
    // a memory clobber keep the compiler from moving LDS accesses across them.
    if (nsteps > 0) {
        int a0, a1, b0, b1, c0, c1;  // block ids of steps i, i + 1, i + 2
        ids(jb, a0, a1);
        dma(lds0, a0, a1);
        ids(jb + 2, b0, b1);
        dma(lds1, b0, b1);  // past the end the loads read block 0 (never used)
        auto publish = [&]() {  // own loads of the next step landed, then the barrier
            if constexpr (kLoads == 4) asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
            else asm volatile("s_waitcnt vmcnt(2)" ::: "memory");
            __builtin_amdgcn_s_barrier();
            asm volatile("" ::: "memory");
        };
        publish();
        auto iteration = [&](int i, const char *cur, char *ahead) {  // step i from cur; step i + 2 into ahead
            ids(jb + 2 * (i + 2), c0, c1);
            dma(ahead, c0, c1);
            if (has_cols && (jb + 2 * i) * kBlockTokens <= lim_hi) step(jb + 2 * i, cur, a0 >= 0, a1 >= 0);
            publish();
            a0 = b0;
            a1 = b1;
            b0 = c0;
            b1 = c1;
        };
        // Whole rounds of three, then the rest (uniform over the workgroup): every
        // way into the loop head comes from the same stage order, which keeps the
        // compiler's waits for each stage exact.
        int i = 0;
        for (; i + 2 < nsteps; i += 3) {
            iteration(i, lds0, lds2);
            iteration(i + 1, lds1, lds0);
            iteration(i + 2, lds2, lds1);
        }
        if (i < nsteps) iteration(i, lds0, lds2);
        if (i + 1 < nsteps) iteration(i + 1, lds1, lds0);
        // The loads issued past the last step (block 0, never read) land before
        // the workgroup ends.
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    if (!has_cols) return;

    // Results: lane (n, q) holds d = 16t + 4q + r of column cw + 16 ct + n.
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
        const float lc = accl[ct][0];  // the column's exp-sum (all four registers hold it)
        if constexpr (!kFinal) mt[ct] = column_max(mt[ct]);
        const int c = cw + 16 * ct + n;
        if (c >= ncols) continue;
        const float inv = lc > 0.f ? 1.f / lc : 0.f;
        if (kFinal) {
            uint16_t *orow = out + qrow_of(c) * D + 4 * q;
#pragma unroll
            for (int t = 0; t < DT; ++t) {
                const f32x4 o = acc[ct][t] * inv;
                *reinterpret_cast<u32x2 *>(orow + 16 * t) = u32x2{pack2_bf16(o[0], o[1]), pack2_bf16(o[2], o[3])};
            }
        } else {
            const size_t row = qrow_of(c) * max_parts + p;
            float *orow = tmp_out + row * D + 4 * q;
#pragma unroll
            for (int t = 0; t < DT; ++t) *reinterpret_cast<f32x4 *>(orow + 16 * t) = acc[ct][t] * inv;
            if (q == 0) {
                // exp-sum against the true max: sum 2^(z' - m) * 2^(m - mt).
                exp_sums[row] = mt[ct] == -INFINITY ? 0.f : lc * __builtin_amdgcn_exp2f(m[ct] - mt[ct]);
                max_logits[row] = mt[ct] * kLn2;
            }
        }
    }
}

template <int D, int NCT, bool kFinal>
hipError_t launch_prefill_t(const Problem &pb, const Partials *parts, void *out, hipStream_t stream) {
    const int group = pb.num_q_heads / pb.num_kv_heads;
    const int ygroups = prefill_column_groups(group, pb.qlen, NCT);
    dim3 grid(kFinal ? 1 : parts->max_parts, pb.num_kv_heads * ygroups, pb.num_seqs);
    prefill_kernel<D, NCT, kFinal><<<grid, kPrefillWaves * 64, 0, stream>>>(
        static_cast<const uint16_t *>(pb.query), static_cast<const uint16_t *>(pb.key_cache),
        static_cast<const uint16_t *>(pb.value_cache), pb.block_tables, pb.seq_lens, pb.num_q_heads,
        pb.num_kv_heads, group, pb.qlen, pb.num_blocks, pb.max_blocks, pb.max_seq_len, pb.scale,
        kFinal ? kBlockTokens : parts->partition_size, kFinal ? 0 : parts->max_parts,
        kFinal ? nullptr : parts->tmp_out, kFinal ? nullptr : parts->exp_sums,
        kFinal ? nullptr : parts->max_logits, static_cast<uint16_t *>(out));
    return hipGetLastError();
}

template <int D, bool kFinal>
hipError_t launch_prefill_d(const Problem &pb, const Partials *parts, void *out, int nct,
                            hipStream_t stream) {
    switch (nct) {
        case 1: return launch_prefill_t<D, 1, kFinal>(pb, parts, out, stream);
        case 2: return launch_prefill_t<D, 2, kFinal>(pb, parts, out, stream);
        default: return launch_prefill_t<D, 4, kFinal>(pb, parts, out, stream);
    }
}

}  // namespace

int prefill_column_groups(int group, int qlen, int nct) {
    const int per = kPrefillWaves * 16 * nct;
    return (int)(((long long)group * qlen + per - 1) / per);
}

hipError_t launch_prefill(const Problem &pb, const Partials *parts, void *out, int nct,
                          hipStream_t stream) {
    if (pb.dtype != Dtype::BF16) return hipErrorInvalidValue;
    if (parts == nullptr) {
        return pb.head_dim == 64 ? launch_prefill_d<64, true>(pb, nullptr, out, nct, stream)
                                 : launch_prefill_d<128, true>(pb, nullptr, out, nct, stream);
    }
    return pb.head_dim == 64 ? launch_prefill_d<64, false>(pb, parts, nullptr, nct, stream)
                             : launch_prefill_d<128, false>(pb, parts, nullptr, nct, stream);
}

}  // namespace pa
