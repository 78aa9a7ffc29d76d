/*
 * pa_oracle.c -- CPU reference ("oracle") for paged single-query decode attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may load this file or
 * the library built from it; only the test suite, the smoke check and the CPU
 * baseline leg of the benchmark do.  It shares no code, header, table or helper
 * with the HIP library: it is written from the method's definition alone so
 * that the two can disagree.
 *
 * Sources (pages of the project_6 commit history that define the method):
 *   [p1] commit 900ae0b, vllm/_custom_ops.py -- messages "Two changes based on
 *        CCCL source reading" and "THE SINGLE HIGHEST-IMPACT CODE CHANGE".
 *   [p2] commit 490ff98, paged_attn.py -- the summary_statistics /
 *        online-softmax message and the "Three changes" message.
 *   [p3] commit 15ef28e, paged_attention_v2_pytorch.py -- messages
 *        "[OPT] Vectorize paged_attention_v2" and
 *        "[OPT] PagedAttention V2 implementation".
 *
 * What is computed.  V1 (single pass) and V2 (partitioned, then merged) are two
 * schedules of one exact function: softmax attention of one query vector per
 * (sequence, query head) over that sequence's cached keys and values.  So the
 * reference for both is that function written out, in double precision:
 *
 *   for query head h of sequence s with length L = seq_lens[s]:
 *     kv head        kvh = h / G,  G = num_q_heads / num_kv_heads
 *                    (query heads are grouped contiguously over kv heads;
 *                     [p2] online-softmax message, heads batched as
 *                     [kv_h, gqa, ...]; [p3] Vectorize message, GQA by
 *                     expanding each kv head over its group)
 *     token t < L    lives in physical block block_tables[s][t / 16],
 *                    slot t % 16 ([p3] Vectorize message: keys and values are
 *                    fetched through the per-sequence block id list)
 *     logit          z_t = scale * sum_d q[d] * k_t[d]
 *     output         out = sum_t exp(z_t - M) v_t / sum_t exp(z_t - M),
 *                    M = max_t z_t
 *
 * A second entry computes the pages' two-phase form literally ([p3]
 * "PagedAttention V2 implementation", Phase 1 and Phase 2): per partition of
 * partition_size consecutive tokens the max logit m_p, the exp-sum
 * s_p = sum exp(z_t - m_p) and the normalised partial output
 * o_p = sum exp(z_t - m_p) v_t / s_p; then the merge with the global max,
 * the rescale exp(m_p - M) * s_p and the weighted sum of the o_p.
 *
 * Readings where the pages are silent (each also listed in the design notes):
 *   - paged caches in the split layout of the pages' host project (the pages
 *     gather whole blocks by id and then permute and reshape them into token
 *     order, which leaves the in-block order open): keys
 *     [num_blocks][num_kv_heads][head_dim / x][block_size][x] with x = 16 bytes
 *     / element size (8 bf16 or 4 float32 values), values
 *     [num_blocks][num_kv_heads][head_dim][block_size]; query and output
 *     [num_seqs][num_q_heads][head_dim], block table int32
 *     [num_seqs][max_blocks_per_seq] (all row-major, contiguous);
 *   - the scale multiplies q.k before the max is taken;
 *   - tokens at or beyond L are excluded (never read), not zero-weighted;
 *   - L == 0 gives an all-zero output row;
 *   - bf16 values are widened exactly (bits << 16) and scale is the float
 *     argument widened to double.
 *
 * Parity pins (brute force, closed forms, invariants) live in the test suite.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_F32 0
#define ORACLE_BF16 1

/* Element idx of a float32 or bfloat16 array, widened exactly to double. */
static double elem(const void *base, size_t idx, int dtype) {
    if (dtype == ORACLE_F32) {
        return (double)((const float *)base)[idx];
    }
    uint32_t bits = ((uint32_t)((const uint16_t *)base)[idx]) << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

typedef struct {
    const void *query, *key_cache, *value_cache;
    int dtype;
    const int32_t *block_tables, *seq_lens;
    int num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq;
    double scale;
    int q_len; /* query tokens per sequence (1 for plain decode) */
} problem_t;

/* Values per 16-byte group of the key layout. */
static int key_group(int dtype) { return dtype == ORACLE_BF16 ? 8 : 4; }

static int check_problem(const problem_t *pb) {
    if (!pb->query || !pb->key_cache || !pb->value_cache || !pb->block_tables || !pb->seq_lens)
        return -1;
    if (pb->dtype != ORACLE_F32 && pb->dtype != ORACLE_BF16) return -2;
    if (pb->head_dim % key_group(pb->dtype) != 0) return -3;
    if (pb->num_seqs < 0 || pb->num_q_heads <= 0 || pb->num_kv_heads <= 0 || pb->head_dim <= 0 ||
        pb->block_size <= 0 || pb->max_blocks_per_seq < 0)
        return -3;
    if (pb->num_q_heads % pb->num_kv_heads != 0) return -4;
    return 0;
}

/* (block, kv head) slab index of token t of sequence s, and its slot. */
static size_t slab_of(const problem_t *pb, int s, int kvh, int t, int *slot) {
    int32_t phys = pb->block_tables[(size_t)s * pb->max_blocks_per_seq + t / pb->block_size];
    *slot = t % pb->block_size;
    return (size_t)phys * pb->num_kv_heads + kvh;
}

/* Element index of K[t][d] (token t of sequence s, kv head kvh) in the key cache
 * [num_blocks][num_kv_heads][head_dim / x][block_size][x]. */
static size_t key_index(const problem_t *pb, int s, int kvh, int t, int d) {
    int slot;
    size_t slab = slab_of(pb, s, kvh, t, &slot);
    int x = key_group(pb->dtype);
    return ((slab * (size_t)(pb->head_dim / x) + (size_t)(d / x)) * pb->block_size + slot) * x +
           d % x;
}

/* Element index of V[t][d] in the value cache
 * [num_blocks][num_kv_heads][head_dim][block_size]. */
static size_t value_index(const problem_t *pb, int s, int kvh, int t, int d) {
    int slot;
    size_t slab = slab_of(pb, s, kvh, t, &slot);
    return (slab * (size_t)pb->head_dim + (size_t)d) * pb->block_size + slot;
}

/* Scaled logit z_t of query head h of sequence s against token t.  With q_len
 * query tokens per sequence, h is the combined index j * num_q_heads + head of
 * query token j ([num_seqs][q_len][num_q_heads] rows). */
static double logit(const problem_t *pb, int s, int h, int t) {
    int G = pb->num_q_heads / pb->num_kv_heads;
    size_t qoff = ((size_t)s * pb->q_len * pb->num_q_heads + h) * pb->head_dim;
    h %= pb->num_q_heads;
    double dot = 0.0;
    for (int d = 0; d < pb->head_dim; ++d)
        dot += elem(pb->query, qoff + d, pb->dtype) *
               elem(pb->key_cache, key_index(pb, s, h / G, t, d), pb->dtype);
    return pb->scale * dot;
}

/* Plain softmax attention over tokens [t0, t1) of (s, h).  Writes the
 * normalised weighted V sum to o[head_dim]; returns the max logit through *m
 * and sum_t exp(z_t - max) through *den.  Requires t1 > t0. */
static int attend_range(const problem_t *pb, int s, int h, int t0, int t1, double *o, double *m,
                        double *den) {
    int n = t1 - t0;
    int G = pb->num_q_heads / pb->num_kv_heads;
    int hv = h % pb->num_q_heads; /* query head of the combined (token, head) index h */
    double *z = (double *)malloc(sizeof(double) * (size_t)n);
    if (!z) return -10;
    double zmax = -INFINITY;
    for (int t = t0; t < t1; ++t) {
        z[t - t0] = logit(pb, s, h, t);
        if (z[t - t0] > zmax) zmax = z[t - t0];
    }
    for (int d = 0; d < pb->head_dim; ++d) o[d] = 0.0;
    double sum = 0.0;
    for (int t = t0; t < t1; ++t) {
        double w = exp(z[t - t0] - zmax);
        sum += w;
        for (int d = 0; d < pb->head_dim; ++d)
            o[d] += w * elem(pb->value_cache, value_index(pb, s, hv / G, t, d), pb->dtype);
    }
    for (int d = 0; d < pb->head_dim; ++d) o[d] /= sum;
    free(z);
    *m = zmax;
    *den = sum;
    return 0;
}

/*
 * Full-softmax decode attention.  If rows is NULL, out is [num_seqs][num_q_heads]
 * [head_dim] for every (s, h); otherwise rows holds num_rows (s, h) pairs and out
 * is [num_rows][head_dim].  Returns 0, or a negative code for bad arguments.
 * num_threads <= 0 uses the OpenMP default.
 */
int pa_oracle_decode(double *out, const void *query, const void *key_cache, const void *value_cache,
                     int dtype, const int32_t *block_tables, const int32_t *seq_lens, int num_seqs,
                     int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                     int max_blocks_per_seq, float scale, const int32_t *rows, int num_rows,
                     int num_threads) {
    problem_t pb = {query, key_cache, value_cache, dtype, block_tables, seq_lens,
                    num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                    max_blocks_per_seq, (double)scale, 1};
    int rc = check_problem(&pb);
    if (rc) return rc;
    if (!out) return -1;
    long n = rows ? (long)num_rows : (long)num_seqs * num_q_heads;
    if (rows) {
        for (long i = 0; i < n; ++i)
            if (rows[2 * i] < 0 || rows[2 * i] >= num_seqs || rows[2 * i + 1] < 0 ||
                rows[2 * i + 1] >= num_q_heads)
                return -5;
    }
#ifdef _OPENMP
    if (num_threads > 0) omp_set_num_threads(num_threads);
#else
    (void)num_threads;
#endif
    int failed = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (long i = 0; i < n; ++i) {
        int s = rows ? rows[2 * i] : (int)(i / num_q_heads);
        int h = rows ? rows[2 * i + 1] : (int)(i % num_q_heads);
        double *o = out + (size_t)i * head_dim;
        int L = seq_lens[s];
        if (L <= 0) {
            for (int d = 0; d < head_dim; ++d) o[d] = 0.0;
            continue;
        }
        double m, den;
        if (attend_range(&pb, s, h, 0, L, o, &m, &den)) {
#pragma omp atomic write
            failed = 1;
        }
    }
    return failed ? -10 : 0;
}

/*
 * Phase 1 of the partitioned form: for every (s, h) and every partition
 * p < ceil(L / partition_size), the partial output o_p (normalised), the
 * exp-sum s_p and the max logit m_p of tokens [p*P, min((p+1)*P, L)).
 * tmp_out is [num_seqs][num_q_heads][max_partitions][head_dim]; exp_sums and
 * max_logits are [num_seqs][num_q_heads][max_partitions].  Entries of
 * partitions p >= ceil(L / P) are set to NaN (they are not defined).
 * Returns -6 if some sequence needs more than max_partitions partitions.
 */
int pa_oracle_partials(double *tmp_out, double *exp_sums, double *max_logits, const void *query,
                       const void *key_cache, const void *value_cache, int dtype,
                       const int32_t *block_tables, const int32_t *seq_lens, int num_seqs,
                       int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                       int max_blocks_per_seq, float scale, int partition_size, int max_partitions,
                       int num_threads) {
    problem_t pb = {query, key_cache, value_cache, dtype, block_tables, seq_lens,
                    num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                    max_blocks_per_seq, (double)scale, 1};
    int rc = check_problem(&pb);
    if (rc) return rc;
    if (!tmp_out || !exp_sums || !max_logits) return -1;
    if (partition_size <= 0 || max_partitions < 0) return -3;
    for (int s = 0; s < num_seqs; ++s) {
        long parts = seq_lens[s] > 0 ? ((long)seq_lens[s] + partition_size - 1) / partition_size : 0;
        if (parts > max_partitions) return -6;
    }
#ifdef _OPENMP
    if (num_threads > 0) omp_set_num_threads(num_threads);
#else
    (void)num_threads;
#endif
    long n = (long)num_seqs * num_q_heads * max_partitions;
    int failed = 0;
#pragma omp parallel for schedule(dynamic, 4)
    for (long i = 0; i < n; ++i) {
        int p = (int)(i % max_partitions);
        long sh = i / max_partitions;
        int s = (int)(sh / num_q_heads);
        int h = (int)(sh % num_q_heads);
        int L = seq_lens[s];
        int t0 = p * partition_size;
        double *o = tmp_out + (size_t)i * head_dim;
        if (L <= 0 || t0 >= L) {
            for (int d = 0; d < head_dim; ++d) o[d] = NAN;
            exp_sums[i] = NAN;
            max_logits[i] = NAN;
            continue;
        }
        int t1 = t0 + partition_size < L ? t0 + partition_size : L;
        if (attend_range(&pb, s, h, t0, t1, o, &max_logits[i], &exp_sums[i])) {
#pragma omp atomic write
            failed = 1;
        }
    }
    return failed ? -10 : 0;
}

/*
 * Phase 2 of the partitioned form ([p3] "PagedAttention V2 implementation",
 * Phase 2): over the partitions p < ceil(L / P) of each (s, h),
 *   M = max_p m_p,   r_p = exp(m_p - M) * s_p,   R = sum_p r_p,
 *   out = sum_p (r_p / R) * o_p.
 * Inputs as written by pa_oracle_partials (or any partials of that layout);
 * out is [num_seqs][num_q_heads][head_dim].  L == 0 gives a zero row.
 */
int pa_oracle_merge(double *out, const double *tmp_out, const double *exp_sums,
                    const double *max_logits, const int32_t *seq_lens, int num_seqs,
                    int num_q_heads, int head_dim, int partition_size, int max_partitions) {
    if (!out || !tmp_out || !exp_sums || !max_logits || !seq_lens) return -1;
    if (num_seqs < 0 || num_q_heads <= 0 || head_dim <= 0 || partition_size <= 0 ||
        max_partitions < 0)
        return -3;
    for (int s = 0; s < num_seqs; ++s) {
        int L = seq_lens[s];
        long parts = L > 0 ? ((long)L + partition_size - 1) / partition_size : 0;
        if (parts > max_partitions) return -6;
        for (int h = 0; h < num_q_heads; ++h) {
            size_t sh = (size_t)s * num_q_heads + h;
            double *o = out + sh * head_dim;
            for (int d = 0; d < head_dim; ++d) o[d] = 0.0;
            if (parts == 0) continue;
            const double *m = max_logits + sh * max_partitions;
            const double *es = exp_sums + sh * max_partitions;
            const double *po = tmp_out + sh * max_partitions * head_dim;
            double gmax = -INFINITY;
            for (long p = 0; p < parts; ++p)
                if (m[p] > gmax) gmax = m[p];
            double total = 0.0;
            for (long p = 0; p < parts; ++p) total += exp(m[p] - gmax) * es[p];
            for (long p = 0; p < parts; ++p) {
                double wgt = exp(m[p] - gmax) * es[p] / total;
                for (int d = 0; d < head_dim; ++d) o[d] += wgt * po[p * head_dim + d];
            }
        }
    }
    return 0;
}

/*
 * Decode of q_len query tokens per sequence (q_len >= 1).  The tokens are the
 * last q_len positions of the sequence, already in the cache: query token j of
 * sequence s sits at position L - q_len + j (L = seq_lens[s]) and attends to
 * the tokens 0 .. L - q_len + j (causal over the cache; the pages batch a
 * q_len dimension next to the GQA group, commit 490ff98, the summary_statistics
 * message).  A query token that sees no token (L - q_len + j < 0) gets a zero
 * row.  query and out are [num_seqs][q_len][num_q_heads][head_dim]; the rest
 * as pa_oracle_decode.
 */
int pa_oracle_decode_q(double *out, const void *query, const void *key_cache,
                       const void *value_cache, int dtype, const int32_t *block_tables,
                       const int32_t *seq_lens, int num_seqs, int q_len, int num_q_heads,
                       int num_kv_heads, int head_dim, int block_size, int max_blocks_per_seq,
                       float scale, int num_threads) {
    problem_t pb = {query, key_cache, value_cache, dtype, block_tables, seq_lens,
                    num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                    max_blocks_per_seq, (double)scale, q_len};
    int rc = check_problem(&pb);
    if (rc) return rc;
    if (!out) return -1;
    if (q_len < 1) return -3;
#ifdef _OPENMP
    if (num_threads > 0) omp_set_num_threads(num_threads);
#else
    (void)num_threads;
#endif
    long rows_per_seq = (long)q_len * num_q_heads;
    long n = (long)num_seqs * rows_per_seq;
    int failed = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (long i = 0; i < n; ++i) {
        int s = (int)(i / rows_per_seq);
        int hj = (int)(i % rows_per_seq); /* j * num_q_heads + h */
        int j = hj / num_q_heads;
        double *o = out + (size_t)i * head_dim;
        int visible = seq_lens[s] - q_len + j + 1; /* tokens 0 .. L - q_len + j */
        if (visible <= 0) {
            for (int d = 0; d < head_dim; ++d) o[d] = 0.0;
            continue;
        }
        double m, den;
        if (attend_range(&pb, s, hj, 0, visible, o, &m, &den)) {
#pragma omp atomic write
            failed = 1;
        }
    }
    return failed ? -10 : 0;
}
