/*
 * CPU oracle for one packed paged-attention step (fp64).
 *
 * TEST INFRASTRUCTURE ONLY. This file is the plain, slow, obviously correct
 * definition that the HIP kernels are checked against. It shares no code,
 * header, table or helper with the GPU library, and the GPU library never
 * links or calls it. Only the tests, the graft entry's smoke check and the
 * benchmark's CPU-baseline leg may load it.
 *
 * What it computes, and the passage each part follows:
 *
 *  - slot of a logical position: PageServe, "03 Paged KV cache" (the
 *    attention_wrapper code box) and "01 Scheduler loop / System
 *    architecture": a token at position pos of a sequence lives in
 *    physical block block_table[pos / 16], row pos % 16; the flat slot is
 *    block * 16 + row.
 *  - pool layout: PageServe, "06 Development history", phase 7: one
 *    pre-allocated pool [layers, blocks, 16, H, D]; tinyserve README, "How
 *    it works": K and V are two separate slabs, H is the number of KV heads.
 *  - positions of a step's tokens: PageServe "01 Scheduler loop" (Pack:
 *    explicit position_ids; System architecture: num_computed_tokens is
 *    the only scheduling number). Token i of a sequence whose first c
 *    tokens already have K/V in the pool sits at position c + i.
 *  - the scatter: PageServe "01 Scheduler loop" (Execute: writes K/V into
 *    the pool) and "03 Paged KV cache" (the backend scatters new K/V into
 *    the slots): a pure copy of each new token's K and V rows.
 *  - attention: PageServe "03 Paged KV cache" and phase 8 (attends through
 *    the block table, one packed [1, T] pass mixing prefill chunks and
 *    decodes); tinyserve README "Highlights" (grouped-query attention) and
 *    "How it works" (speculative rows use a stepped causal mask). Query
 *    token at position p of sequence s, head h, attends keys 0..p of s
 *    through KV head h / (Hq / Hkv) with softmax(scale * q.k) weights.
 *
 *  - rotary position embedding: tinyserve README, "Highlights" (the Qwen2
 *    forward pass applies rotary embeddings) with PageServe "01 Scheduler
 *    loop" (Pack: explicit position_ids). Read as Qwen2's rotation: for
 *    j < D/2 the pair (x[j], x[j + D/2]) turns by the angle
 *    pos * theta^(-2j/D).
 *  - speculative verification: PageServe "06 Development history" / Next
 *    steps (rejection sampling, so speculation also serves sampled
 *    requests) and tinyserve README "How it works" (Speculative decoding:
 *    draft i is kept with probability min(1, p_i(d_i) / q_i(d_i)); at the
 *    first rejection the replacement comes from normalize(max(p_i - q_i,
 *    0)); when every draft survives a bonus token comes from the last
 *    target distribution). The random numbers are inputs: one uniform per
 *    draft for its acceptance and one per sequence for the final draw.
 *
 * Everything is fp64; inputs arrive already rounded to the storage dtype
 * and upcast by the caller.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* Flat slot of logical position pos (PageServe "03 Paged KV cache"). */
int64_t oracle_slot(const int32_t *block_table_row, int64_t pos, int32_t block_size)
{
    return (int64_t)block_table_row[pos / block_size] * block_size + pos % block_size;
}

/* Byte offset of (layer, slot) row inside a pool laid out as
 * [layers, blocks, block_size, Hkv, D] with elt-byte elements. */
static int64_t pool_row_offset(int32_t layer, int32_t num_blocks, int32_t block_size,
                               int64_t slot, int64_t row_bytes)
{
    return ((int64_t)layer * num_blocks * block_size + slot) * row_bytes;
}

/*
 * Store n consecutive token rows of one sequence, starting at logical
 * position pos0, into the pools. k_rows / v_rows hold n rows of
 * Hkv * D * elt bytes each. A pure byte copy.
 */
void oracle_store_tokens(uint8_t *pool_k, uint8_t *pool_v,
                         int32_t layer, int32_t num_blocks, int32_t block_size,
                         int32_t num_kv_heads, int32_t head_dim, int32_t elt,
                         const int32_t *block_table_row, int64_t pos0, int64_t n,
                         const uint8_t *k_rows, const uint8_t *v_rows)
{
    const int64_t row_bytes = (int64_t)num_kv_heads * head_dim * elt;
    for (int64_t i = 0; i < n; ++i) {
        const int64_t slot = oracle_slot(block_table_row, pos0 + i, block_size);
        const int64_t off = pool_row_offset(layer, num_blocks, block_size, slot, row_bytes);
        memcpy(pool_k + off, k_rows + i * row_bytes, (size_t)row_bytes);
        memcpy(pool_v + off, v_rows + i * row_bytes, (size_t)row_bytes);
    }
}

/*
 * The step's KV scatter: token i of sequence s (packed at row
 * sum_{s'<s} q_lens[s'] + i of k and v) goes to position
 * num_computed[s] + i of s.
 */
void oracle_reshape_and_cache(uint8_t *pool_k, uint8_t *pool_v,
                              int32_t layer, int32_t num_blocks, int32_t block_size,
                              int32_t num_kv_heads, int32_t head_dim, int32_t elt,
                              const uint8_t *k, const uint8_t *v,
                              const int32_t *q_lens, const int32_t *num_computed,
                              const int32_t *block_tables, int32_t bt_stride, int32_t num_seqs)
{
    const int64_t row_bytes = (int64_t)num_kv_heads * head_dim * elt;
    int64_t t0 = 0;
    for (int32_t s = 0; s < num_seqs; ++s) {
        oracle_store_tokens(pool_k, pool_v, layer, num_blocks, block_size,
                            num_kv_heads, head_dim, elt,
                            block_tables + (int64_t)s * bt_stride,
                            num_computed[s], q_lens[s],
                            k + t0 * row_bytes, v + t0 * row_bytes);
        t0 += q_lens[s];
    }
}

/*
 * Read positions [0, n) of one sequence back out of the pools through its
 * block table into contiguous rows (used to check that the pool holds each
 * sequence's logical K/V).
 */
void oracle_gather(const uint8_t *pool_k, const uint8_t *pool_v,
                   int32_t layer, int32_t num_blocks, int32_t block_size,
                   int32_t num_kv_heads, int32_t head_dim, int32_t elt,
                   const int32_t *block_table_row, int64_t n,
                   uint8_t *k_rows, uint8_t *v_rows)
{
    const int64_t row_bytes = (int64_t)num_kv_heads * head_dim * elt;
    for (int64_t pos = 0; pos < n; ++pos) {
        const int64_t slot = oracle_slot(block_table_row, pos, block_size);
        const int64_t off = pool_row_offset(layer, num_blocks, block_size, slot, row_bytes);
        memcpy(k_rows + pos * row_bytes, pool_k + off, (size_t)row_bytes);
        memcpy(v_rows + pos * row_bytes, pool_v + off, (size_t)row_bytes);
    }
}

/*
 * Causal grouped-query attention of a packed step over each sequence's
 * contiguous K/V.
 *
 *   q        [T, Hq, D]   this step's queries, packed sequence after sequence
 *   kctx     [sum_s num_computed[s], Hkv, D]  cached context K of every
 *            sequence, sequence after sequence (positions 0..c_s-1)
 *   vctx     same for V
 *   knew     [T, Hkv, D]  this step's K (positions c_s..c_s+n_s-1)
 *   vnew     same for V
 *   row_sel  [T * Hq] bytes; nonzero selects the (token, head) rows to
 *            compute, NULL computes all. Unselected rows are left alone.
 *   out      [T, Hq, D]
 *
 * For query token i of sequence s (position p = c_s + i) and head h, with
 * j = h / (Hq / Hkv):
 *   z_t = scale * sum_d q[h, d] * K_s[t, j, d]      for t = 0..p
 *   w_t = exp(z_t - max z) / sum_t' exp(z_t' - max z)
 *   out[h, :] = sum_t w_t * V_s[t, j, :]
 * Rows run in parallel (one OpenMP iteration per (token, head)).
 */
void oracle_attention(const double *q, const double *kctx, const double *vctx,
                      const double *knew, const double *vnew,
                      const int32_t *q_lens, const int32_t *num_computed, int32_t num_seqs,
                      int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                      double scale, const uint8_t *row_sel, double *out)
{
    const int64_t D = head_dim;
    const int32_t group = num_q_heads / num_kv_heads;

    int64_t T = 0, max_ctx = 0;
    for (int32_t s = 0; s < num_seqs; ++s) {
        T += q_lens[s];
        const int64_t ctx = (int64_t)num_computed[s] + q_lens[s];
        if (ctx > max_ctx) max_ctx = ctx;
    }
    /* per-token sequence index, local index, and offsets of the sequence's
     * first new token and first cached-context row */
    int32_t *tok_seq = (int32_t *)malloc(sizeof(int32_t) * (size_t)(T > 0 ? T : 1));
    int64_t *seq_t0 = (int64_t *)malloc(sizeof(int64_t) * (size_t)(num_seqs + 1));
    int64_t *seq_c0 = (int64_t *)malloc(sizeof(int64_t) * (size_t)(num_seqs + 1));
    seq_t0[0] = 0;
    seq_c0[0] = 0;
    for (int32_t s = 0; s < num_seqs; ++s) {
        seq_t0[s + 1] = seq_t0[s] + q_lens[s];
        seq_c0[s + 1] = seq_c0[s] + num_computed[s];
        for (int64_t t = seq_t0[s]; t < seq_t0[s + 1]; ++t) tok_seq[t] = s;
    }

    const int64_t rows = T * num_q_heads;
#pragma omp parallel
    {
        double *z = (double *)malloc(sizeof(double) * (size_t)(max_ctx > 0 ? max_ctx : 1));
#pragma omp for schedule(dynamic, 1)
        for (int64_t r = 0; r < rows; ++r) {
            if (row_sel && !row_sel[r]) continue;
            const int64_t t = r / num_q_heads;
            const int32_t h = (int32_t)(r % num_q_heads);
            const int32_t s = tok_seq[t];
            const int64_t c = num_computed[s];
            const int64_t i = t - seq_t0[s];
            const int64_t p = c + i;                 /* query position */
            const int32_t j = h / group;             /* its KV head */
            const double *qrow = q + (t * num_q_heads + h) * D;

            double zmax = -INFINITY;
            for (int64_t tau = 0; tau <= p; ++tau) {
                const double *krow = tau < c
                    ? kctx + ((seq_c0[s] + tau) * num_kv_heads + j) * D
                    : knew + ((seq_t0[s] + (tau - c)) * num_kv_heads + j) * D;
                double acc = 0.0;
                for (int64_t d = 0; d < D; ++d) acc += qrow[d] * krow[d];
                z[tau] = scale * acc;
                if (z[tau] > zmax) zmax = z[tau];
            }
            double denom = 0.0;
            for (int64_t tau = 0; tau <= p; ++tau) {
                z[tau] = exp(z[tau] - zmax);
                denom += z[tau];
            }
            double *orow = out + (t * num_q_heads + h) * D;
            for (int64_t d = 0; d < D; ++d) orow[d] = 0.0;
            for (int64_t tau = 0; tau <= p; ++tau) {
                const double *vrow = tau < c
                    ? vctx + ((seq_c0[s] + tau) * num_kv_heads + j) * D
                    : vnew + ((seq_t0[s] + (tau - c)) * num_kv_heads + j) * D;
                const double w = z[tau] / denom;
                for (int64_t d = 0; d < D; ++d) orow[d] += w * vrow[d];
            }
        }
        free(z);
    }
    free(tok_seq);
    free(seq_t0);
    free(seq_c0);
}

/*
 * Block copy: for each pair and each layer, block src_ids[i] of the source
 * pools is copied to block dst_ids[i] of the destination pools, K and V
 * (copy-on-write and swap move whole blocks; PageServe "04 Preemption",
 * tinyserve README "How it works"). block_bytes is one layer's block of one
 * pool: block_size * Hkv * D * elt.
 */
void oracle_copy_blocks(const uint8_t *src_k, const uint8_t *src_v, uint8_t *dst_k, uint8_t *dst_v,
                        int32_t num_layers, int32_t src_blocks, int32_t dst_blocks,
                        int64_t block_bytes, const int32_t *src_ids, const int32_t *dst_ids,
                        int32_t num_pairs)
{
    for (int32_t i = 0; i < num_pairs; ++i) {
        for (int32_t l = 0; l < num_layers; ++l) {
            const int64_t so = ((int64_t)l * src_blocks + src_ids[i]) * block_bytes;
            const int64_t d0 = ((int64_t)l * dst_blocks + dst_ids[i]) * block_bytes;
            memcpy(dst_k + d0, src_k + so, (size_t)block_bytes);
            memcpy(dst_v + d0, src_v + so, (size_t)block_bytes);
        }
    }
}

/*
 * Rotary position embedding of T rows of H heads each ([T, H, D], fp64):
 * row t is at position positions[t]. For each head and j in [0, D/2),
 * with a = positions[t] * theta^(-2j/D):
 *   out[j]       = x[j] cos a - x[j + D/2] sin a
 *   out[j + D/2] = x[j + D/2] cos a + x[j] sin a
 * i.e. the complex number x[j] + i x[j + D/2] multiplied by e^{ia}.
 * out may equal x.
 */
void oracle_rope(const double *x, int64_t T, int32_t H, int32_t D, const int32_t *positions,
                 double theta, double *out)
{
    const int32_t half = D / 2;
    for (int64_t t = 0; t < T; ++t) {
        for (int32_t j = 0; j < half; ++j) {
            const double a = (double)positions[t] * pow(theta, -2.0 * j / D);
            const double c = cos(a), s = sin(a);
            for (int32_t h = 0; h < H; ++h) {
                const double *xr = x + (t * H + h) * D;
                double *orow = out + (t * H + h) * D;
                const double x1 = xr[j], x2 = xr[j + half];
                orow[j] = x1 * c - x2 * s;
                orow[j + half] = x2 * c + x1 * s;
            }
        }
    }
}

/*
 * One categorical draw by inverse CDF. Weights are taken at fixed point:
 * w_int[t] = floor(clamp(w[t], 0, 1) * 2^40) (NaN counts as 0), so the
 * running sums are exact integers and do not depend on summation order.
 * With total = sum_t w_int[t] and v53 = floor(clamp(v, 0, 1 - 2^-53) * 2^53),
 * the draw is the smallest t whose running sum exceeds
 * floor(v53 * total / 2^53). Returns -1 when total is 0.
 */
static uint64_t fixed_weight(double w)
{
    if (!(w > 0.0)) return 0;
    if (w > 1.0) w = 1.0;
    return (uint64_t)(w * 1099511627776.0); /* 2^40 */
}

static uint64_t uniform53(double v)
{
    if (!(v > 0.0)) return 0;
    const uint64_t top = ((uint64_t)1 << 53) - 1;
    if (v >= 1.0) return top;
    const uint64_t x = (uint64_t)(v * 9007199254740992.0); /* 2^53 */
    return x > top ? top : x;
}

static int32_t categorical_draw(const double *w, int32_t n, double v)
{
    uint64_t total = 0;
    for (int32_t t = 0; t < n; ++t) total += fixed_weight(w[t]);
    if (total == 0) return -1;
    const uint64_t target = (uint64_t)(((unsigned __int128)uniform53(v) * total) >> 53);
    uint64_t run = 0;
    for (int32_t t = 0; t < n; ++t) {
        run += fixed_weight(w[t]);
        if (run > target) return t;
    }
    return -1; /* unreachable: target < total */
}

/*
 * Rejection-sampling verification of a batch of speculative rounds.
 *
 * Sequence s proposed k_s = draft_start[s + 1] - draft_start[s] drafts
 * d_0..d_{k_s - 1} (draft_tokens[draft_start[s] + i]); q_i
 * (draft_probs row draft_start[s] + i) is the distribution d_i was drawn
 * from and p_i (target_probs row draft_start[s] + s + i) the target's
 * distribution at the same position; p_{k_s} is the target's distribution
 * after the last draft. Rows are vocab entries long.
 *
 * For i = 0, 1, ...: d_i is kept when accept_u[draft_start[s] + i] * q_i(d_i)
 * < p_i(d_i) (probability min(1, p_i(d_i) / q_i(d_i)) for a uniform in
 * [0, 1)). At the first rejection the next token is drawn with sample_u[s]
 * from max(p_i - q_i, 0) (elementwise, fp64), or from p_i if that residual
 * has no mass at the draw's resolution; if no draft is rejected it is
 * drawn from p_{k_s}. Outputs: num_accepted[s] (drafts kept) and
 * next_token[s] (-1 if the distribution drawn from has no mass). A
 * sequence with k_s < 0 or a draft token outside [0, vocab) gets -1 in
 * both outputs.
 */
void oracle_spec_verify(const float *target_probs, const float *draft_probs,
                        const int32_t *draft_tokens, const int32_t *draft_start,
                        const double *accept_u, const double *sample_u,
                        int32_t num_seqs, int32_t vocab,
                        int32_t *num_accepted, int32_t *next_token)
{
    double *w = (double *)malloc(sizeof(double) * (size_t)(vocab > 0 ? vocab : 1));
    for (int32_t s = 0; s < num_seqs; ++s) {
        const int64_t d0 = draft_start[s];
        const int32_t k = draft_start[s + 1] - draft_start[s];
        int bad = k < 0;
        for (int32_t i = 0; !bad && i < k; ++i)
            bad = draft_tokens[d0 + i] < 0 || draft_tokens[d0 + i] >= vocab;
        if (bad) {
            num_accepted[s] = -1;
            next_token[s] = -1;
            continue;
        }
        int32_t i = 0;
        for (; i < k; ++i) {
            const int32_t d = draft_tokens[d0 + i];
            const double p = target_probs[(d0 + s + i) * vocab + d];
            const double q = draft_probs[(d0 + i) * vocab + d];
            if (!(accept_u[d0 + i] * q < p)) break; /* rejected */
        }
        num_accepted[s] = i;
        const float *prow = target_probs + (d0 + s + i) * vocab;
        int32_t tok = -1;
        if (i < k) {
            const float *qrow = draft_probs + (d0 + i) * vocab;
            for (int32_t t = 0; t < vocab; ++t) {
                const double r = (double)prow[t] - (double)qrow[t];
                w[t] = r > 0.0 ? r : 0.0;
            }
            tok = categorical_draw(w, vocab, sample_u[s]);
        }
        if (tok < 0) {
            for (int32_t t = 0; t < vocab; ++t) w[t] = prow[t];
            tok = categorical_draw(w, vocab, sample_u[s]);
        }
        next_token[s] = tok;
    }
    free(w);
}

/* Threads the OpenMP runtime will use for oracle_attention. */
int32_t oracle_num_threads(void)
{
#ifdef _OPENMP
    extern int omp_get_max_threads(void);
    return (int32_t)omp_get_max_threads();
#else
    return 1;
#endif
}
