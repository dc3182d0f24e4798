// C ABI glue: error reporting, status strings, the scatter entry points
// (plain and with rotary embedding) and the block copy.

#include <cmath>
#include <cstdarg>
#include <cstdio>

#include "ps_internal.h"

namespace {
thread_local char g_err[512] = "";
}

ps_status ps_fail(ps_status st, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return st;
}

extern "C" const char *ps_last_error_message(void) { return g_err; }

extern "C" const char *ps_status_string(ps_status status) {
    switch (status) {
        case PS_OK: return "ok";
        case PS_ERR_INVALID_ARGUMENT: return "invalid argument";
        case PS_ERR_UNSUPPORTED: return "unsupported";
        case PS_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
        case PS_ERR_HIP: return "HIP runtime error";
        case PS_ERR_HOST_MEMORY: return "host memory exhausted";
        default: return "unknown status";
    }
}

extern "C" int32_t ps_abi_version(void) { return PS_ABI_VERSION; }

// Checks shared by the calls that write one layer of the pool.
static ps_status check_cache_pool(const ps_pool *pool) {
    if (!pool) return ps_fail(PS_ERR_INVALID_ARGUMENT, "pool is NULL");
    if (pool->block_size != PS_BLOCK)
        return ps_fail(PS_ERR_UNSUPPORTED, "block_size %d (only 16 is supported)", pool->block_size);
    if (pool->head_dim != 64 && pool->head_dim != 128)
        return ps_fail(PS_ERR_UNSUPPORTED, "head_dim %d (64 or 128 supported)", pool->head_dim);
    if (pool->dtype != PS_F32 && pool->dtype != PS_F16 && pool->dtype != PS_BF16)
        return ps_fail(PS_ERR_UNSUPPORTED, "dtype %d", pool->dtype);
    if (pool->num_kv_heads < 1 || pool->num_layers < 1 || pool->num_blocks < 1)
        return ps_fail(PS_ERR_INVALID_ARGUMENT, "pool needs num_kv_heads, num_layers, num_blocks >= 1");
    if (pool->layer < 0 || pool->layer >= pool->num_layers)
        return ps_fail(PS_ERR_INVALID_ARGUMENT, "layer %d outside [0, %d)", pool->layer, pool->num_layers);
    if ((int64_t)pool->num_blocks * PS_BLOCK > INT32_MAX)
        return ps_fail(PS_ERR_UNSUPPORTED, "num_blocks %d: slots exceed int32", pool->num_blocks);
    if (ps_block_bytes(pool) > INT32_MAX)
        return ps_fail(PS_ERR_UNSUPPORTED, "num_kv_heads %d: a pool block exceeds INT32_MAX bytes", pool->num_kv_heads);
    return PS_OK;
}

extern "C" ps_status ps_reshape_and_cache(const void *k, const void *v, const int32_t *slot_mapping,
                                          int32_t num_tokens, const ps_pool *pool, void *stream) {
    const ps_status st = check_cache_pool(pool);
    if (st != PS_OK) return st;
    if (num_tokens < 0) return ps_fail(PS_ERR_INVALID_ARGUMENT, "num_tokens < 0");
    if (num_tokens == 0) return PS_OK;
    if (!k || !v || !slot_mapping || !pool->k || !pool->v)
        return ps_fail(PS_ERR_INVALID_ARGUMENT, "a device pointer is NULL");
    const int err = ps_launch_scatter(k, v, slot_mapping, num_tokens, pool, stream);
    if (err != 0) return ps_fail(PS_ERR_HIP, "scatter launch: %s", ps_hip_error_string(err));
    return PS_OK;
}

extern "C" ps_status ps_rope_reshape_and_cache(const void *q, void *q_out, const void *k, const void *v,
                                               const int32_t *positions, const int32_t *slot_mapping,
                                               int32_t num_tokens, int32_t num_q_heads, double rope_theta,
                                               const ps_pool *pool, void *stream) {
    const ps_status st = check_cache_pool(pool);
    if (st != PS_OK) return st;
    if (num_tokens < 0) return ps_fail(PS_ERR_INVALID_ARGUMENT, "num_tokens < 0");
    if (num_q_heads < 0) return ps_fail(PS_ERR_INVALID_ARGUMENT, "num_q_heads < 0");
    if (!(rope_theta > 0.0) || !std::isfinite(rope_theta))
        return ps_fail(PS_ERR_INVALID_ARGUMENT, "rope_theta must be finite and > 0");
    if (num_tokens == 0) return PS_OK;
    if (!k || !v || !positions || !slot_mapping || !pool->k || !pool->v)
        return ps_fail(PS_ERR_INVALID_ARGUMENT, "a device pointer is NULL");
    const int D = pool->head_dim;
    const int64_t elt = pool->dtype == PS_F32 ? 4 : 2;
    if (num_q_heads > 0) {
        if (!q || !q_out) return ps_fail(PS_ERR_INVALID_ARGUMENT, "q or q_out is NULL");
        const uintptr_t n = (uintptr_t)((int64_t)num_tokens * num_q_heads * D * elt);
        const uintptr_t a0 = (uintptr_t)q, b0 = (uintptr_t)q_out;
        if (a0 != b0 && a0 < b0 + n && b0 < a0 + n)
            return ps_fail(PS_ERR_INVALID_ARGUMENT, "q and q_out overlap without being equal");
    }
    ps_rope_launch a{};
    a.q = q;
    a.q_out = q_out;
    a.k = k;
    a.v = v;
    a.positions = positions;
    a.slots = slot_mapping;
    const int64_t layer_bytes = (int64_t)pool->num_blocks * PS_BLOCK * pool->num_kv_heads * D * elt;
    a.pool_k = static_cast<uint8_t *>(pool->k) + pool->layer * layer_bytes;
    a.pool_v = static_cast<uint8_t *>(pool->v) + pool->layer * layer_bytes;
    a.num_tokens = num_tokens;
    a.num_q_heads = num_q_heads;
    a.num_kv_heads = pool->num_kv_heads;
    a.head_dim = D;
    a.dtype = pool->dtype;
    a.num_slots = pool->num_blocks * PS_BLOCK;
    for (int j = 0; j < D / 2; ++j) a.inv_freq[j] = std::pow(rope_theta, -2.0 * j / D);
    const int err = ps_launch_rope_cache(a, stream);
    if (err != 0) return ps_fail(PS_ERR_HIP, "rope launch: %s", ps_hip_error_string(err));
    return PS_OK;
}

static ps_status check_pool_layout(const ps_pool *p, const char *what) {
    if (!p) return ps_fail(PS_ERR_INVALID_ARGUMENT, "%s pool is NULL", what);
    if (p->block_size != PS_BLOCK)
        return ps_fail(PS_ERR_UNSUPPORTED, "%s pool: block_size %d (only 16 is supported)", what, p->block_size);
    if (p->head_dim != 64 && p->head_dim != 128)
        return ps_fail(PS_ERR_UNSUPPORTED, "%s pool: head_dim %d (64 or 128 supported)", what, p->head_dim);
    if (p->dtype != PS_F32 && p->dtype != PS_F16 && p->dtype != PS_BF16)
        return ps_fail(PS_ERR_UNSUPPORTED, "%s pool: dtype %d", what, p->dtype);
    if (p->num_kv_heads < 1 || p->num_layers < 1 || p->num_blocks < 1)
        return ps_fail(PS_ERR_INVALID_ARGUMENT, "%s pool needs num_kv_heads, num_layers, num_blocks >= 1", what);
    if (ps_block_bytes(p) > INT32_MAX)
        return ps_fail(PS_ERR_UNSUPPORTED, "%s pool: num_kv_heads %d: a block exceeds INT32_MAX bytes", what,
                       p->num_kv_heads);
    return PS_OK;
}

extern "C" ps_status ps_copy_blocks(const ps_pool *src, const ps_pool *dst, const int32_t *src_blocks,
                                    const int32_t *dst_blocks, int32_t num_pairs, void *stream) {
    ps_status st = check_pool_layout(src, "source");
    if (st != PS_OK) return st;
    if ((st = check_pool_layout(dst, "destination")) != PS_OK) return st;
    if (src->num_layers != dst->num_layers || src->num_kv_heads != dst->num_kv_heads ||
        src->head_dim != dst->head_dim || src->dtype != dst->dtype)
        return ps_fail(PS_ERR_INVALID_ARGUMENT, "source and destination pools differ in layout");
    if (num_pairs < 0) return ps_fail(PS_ERR_INVALID_ARGUMENT, "num_pairs < 0");
    if (num_pairs == 0) return PS_OK;
    if (!src_blocks || !dst_blocks || !src->k || !src->v || !dst->k || !dst->v)
        return ps_fail(PS_ERR_INVALID_ARGUMENT, "a device pointer is NULL");
    if ((int64_t)num_pairs * src->num_layers > 0x7fffffff)
        return ps_fail(PS_ERR_UNSUPPORTED, "too many block copies in one call");
    const int err = ps_launch_copy_blocks(src, dst, src_blocks, dst_blocks, num_pairs, stream);
    if (err != 0) return ps_fail(PS_ERR_HIP, "copy launch: %s", ps_hip_error_string(err));
    return PS_OK;
}

extern "C" size_t ps_spec_verify_workspace_bytes(int32_t num_seqs, int32_t vocab_size) {
    if (num_seqs <= 0 || vocab_size <= 0) return 0;
    return ps_spec_workspace(num_seqs, vocab_size);
}

extern "C" ps_status ps_spec_verify(const float *target_probs, const float *draft_probs,
                                    const int32_t *draft_tokens, const int32_t *draft_start,
                                    const double *accept_uniforms, const double *sample_uniforms,
                                    int32_t num_seqs, int32_t total_drafts, int32_t vocab_size,
                                    int32_t *num_accepted, int32_t *next_token, void *workspace,
                                    size_t workspace_bytes, void *stream) {
    if (num_seqs < 0) return ps_fail(PS_ERR_INVALID_ARGUMENT, "num_seqs < 0");
    if (total_drafts < 0) return ps_fail(PS_ERR_INVALID_ARGUMENT, "total_drafts < 0");
    if (vocab_size < 1 || vocab_size > PS_SPEC_MAX_VOCAB)
        return ps_fail(PS_ERR_UNSUPPORTED, "vocab_size %d outside [1, %d]", vocab_size, PS_SPEC_MAX_VOCAB);
    if (num_seqs == 0) return PS_OK;
    if (!target_probs || !draft_start || !sample_uniforms || !num_accepted || !next_token || !workspace)
        return ps_fail(PS_ERR_INVALID_ARGUMENT, "a device pointer is NULL");
    if (total_drafts > 0 && (!draft_probs || !draft_tokens || !accept_uniforms))
        return ps_fail(PS_ERR_INVALID_ARGUMENT, "draft_probs, draft_tokens or accept_uniforms is NULL");
    const size_t need = ps_spec_workspace(num_seqs, vocab_size);
    if (workspace_bytes < need)
        return ps_fail(PS_ERR_WORKSPACE_TOO_SMALL, "workspace holds %zu bytes, the call needs %zu",
                       workspace_bytes, need);
    if (((uintptr_t)workspace & 7) != 0)
        return ps_fail(PS_ERR_INVALID_ARGUMENT, "workspace is not 8-byte aligned");
    ps_spec_launch a{};
    a.target = target_probs;
    a.draft = draft_probs;
    a.tokens = draft_tokens;
    a.starts = draft_start;
    a.accept_u = accept_uniforms;
    a.sample_u = sample_uniforms;
    a.num_accepted = num_accepted;
    a.next_token = next_token;
    a.chunk_sums = static_cast<uint64_t *>(workspace);
    a.decisions = reinterpret_cast<int32_t *>(static_cast<uint8_t *>(workspace) +
                                              ps_spec_sums_bytes(num_seqs, vocab_size));
    a.num_seqs = num_seqs;
    a.total_drafts = total_drafts;
    a.vocab = vocab_size;
    a.n_chunks = (vocab_size + PS_SPEC_CHUNK - 1) / PS_SPEC_CHUNK;
    // 16-byte loads when every row starts 16-byte aligned
    const bool vec = vocab_size % 4 == 0 && ((uintptr_t)target_probs & 15) == 0 &&
                     (total_drafts == 0 || ((uintptr_t)draft_probs & 15) == 0);
    const int err = ps_launch_spec_verify(a, vec, stream);
    if (err != 0) return ps_fail(PS_ERR_HIP, "verify launch: %s", ps_hip_error_string(err));
    return PS_OK;
}
