/*
 * ps.h — C ABI of a packed paged-attention step for AMD Instinct MI355X
 * (gfx950).
 *
 * One scheduler step packs every scheduled token of every sequence into a
 * single ragged [1, T] batch: prefill chunks, single decode tokens and
 * speculative-verify rows (1 + k tokens) side by side (PageServe, "01
 * Scheduler loop", Pack; "06 Development history", phase 8). The step
 *   1. scatters this step's new K/V rows into a pre-allocated block pool
 *      at slot = block_table[pos / 16] * 16 + pos % 16 (PageServe, "03
 *      Paged KV cache", attention_wrapper code box), then
 *   2. runs causal grouped-query attention for every packed query token
 *      over its own sequence's context, reading K/V through the
 *      sequence's block table (PageServe "03 Paged KV cache"; tinyserve
 *      README "How it works": stepped causal mask over 1 + k rows).
 *
 * Conventions shared by every call:
 *  - Device pointers are caller-owned (e.g. torch tensors); the library
 *    never allocates or frees device memory. Host arrays are read during
 *    the call only.
 *  - A "stream" is a hipStream_t passed as void* (NULL = default stream).
 *    Device work is enqueued asynchronously on it; the library never
 *    synchronises. ps_paged_attention must be enqueued after
 *    ps_reshape_and_cache of the same step on the same stream: attention
 *    reads this step's K/V from the pool.
 *  - Every call returns a ps_status. Argument errors are detected on the
 *    host and returned before anything is enqueued. A launch failure
 *    returns PS_ERR_HIP. ps_last_error_message() gives a readable reason
 *    for the calling thread's last failure.
 *  - No C++ exception crosses this boundary. Calls are reentrant; the
 *    only global state is the per-thread error message.
 *  - Supported: block_size 16; head_dim 64 or 128; fp32, fp16, bf16
 *    storage with fp32 accumulation; num_q_heads a multiple of
 *    num_kv_heads.
 *
 * Around the step: ps_rope_reshape_and_cache (rotary embedding fused with
 * the scatter, for K that arrives unrotated), ps_copy_blocks (copy-on-write
 * and swap between device and pinned host pools) and ps_spec_verify
 * (rejection sampling over the verify rows' distributions).
 */
#ifndef PS_H
#define PS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PS_ABI_VERSION 5

typedef int32_t ps_status;
enum {
    PS_OK = 0,
    PS_ERR_INVALID_ARGUMENT = 1,    /* bad pointer, size, length or metadata */
    PS_ERR_UNSUPPORTED = 2,         /* valid but not built: dtype, head_dim, block_size */
    PS_ERR_WORKSPACE_TOO_SMALL = 3, /* workspace_bytes below ps_plan_sizes' figure */
    PS_ERR_HIP = 4,                 /* the HIP runtime reported an error */
    PS_ERR_HOST_MEMORY = 5          /* host allocation failed */
};

typedef enum { PS_F32 = 0, PS_F16 = 1, PS_BF16 = 2 } ps_dtype;

/*
 * The KV pool: two device arrays (K and V), each laid out
 * [num_layers, num_blocks, block_size, num_kv_heads, head_dim] and
 * contiguous (PageServe "06 Development history", phase 7: one pool
 * [layers, blocks, 16, H, D]; tinyserve README "How it works": K and V in
 * two slabs, H = number of KV heads). Every layer addresses the same block
 * ids; `layer` picks the layer a call works on. Limits (else
 * PS_ERR_UNSUPPORTED): num_blocks * 16 slots and the bytes of one block
 * (16 * num_kv_heads * head_dim elements) each at most INT32_MAX; the
 * arrays themselves may be any size (offsets are 64-bit).
 */
typedef struct {
    void *k;
    void *v;
    int32_t num_layers;
    int32_t num_blocks;
    int32_t block_size;   /* must be 16 */
    int32_t num_kv_heads;
    int32_t head_dim;     /* 64 or 128 */
    int32_t dtype;        /* ps_dtype of K, V, Q and the output */
    int32_t layer;        /* 0 <= layer < num_layers */
} ps_pool;

/*
 * Opaque host object made by ps_plan_step: the step's metadata (the packed
 * batch's index arrays) plus the kernels' work lists. One plan serves every
 * layer of the step.
 */
typedef struct ps_plan ps_plan;

/*
 * ps_plan_step flags. The low two bits choose the attention kernel of each
 * sequence; the others are independent switches.
 */
enum {
    PS_PLAN_DEFAULT = 0,        /* few query rows per KV head (g * n_s <= 32): split-K decode kernel; else prefill kernel */
    PS_PLAN_ALL_DECODE = 1,     /* every sequence through the decode/verify kernel (g * n_s <= 32 required per work item row range) */
    PS_PLAN_ALL_PREFILL = 2,    /* every sequence through the prefill-chunk kernel */
    /* Shared-prefix pass (opt-in). Decode sequences whose tables open with
     * the same physical blocks (blocks shared by reference: PageServe "03
     * Paged KV cache"; tinyserve README "How it works", copy-on-write)
     * form groups; attention over a group's common blocks then runs once,
     * on rows gathered from every member, and merges with each member's
     * own keys like a key split. The result is the same softmax summed in
     * another order, so with this flag the output bits depend on which
     * blocks are physically shared. Without it (the default) a step gives
     * the same bits whether its prefix blocks are shared or private
     * copies. Applies with PS_PLAN_DEFAULT routing only. */
    PS_PLAN_SHARED_PREFIX = 4,
    /* Decode and prefill items in two launches (decode kernel, then
     * prefill kernel) instead of one launch that runs both kinds. Same
     * results bit for bit; a measurement switch. */
    PS_PLAN_SEPARATE_LAUNCHES = 8,
    /* Graph-replayable shape: the metadata layout, the launch grids and
     * every kernel argument depend only on the options' capacities (and
     * the geometry), not on this step's lengths. Steps planned with the
     * same options, uploaded into the same metadata buffer, can replay one
     * captured graph of ps_step / ps_paged_attention. Work lists are
     * padded with idle items that exit at once. Every sequence must take
     * the decode kernel (no PS_PLAN_ALL_PREFILL, no shared-prefix pass). */
    PS_PLAN_FIXED_SHAPE = 16
};

/*
 * Tuning and capacity options of ps_plan_step (NULL = all zero = chosen by
 * the planner). Every choice is recorded in ps_plan_info; nothing outside
 * the arguments (no environment variable) changes a plan.
 */
typedef struct {
    int32_t decode_split_keys;   /* keys per decode work item: 0 = planner's choice, else a
                                    multiple of 16 in [16, 16384] */
    int32_t prefill_split_keys;  /* keys per prefill work item: 0 = planner's choice, else a
                                    multiple of 64 in [64, 16384] */
    int32_t decode_waves;        /* waves per decode workgroup: 0 = planner's choice, 4 or 8
                                    (16 for head_dim 64 16-bit steps of one row tile) */
    int32_t prefix_min_seqs;     /* PS_PLAN_SHARED_PREFIX: members a group needs (0 = 8; >= 2) */
    int32_t prefix_min_keys;     /* ... tokens each member shares with the group's first
                                    (0 = 256; >= 16) */
    int32_t prefix_slice_keys;   /* ... keys per prefix work item: 0 = planner's choice, else a
                                    multiple of 64 in [64, 16384] */
    /* PS_PLAN_FIXED_SHAPE capacities (ignored otherwise): */
    int32_t max_seqs;            /* >= num_seqs */
    int32_t max_tokens;          /* >= num_tokens */
    int32_t max_query_len;       /* >= every q_lens[s]; (num_q_heads / num_kv_heads) *
                                    max_query_len <= 32 */
    int32_t max_decode_items;    /* 0 = max_seqs * num_kv_heads */
    int32_t max_merge_items;     /* 0: no key splits allowed */
    int32_t max_workspace_rows;  /* split-K partial rows (0 with no splits) */
    int32_t decode_walk_rotation; /* each decode item starts its walk over its key tiles at an
                                    item-dependent tile (helps when many items read the same
                                    shared blocks): 0 = planner's choice (on from 512 decode
                                    items up, off for PS_PLAN_FIXED_SHAPE), 1 = on, 2 = off.
                                    A function of the item and the step's logical shape, never
                                    of physical sharing; it changes the summation order */
    int32_t decode_stream_kv;    /* cache policy of the decode kernel's K/V loads: 0 = planner's
                                    choice, 1 = non-temporal (streamed), 2 = cached. Results are the
                                    same either way; the planner streams when no physical block is
                                    read by two sequences of the step and the decode sequences' K/V
                                    exceed 256 MiB (MI355X's last-level cache: none of it would
                                    still be cached at its next use), never for PS_PLAN_FIXED_SHAPE */
    int32_t reserved[2];         /* must be 0 */
} ps_plan_options;

/*
 * Build the packed step's metadata on the host (the Pack stage of
 * PageServe "01 Scheduler loop").
 *
 *   q_lens[num_seqs]               n_s >= 1: new tokens of sequence s this
 *                                  step; they occupy rows
 *                                  sum_{s'<s} n_s' .. +n_s-1 of the packed
 *                                  batch, in sequence order
 *   num_computed_tokens[num_seqs]  c_s >= 0: tokens of s whose K/V are
 *                                  already in the pool (PageServe "01
 *                                  Scheduler loop", System architecture).
 *                                  Token i of s has position c_s + i.
 *   block_tables[num_seqs * block_table_stride]
 *                                  row s lists the physical blocks of s in
 *                                  logical order; entries past
 *                                  ceil((c_s + n_s) / 16) are ignored
 *   num_q_heads                    query heads (a multiple of the pool's
 *                                  num_kv_heads; head h reads KV head
 *                                  h / (num_q_heads / num_kv_heads))
 *   pool                           geometry and dtype (pointers unused here)
 *   flags                          PS_PLAN_* (kernel choice | switches)
 *   options                        NULL or tuning / capacity options
 *
 * Validates: lengths, table width, block ids in [0, num_blocks), no block
 * twice in one table, and no new token written into a block that more than
 * one table references (shared blocks are read-only; tinyserve README "How
 * it works": copy-on-write precedes any write into a shared block). Work
 * is proportional to the table entries the step covers, not to the pool.
 * On success *out_plan owns host memory until ps_plan_destroy. num_seqs ==
 * 0 gives an empty plan.
 */
ps_status ps_plan_step(const int32_t *q_lens, const int32_t *num_computed_tokens,
                       int32_t num_seqs, const int32_t *block_tables,
                       int32_t block_table_stride, int32_t num_q_heads,
                       const ps_pool *pool, uint32_t flags, const ps_plan_options *options,
                       ps_plan **out_plan);

/*
 * Device memory the caller must provide: metadata_bytes for
 * ps_plan_upload (256-byte aligned), workspace_bytes for
 * ps_paged_attention's split-K partial results (may be 0).
 */
ps_status ps_plan_sizes(const ps_plan *plan, size_t *metadata_bytes, size_t *workspace_bytes);

/*
 * Copy the plan's metadata into caller device memory metadata_dev
 * (metadata_bytes long, 256-byte aligned) on `stream`. The plan remembers
 * metadata_dev; that memory must stay valid, and unchanged, while the plan
 * is used. The host copy stays owned by the plan, so the plan must outlive
 * the copy (synchronise the stream before ps_plan_destroy). With
 * PS_PLAN_FIXED_SHAPE, the next step's plan may be uploaded into the same
 * buffer once the previous step's work on it is done (same stream).
 */
ps_status ps_plan_upload(ps_plan *plan, void *metadata_dev, size_t metadata_bytes, void *stream);

/* Device addresses of the uploaded index arrays (valid after ps_plan_upload). */
typedef struct {
    const int32_t *slot_mapping;        /* [T]   flat slot of each packed token */
    const int32_t *block_tables;        /* [S, block_table_stride] */
    int32_t block_table_stride;
    const int32_t *query_start_loc;     /* [S + 1] exclusive prefix sum of q_lens */
    const int32_t *num_computed_tokens; /* [S] */
    const int32_t *context_lens;        /* [S]   c_s + n_s */
    const int32_t *positions;           /* [T]   position c_s + i of each packed token */
} ps_step_arrays;

ps_status ps_plan_device_arrays(const ps_plan *plan, ps_step_arrays *arrays);

/* Host copies of the same arrays (valid until ps_plan_destroy). */
ps_status ps_plan_host_arrays(const ps_plan *plan, ps_step_arrays *arrays);

/*
 * What the step costs by definition (algorithmic work, not what a kernel
 * happens to move), and what the planner chose. KV bytes count each
 * visible (token, KV head) row of K and V once per sequence, shared by the
 * query heads of its group; the "unique" figure counts each physical block
 * once however many tables share it. flops = 4 * head_dim per (query row,
 * visible key): one multiply-add each for q.k and for p.v.
 */
typedef struct {
    int32_t num_seqs, num_tokens, num_q_heads, num_kv_heads, head_dim, dtype;
    int32_t decode_seqs, prefill_seqs;          /* sequences per attention kernel */
    int32_t decode_items, prefill_items, merge_items;  /* launched (fixed shape: capacities) */
    int32_t decode_row_tiles;                   /* 16-row MFMA tiles per decode work item */
    int64_t kv_bytes_decode, kv_bytes_prefill;  /* logical K+V bytes read */
    int64_t kv_bytes_unique;                    /* distinct physical K+V bytes read */
    int64_t q_bytes, out_bytes, scatter_bytes, table_bytes;
    double flops_decode, flops_prefill;
    /* Shared prefixes (PS_PLAN_SHARED_PREFIX): decode sequences whose
     * tables open with the same blocks form groups; attention over a
     * group's prefix runs once, in prefix_items prefill-kernel items
     * (counted in prefill_items) whose rows come from every member, and
     * merges with each member's own keys like a key split. step_fused:
     * ps_step runs the scatter inside the attention launch. */
    int32_t prefix_groups, prefix_items, step_fused, flags;
    /* the choices the planner made (options resolved) */
    int32_t decode_split_keys, prefill_split_keys, decode_waves, mixed_launch;
    int32_t active_decode_items, active_merge_items;  /* items that do work (fixed shape pads) */
    int32_t decode_walk_rotation;               /* 1: decode items rotate their walks */
    int32_t decode_stream_kv;                   /* 1: decode K/V loads are non-temporal */
    int64_t workspace_rows;                     /* split-K partial rows */
    double plan_us;                             /* host time ps_plan_step took */
} ps_plan_info;

ps_status ps_plan_get_info(const ps_plan *plan, ps_plan_info *info);

/*
 * Which attention kernel serves each sequence:
 * kinds[s] = 0 decode / verify kernel, 1 prefill-chunk kernel, 2 decode
 * kernel for the keys past a shared prefix whose attention runs in
 * prefill-kernel items (PS_PLAN_SHARED_PREFIX). kinds holds num_seqs
 * entries (host memory).
 */
ps_status ps_plan_sequence_kernels(const ps_plan *plan, int32_t *kinds, int32_t num_seqs);

void ps_plan_destroy(ps_plan *plan);

/*
 * Scatter this step's K/V into the pool (PageServe "01 Scheduler loop",
 * Execute: writes K/V into the pool; "03 Paged KV cache": scatters new K/V
 * into those slots). For t in [0, num_tokens):
 *   pool.k[layer, slot/16, slot%16, :, :] = k[t, :, :]   (same for v)
 * with slot = slot_mapping[t]. A byte copy.
 *
 *   k, v          device [num_tokens, num_kv_heads, head_dim], pool dtype
 *   slot_mapping  device [num_tokens], distinct slots in [0, num_blocks*16);
 *                 an entry outside that range is skipped
 */
ps_status ps_reshape_and_cache(const void *k, const void *v, const int32_t *slot_mapping,
                               int32_t num_tokens, const ps_pool *pool, void *stream);

/*
 * Causal GQA attention of the packed step over the pool (PageServe "03
 * Paged KV cache": attends through the table; tinyserve README
 * "Highlights": grouped-query attention, "How it works": stepped causal
 * mask). For packed token t = query_start_loc[s] + i of sequence s
 * (position p = num_computed_tokens[s] + i) and query head h, with KV head
 * j = h / (num_q_heads / num_kv_heads):
 *   out[t, h, :] = sum_{tau <= p} softmax_tau(scale * q[t, h, :] . K_s[tau, j, :]) V_s[tau, j, :]
 * where K_s[tau] is the pool row at block_tables[s][tau / 16], tau % 16.
 * Softmax and accumulation run in fp32; the output is rounded to the pool
 * dtype (round to nearest even).
 *
 * The plan fixes how the work is cut (which sequence, KV head, query rows
 * and key range each workgroup covers); the kernels read everything about
 * a sequence from the call's own device arrays: its first packed row from
 * query_start_loc[s], its offset c_s from num_computed_tokens[s], its key
 * count from context_lens[s] (keys at or past it are never read) and every
 * block id from block_tables[s]. They need not be the arrays
 * ps_plan_device_arrays returns (any caller-owned copies), but they must
 * hold the values ps_plan_step derived or was given for this step, with
 * block ids that may differ (a table pointing at other blocks holding the
 * same tokens gives the same result). If they hold other values the result
 * is undefined, but every access stays inside the buffers the call's
 * sizes describe: a block id outside [0, num_blocks) reads block
 * num_blocks - 1, a packed row outside [0, num_tokens) is clamped into it.
 *
 *   q           device [num_tokens, num_q_heads, head_dim], pool dtype
 *   block_tables          device [num_seqs, block_table_stride]
 *   query_start_loc       device [num_seqs + 1]
 *   num_computed_tokens   device [num_seqs]
 *   context_lens          device [num_seqs], c_s + n_s
 *   out         device [num_tokens, num_q_heads, head_dim], pool dtype
 *   plan        the uploaded plan of this step; num_seqs, num_tokens,
 *               num_q_heads, block_table_stride and the pool geometry must
 *               be the plan's
 *   workspace   device scratch of at least ps_plan_sizes' workspace_bytes
 *               (256-byte aligned); the call overwrites it
 */
ps_status ps_paged_attention(const void *q, const ps_pool *pool,
                             const int32_t *block_tables, int32_t block_table_stride,
                             const int32_t *query_start_loc,
                             const int32_t *num_computed_tokens,
                             const int32_t *context_lens, void *out,
                             int32_t num_seqs, int32_t num_tokens, int32_t num_q_heads,
                             float scale, const ps_plan *plan,
                             void *workspace, size_t workspace_bytes, void *stream);

/*
 * The whole step in the fewest launches: ps_reshape_and_cache followed by
 * ps_paged_attention, with the same arguments and results (pool contents
 * and output bit for bit). When the plan puts every sequence on the
 * decode / verify kernel, the scatter is fused into it: keys of this step
 * are read from k and v directly, and the work item that holds a
 * sequence's last keys writes them into their slots, so the step is one
 * attention launch (plus the split-K merge) instead of two. Otherwise the
 * scatter is launched first. Same checks and errors as the two calls.
 *
 *   k, v, slot_mapping  as for ps_reshape_and_cache
 *   the rest            as for ps_paged_attention
 */
ps_status ps_step(const void *q, const void *k, const void *v, const int32_t *slot_mapping,
                  const ps_pool *pool, const int32_t *block_tables, int32_t block_table_stride,
                  const int32_t *query_start_loc, const int32_t *num_computed_tokens,
                  const int32_t *context_lens, void *out, int32_t num_seqs, int32_t num_tokens,
                  int32_t num_q_heads, float scale, const ps_plan *plan, void *workspace,
                  size_t workspace_bytes, void *stream);

/*
 * ps_step for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation.
 * Same arguments and results as ps_step (bit for bit), without the
 * workspace: the split-K partials go to a static device array of
 * PS_STATIC_WORKSPACE_BYTES that the library holds on each GPU it runs on
 * until the process ends. A plan whose workspace (ps_plan_sizes) exceeds
 * it is refused with PS_ERR_WORKSPACE_TOO_SMALL before anything is
 * enqueued (longer key splits, ps_plan_options, shrink it). The call
 * allocates nothing; its first call on a device (which must be current)
 * looks up that device's array, so make it outside a graph capture. All
 * calls on one GPU share its array: calls that overlap in time on that GPU
 * (other streams, other threads) race on it and must be serialised by the
 * caller. Nothing needs to start zeroed: every partial is written before
 * it is read.
 */
#define PS_STATIC_WORKSPACE_BYTES ((size_t)128 << 20)

ps_status ps_step_no_alloc(const void *q, const void *k, const void *v, const int32_t *slot_mapping,
                           const ps_pool *pool, const int32_t *block_tables, int32_t block_table_stride,
                           const int32_t *query_start_loc, const int32_t *num_computed_tokens,
                           const int32_t *context_lens, void *out, int32_t num_seqs, int32_t num_tokens,
                           int32_t num_q_heads, float scale, const ps_plan *plan, void *stream);

/*
 * Copy whole blocks between two pools of the same layout (num_layers,
 * block_size, num_kv_heads, head_dim, dtype; num_blocks may differ): for
 * every pair i and every layer, block src_blocks[i] of (src->k, src->v) is
 * copied byte for byte to block dst_blocks[i] of (dst->k, dst->v). The
 * `layer` fields are ignored: a block id names storage in every layer
 * (PageServe, "06 Development history", phase 7).
 *
 * This is the data movement of copy-on-write (same pool: a shared block
 * is duplicated before a sequence writes into it; tinyserve README, "How
 * it works") and of swapping a preempted sequence's blocks out to a pinned
 * host pool and back in (PageServe, "04 Preemption"; tinyserve README,
 * "How it works"). Host pools must be pinned, device-accessible memory
 * (hipHostMalloc, torch pin_memory).
 *
 *   src_blocks, dst_blocks  device (or device-accessible) [num_pairs]; a
 *                           pair with an id outside its pool is skipped.
 *                           Destination ids must be distinct and must not
 *                           be read by another pair of the same call.
 */
ps_status ps_copy_blocks(const ps_pool *src, const ps_pool *dst, const int32_t *src_blocks,
                         const int32_t *dst_blocks, int32_t num_pairs, void *stream);

/*
 * Rotary position embedding fused with the KV scatter: the step just
 * upstream of attention in the packed forward pass (tinyserve README,
 * "Highlights": the Qwen2 forward applies rotary embeddings to a
 * flattened ragged batch; PageServe "01 Scheduler loop", Pack: explicit
 * position_ids and a slot per token). For packed token t at position
 * p = positions[t] and every head, each pair (x[j], x[j + D/2]),
 * j < D/2, is turned by the angle p * rope_theta^(-2j/D):
 *   y[j]       = x[j] cos a - x[j + D/2] sin a
 *   y[j + D/2] = x[j + D/2] cos a + x[j] sin a
 * (the Qwen2 pairing of a head's halves). Then
 *   q_out[t, h, :]                         = rotated q[t, h, :]
 *   pool.k[layer, slot/16, slot%16, j, :]  = rotated k[t, j, :]
 *   pool.v[layer, slot/16, slot%16, j, :]  = v[t, j, :]   (byte copy)
 * with slot = slot_mapping[t]. This replaces ps_reshape_and_cache for a
 * step whose K arrives unrotated.
 *
 * Angles are formed in fp64 (an exact product of the position and a
 * host-computed fp64 frequency), cos and sin in fp64, the rotation in fp32;
 * results are rounded to the pool dtype (round to nearest even).
 *
 *   q, q_out      device [num_tokens, num_q_heads, head_dim], pool dtype.
 *                 q_out may equal q (rotation in place); otherwise the two
 *                 must not overlap. Both may be NULL when num_q_heads = 0
 *                 (K rotation and scatter only).
 *   k, v          device [num_tokens, num_kv_heads, head_dim], pool dtype
 *   positions     device [num_tokens] int32 (e.g. ps_step_arrays.positions)
 *   slot_mapping  device [num_tokens], distinct slots in [0, num_blocks*16);
 *                 a token whose slot is outside that range writes nothing
 *                 to the pool (its q is still rotated)
 *   rope_theta    frequency base, finite and > 0 (Qwen2.5 uses 1e6)
 */
ps_status ps_rope_reshape_and_cache(const void *q, void *q_out, const void *k, const void *v,
                                    const int32_t *positions, const int32_t *slot_mapping,
                                    int32_t num_tokens, int32_t num_q_heads, double rope_theta,
                                    const ps_pool *pool, void *stream);

/*
 * Rejection-sampling verification of speculative drafts, for the 1 + k
 * verify rows a packed step scores (tinyserve README, "How it works",
 * Speculative decoding; PageServe "06 Development history", Next steps:
 * rejection sampling, so that sampled requests can speculate too).
 *
 * Sequence s proposed k_s = draft_start[s + 1] - draft_start[s] drafts
 * d_i = draft_tokens[draft_start[s] + i]. q_i, row draft_start[s] + i of
 * draft_probs, is the distribution d_i was drawn from; p_i, row
 * draft_start[s] + s + i of target_probs, is the target's distribution at
 * the same position (the verify row scoring the token before d_i), and
 * p_{k_s} the one after the last draft (rows per sequence: k_s + 1).
 *
 *  - Draft d_i is kept while accept_uniforms[draft_start[s] + i] * q_i(d_i)
 *    < p_i(d_i), evaluated in fp64: kept with probability
 *    min(1, p_i(d_i) / q_i(d_i)) for a uniform in [0, 1).
 *  - At the first rejection (index j) the next token is drawn with
 *    sample_uniforms[s] from max(p_j - q_j, 0) (elementwise, fp64), or
 *    from p_j when that residual has no mass at the draw's resolution;
 *    when every draft is kept (j = k_s) it is drawn from p_{k_s} (the
 *    bonus token). A zero-draft sequence is a plain sampled decode.
 *  - A draw from weights w with uniform v is the smallest t whose running
 *    sum of floor(clamp(w, 0, 1) * 2^40) exceeds
 *    floor(floor(clamp(v, 0, 1 - 2^-53) * 2^53) * total / 2^53), in exact
 *    integers, so it is independent of how the vocabulary is split; NaN
 *    weights count as 0, and weights below 2^-40 are never drawn.
 *
 * Outputs num_accepted[s] = j and next_token[s] (-1 if the row drawn from
 * has no mass). A sequence whose draft_start entries are not
 * 0 <= draft_start[s] <= draft_start[s + 1] <= total_drafts, or with a
 * draft token outside [0, vocab_size), gets -1 in both outputs; the other
 * sequences are unaffected.
 *
 *   target_probs     device fp32 [total_drafts + num_seqs, vocab_size]
 *   draft_probs      device fp32 [total_drafts, vocab_size]
 *   draft_tokens     device int32 [total_drafts]
 *   draft_start      device int32 [num_seqs + 1]
 *   accept_uniforms  device fp64 [total_drafts]
 *   sample_uniforms  device fp64 [num_seqs]
 *   num_accepted, next_token  device int32 [num_seqs], written
 *   workspace        device, 8-byte aligned, at least
 *                    ps_spec_verify_workspace_bytes(num_seqs, vocab_size)
 *                    bytes; overwritten
 * vocab_size is at most 2^23. draft_probs, draft_tokens and
 * accept_uniforms may be NULL when total_drafts is 0.
 */
size_t ps_spec_verify_workspace_bytes(int32_t num_seqs, int32_t vocab_size);

ps_status ps_spec_verify(const float *target_probs, const float *draft_probs,
                         const int32_t *draft_tokens, const int32_t *draft_start,
                         const double *accept_uniforms, const double *sample_uniforms,
                         int32_t num_seqs, int32_t total_drafts, int32_t vocab_size,
                         int32_t *num_accepted, int32_t *next_token, void *workspace,
                         size_t workspace_bytes, void *stream);

const char *ps_status_string(ps_status status);

/* Reason for the calling thread's last failed call ("" if none). */
const char *ps_last_error_message(void);

int32_t ps_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PS_H */
