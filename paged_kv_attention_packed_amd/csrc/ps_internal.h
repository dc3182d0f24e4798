// Internal structures shared by the host planner and the HIP kernels.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "ps.h"

// Rows of one attention work item are "packed rows" of one sequence and one
// KV head: row r stands for query token r / g of the sequence and query head
// kv_head * g + r % g (g = num_q_heads / num_kv_heads), so the g heads that
// read the same K/V share every K/V load.
struct ps_item {
    int32_t seq;         // sequence index; < 0: an idle item (fixed-shape padding) that exits
    int32_t kv_head;
    int32_t row_begin;   // first packed row
    int32_t row_end;     // one past the last packed row
    int32_t key_begin;   // first key position (a multiple of 16)
    int32_t key_end;     // one past the last key position (<= context length)
    int32_t partial_row; // -1: write the output; else first workspace row of this item's partials
    int32_t flags;       // PS_ITEM_* bits
    // Decode items walk their 32-key tiles starting at tile `rot` (mod the
    // tile count); nonzero only with the walk-rotation plan option, where
    // items that share prefix blocks then do not request the same lines at
    // the same time (softmax order is free). Prefill: 0.
    int32_t rot;
    // Gathered items (PS_ITEM_GATHERED): which slice of the shared prefix's
    // keys the item covers; its partials go to a row's dest + split * stride.
    int32_t split;
    int32_t pad[2];
};
static_assert(sizeof(ps_item) == 48, "ps_item layout");
// The one item per (sequence, KV head) that holds the sequence's last keys
// (last row range, last key slice): with the scatter fused into the
// decode launch it writes the step's new K/V rows of its KV head.
constexpr int32_t PS_ITEM_WRITES_NEW = 1;
// A prefill-kernel item of the shared-prefix pass: its rows come from
// several sequences, listed by the row map from entry partial_row on, and
// every key of its range is visible to every row.
constexpr int32_t PS_ITEM_GATHERED = 2;

// One gathered row: which sequence and packed row it is, and where its
// partial goes.
struct ps_row {
    int32_t seq;     // the row's sequence
    int32_t row;     // packed row within the sequence's KV head (token r / g, head j g + r % g)
    int32_t dest;    // workspace row of the first prefix slice's partial
    int32_t stride;  // rows from one slice's partial to the next
};
static_assert(sizeof(ps_row) == 16, "ps_row layout");

// A chunk of rows (at most ps_merge_rows(D)) of one set of split-K
// partials, merged into the output by one workgroup of the merge kernel.
struct ps_merge {
    int32_t seq;          // < 0: idle (fixed-shape padding)
    int32_t kv_head;
    int32_t row_begin;
    int32_t row_end;
    int32_t partial_row; // split i's row r is partial_row + i * split_stride + (r - row_begin)
    int32_t num_splits;
    int32_t split_stride; // rows of each split's partial block
    int32_t pad;
};
// rows one merge workgroup covers: 256 threads, each 4 elements of a row
inline int ps_merge_rows(int head_dim) { return 1024 / head_dim; }
static_assert(sizeof(ps_merge) == 32, "ps_merge layout");

// Bytes of one pool block (16 slots of num_kv_heads x head_dim elements).
// The kernels take a block's offset as a 32 x 32 -> 64-bit product of its
// id and this size, so a pool whose block exceeds INT32_MAX bytes is
// refused.
inline int64_t ps_block_bytes(const ps_pool *p) {
    return (int64_t)16 * p->num_kv_heads * p->head_dim * (p->dtype == PS_F32 ? 4 : 2);
}

// Tile geometry the planner and kernels agree on.
constexpr int PS_BLOCK = 16;            // tokens per pool block
constexpr int PS_DEC_TILE = 32;         // keys per decode-kernel wave iteration
constexpr int PS_DEC_MAX_ROWS = 32;     // packed rows per decode work item (two 16-row MFMA tiles)
constexpr int PS_DEC_MAX_SPLIT = 16384; // keys per decode work item at most
// Block ids of a decode item's first tiles in walk order (two per 32-key
// tile), laid out per item in the metadata: a wave's first tiles read
// their ids there, with no wait on the block table's row.
constexpr int PS_DEC_HEAD_TILES = 16;
constexpr int PS_PRE_TILE = 64;         // keys per prefill LDS tile
constexpr int PS_PRE_WAVES = 4;         // waves per prefill work item
constexpr int PS_PRE_ROWS_PER_WAVE = 32;
constexpr int PS_PRE_ROWS = PS_PRE_WAVES * PS_PRE_ROWS_PER_WAVE;  // 128 packed rows per prefill item
constexpr int PS_PRE_MAX_KEYS = 16384;  // keys per prefill item (its block ids are staged in LDS)

// Workspace layout for split-K partials (all fp32):
//   m[ws_rows]  running max (log2 domain), l[ws_rows] softmax denominator,
//   acc[ws_rows][D] unnormalised output.
inline size_t ps_align256(size_t x) { return (x + 255) & ~size_t(255); }

struct ps_ws_layout {
    size_t off_m, off_l, off_acc, bytes;
};

inline ps_ws_layout ps_workspace_layout(int64_t ws_rows, int head_dim) {
    ps_ws_layout w;
    w.off_m = 0;
    w.off_l = ps_align256(sizeof(float) * (size_t)ws_rows);
    w.off_acc = w.off_l + ps_align256(sizeof(float) * (size_t)ws_rows);
    w.bytes = ws_rows > 0 ? w.off_acc + ps_align256(sizeof(float) * (size_t)ws_rows * head_dim) : 0;
    return w;
}

// Everything a launch needs, resolved from the plan and the call's arguments.
struct ps_attn_launch {
    const void *q;
    void *out;
    const void *pool_k;
    const void *pool_v;
    // the call's per-sequence arrays: the kernels read every sequence's
    // offsets and block ids here
    const int32_t *block_tables;
    const int32_t *query_start_loc;
    const int32_t *num_computed;
    const int32_t *context_lens;
    const ps_item *decode_items;
    const ps_item *prefill_items;
    const ps_merge *merges;
    // [n_decode][2 * PS_DEC_HEAD_TILES] block ids of each decode item's
    // first tiles, copied from the plan's table. head_ok: the call reads
    // the plan's own uploaded table, so these are that table's entries
    // and a wave's first tiles need no table read; otherwise they are
    // never used.
    const int32_t *decode_head;
    int32_t head_ok;
    const ps_row *row_map;        // rows of the gathered (shared-prefix) items
    float *ws_m;
    float *ws_l;
    float *ws_acc;
    int64_t layer_offset;   // elements from pool start to this layer
    int32_t bt_stride;
    int32_t num_blocks;
    int32_t num_tokens;     // packed rows of q / out: row indexes are clamped below it
    int32_t num_q_heads;
    int32_t num_kv_heads;
    int32_t head_dim;
    int32_t dtype;
    int32_t n_decode, n_prefill, n_merge;
    int32_t decode_row_tiles;
    int32_t decode_waves;   // waves per decode workgroup (4, 8 or 16)
    int32_t mixed;          // decode and prefill items share one launch
    int32_t stream_kv;      // decode items load K/V non-temporally
    float scale_log2;       // softmax scale * log2(e)
    // g = num_q_heads / num_kv_heads, and r / g for 0 <= r < 2^31 as
    // (r * g_magic) >> g_shift (see ps_group_divisor)
    int32_t g;
    uint32_t g_magic;
    int32_t g_shift;
    // Scatter fused into the decode kernel (steps without prefill items):
    // keys at positions >= num_computed are read from k_new / v_new
    // ([T, Hkv, D]) and the item holding a sequence's last keys writes
    // them into their slots.
    int32_t fuse_scatter;
    int32_t num_slots;      // num_blocks * 16
    const void *k_new;
    const void *v_new;
    const int32_t *slot_mapping;
};

// Division by the group size g with a multiply and a shift (Granlund and
// Montgomery, "Division by invariant integers using multiplication", 1994):
// with l = ceil(log2 g), s = 31 + l and m = floor(2^s / g) + 1, the error
// e = m g - 2^s lies in (0, 2^l], so for 0 <= r < 2^31
// r m / 2^s = r / g + r e / (g 2^s) with the last term below 1 / g, and
// floor(r m / 2^s) = floor(r / g). m < 2^32.
inline void ps_group_divisor(int32_t g, uint32_t *magic, int32_t *shift) {
    int32_t l = 0;
    while ((int64_t(1) << l) < g) ++l;
    *shift = 31 + l;
    *magic = (uint32_t)(((uint64_t)1 << (31 + l)) / (uint64_t)g + 1);
}

// Rotary embedding + KV scatter launch (ps_rope.hip). The pair frequencies
// travel by value in the kernel arguments, so the call needs no device
// buffer of its own.
constexpr int PS_ROPE_MAX_HALF = 64;  // head_dim / 2 for head_dim <= 128
struct ps_rope_launch {
    const void *q;
    void *q_out;
    const void *k;
    const void *v;
    const int32_t *positions;
    const int32_t *slots;
    void *pool_k;            // this layer's K block array
    void *pool_v;
    int32_t num_tokens;
    int32_t num_q_heads;
    int32_t num_kv_heads;
    int32_t head_dim;
    int32_t dtype;
    int32_t num_slots;       // num_blocks * 16
    int32_t tokens_per_wg;   // set by the launcher
    double inv_freq[PS_ROPE_MAX_HALF];  // theta^(-2j/D), j < head_dim / 2
};

// Speculative verification launch (ps_spec.hip).
constexpr int PS_SPEC_CHUNK = 4096;   // vocab entries per first-pass workgroup
constexpr int PS_SPEC_MAX_VOCAB = 1 << 23;   // fixed-point sums stay below 2^63
struct ps_spec_launch {
    const float *target;       // [total_drafts + num_seqs, vocab]
    const float *draft;        // [total_drafts, vocab]
    const int32_t *tokens;     // [total_drafts]
    const int32_t *starts;     // [num_seqs + 1]
    const double *accept_u;    // [total_drafts]
    const double *sample_u;    // [num_seqs]
    int32_t *num_accepted;     // [num_seqs]
    int32_t *next_token;       // [num_seqs]
    uint64_t *chunk_sums;      // workspace [num_seqs, n_chunks]
    int32_t *decisions;        // workspace [num_seqs, 2]: drafts kept, malformed flag
    int32_t num_seqs, total_drafts, vocab, n_chunks;
};
inline size_t ps_spec_sums_bytes(int64_t num_seqs, int64_t vocab) {
    const int64_t chunks = (vocab + PS_SPEC_CHUNK - 1) / PS_SPEC_CHUNK;
    return ps_align256((size_t)(num_seqs * chunks * sizeof(uint64_t)));
}
inline size_t ps_spec_workspace(int64_t num_seqs, int64_t vocab) {
    return ps_spec_sums_bytes(num_seqs, vocab) + ps_align256((size_t)(num_seqs * 2 * sizeof(int32_t)));
}

// Kernel launchers (ps_kernels.hip, ps_rope.hip, ps_spec.hip). Return hipError_t as int.
int ps_launch_scatter(const void *k, const void *v, const int32_t *slot_mapping,
                      int32_t num_tokens, const ps_pool *pool, void *stream);
int ps_launch_attention(const ps_attn_launch &a, void *stream);
// The current device's static split-K workspace (PS_STATIC_WORKSPACE_BYTES),
// looked up once per device (ps_kernels.hip). Returns hipError_t as int.
int ps_static_workspace(void **ptr);
int ps_prefill_rows(int dtype);  // packed rows per prefill work item
int ps_launch_copy_blocks(const ps_pool *src, const ps_pool *dst, const int32_t *src_blocks,
                          const int32_t *dst_blocks, int32_t num_pairs, void *stream);
int ps_launch_rope_cache(const ps_rope_launch &a, void *stream);
int ps_launch_spec_verify(const ps_spec_launch &a, bool vec, void *stream);
const char *ps_hip_error_string(int err);

// Set the calling thread's error message (ps_capi.cpp).
ps_status ps_fail(ps_status st, const char *fmt, ...);
