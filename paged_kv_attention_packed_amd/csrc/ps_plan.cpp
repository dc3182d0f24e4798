// Host metadata builder for one packed step: validation, the packed batch's
// index arrays, the attention kernels' work lists and the step's
// algorithmic byte / FLOP counts. Pure host code: no HIP call happens here
// except in ps_plan_upload and the launches of the attention entry points.
//
// The packed layout follows PageServe "01 Scheduler loop" (Pack: one
// [1, T] batch, explicit positions, a slot mapping per token, no padding)
// and "03 Paged KV cache" (slot = block_table[pos / 16] * 16 + pos % 16).
//
// Every choice the planner makes comes from its arguments (flags and
// options) and is recorded in ps_plan_info; nothing is read from the
// process environment.

#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <chrono>
#include <cstdlib>
#include <cstring>
#include <new>
#include <vector>

#include "ps_internal.h"

struct ps_plan {
    int32_t S = 0, T = 0, Hq = 0, Hkv = 0, D = 0, dtype = 0;
    int32_t num_blocks = 0, num_layers = 0, bt_stride = 0;
    uint32_t flags = 0;
    int32_t dec_rt = 1, dec_waves = 4;
    bool mixed = false, fixed = false;
    bool stream_kv = false;   // decode K/V loads non-temporal
    bool rotate = false;      // decode walk rotation
    int64_t ws_rows = 0;                 // workspace layout rows (fixed shape: the capacity)
    int32_t rows_cap = 0;                // packed tokens q / out hold (fixed shape: max_tokens)
    int32_t n_dec = 0, n_pre = 0, n_mrg = 0;   // launched items (fixed shape: capacities)
    int32_t n_gathered = 0;              // prefill items of the shared-prefix pass
    // the metadata blob, laid out exactly as it is copied to the device
    std::vector<uint8_t> blob;
    size_t off_qsl = 0, off_nc = 0, off_ctx = 0, off_slot = 0, off_pos = 0, off_bt = 0;
    size_t off_dec = 0, off_pre = 0, off_mrg = 0, off_dhead = 0, off_rmap = 0;
    std::vector<int32_t> kinds;          // per sequence: 0 decode, 1 prefill, 2 decode after a shared prefix
    void *dev = nullptr;
    ps_plan_info info{};

    template <class X> X *host(size_t off) { return reinterpret_cast<X *>(blob.data() + off); }
    template <class X> const X *host(size_t off) const {
        return reinterpret_cast<const X *>(blob.data() + off);
    }
};

namespace {

int elt_bytes(int dtype) { return dtype == PS_F32 ? 4 : 2; }

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
int64_t round_up(int64_t a, int64_t b) { return ceil_div(a, b) * b; }

// Split [0, kmax) into near-equal pieces of at most `target` keys, each a
// multiple of `align` long except possibly the last (target a multiple of
// align). The split set depends only on logical lengths, so physical
// placement never changes results (only PS_PLAN_SHARED_PREFIX, which
// groups sequences by the blocks they share, makes the work depend on it).
void key_splits(int64_t kmax, int64_t target, int64_t align, std::vector<int64_t> &bounds) {
    bounds.clear();
    if (kmax <= target) {   // one slice (the common case, without the divisions)
        bounds.push_back(0);
        bounds.push_back(kmax);
        return;
    }
    int64_t n = std::max<int64_t>(1, ceil_div(kmax, target));
    int64_t len = round_up(ceil_div(kmax, n), align);
    n = ceil_div(kmax, len);
    for (int64_t i = 0; i <= n; ++i) bounds.push_back(std::min(kmax, i * len));
}

// Marks on the physical blocks a step's tables cover. The mark of block id
// is ((s + 1) << 6) | shared << 5 | n: the last sequence s that listed it
// (a block twice in one table is an error), whether more than one table
// lists it, and the most tokens n any of them reads from it. Marks live in
// one of two stores, kept per thread and reused, whose entries are all
// zero between plans (a plan clears what it set):
//   - dense: one mark per pool block, when the pool has at most four
//     blocks per table entry the step covers;
//   - hashed: an open-addressing table of 2-4 slots per table entry,
//     otherwise.
// Either way a plan costs time in proportion to the table entries it
// covers, and the memory it walks stays within a small multiple of them,
// however large the pool.
struct BlockMarks {
    std::vector<uint32_t> dense;
    struct Slot {
        int32_t id;      // -1: empty
        uint32_t mark;
    };
    std::vector<Slot> hashed;
    std::vector<uint32_t> used;   // hashed slots in use
    uint32_t mask = 0;
    int shift = 32;
    bool is_dense = true;

    void prepare(int32_t nb, int64_t entries) {
        is_dense = (int64_t)nb <= 4 * entries;
        if (is_dense) {
            if ((int64_t)dense.size() < nb) dense.assign((size_t)nb, 0u);
            return;
        }
        size_t cap = 64;
        int bits = 6;
        while ((int64_t)cap < 2 * entries) {
            cap <<= 1;
            ++bits;
        }
        if (hashed.size() < cap) hashed.assign(cap, Slot{-1, 0u});
        mask = (uint32_t)(cap - 1);
        shift = 32 - bits;
        used.clear();
        used.reserve((size_t)entries);
    }
    // start fetching the mark of id (the loop over table entries issues
    // these a few entries ahead, so that the random accesses overlap)
    void prefetch(int32_t id) const {
        if (is_dense) __builtin_prefetch(dense.data() + id, 1);
        else __builtin_prefetch(hashed.data() + (((uint32_t)id * 0x9E3779B1u) >> shift), 1);
    }
    uint32_t &at(int32_t id) {
        if (is_dense) return dense[(size_t)id];
        uint32_t h = ((uint32_t)id * 0x9E3779B1u) >> shift;
        while (hashed[h].id != id && hashed[h].id != -1) h = (h + 1) & mask;
        if (hashed[h].id == -1) {
            hashed[h].id = id;
            used.push_back(h);
        }
        return hashed[h].mark;
    }
    // zero every mark a plan over `entries` table entries set
    template <class ForEachId>
    void clear(int32_t nb, int64_t entries, ForEachId each_id) {
        if (!is_dense) {
            for (uint32_t h : used) hashed[h] = Slot{-1, 0u};
            used.clear();
        } else if ((int64_t)nb <= 8 * entries) {
            std::memset(dense.data(), 0, sizeof(uint32_t) * (size_t)nb);
        } else {
            each_id([&](int32_t id) { dense[(size_t)id] = 0u; });
        }
    }
};

thread_local BlockMarks t_marks;

bool is_multiple_in(int64_t v, int64_t m, int64_t lo, int64_t hi) { return v % m == 0 && v >= lo && v <= hi; }

ps_status check_options(const ps_plan_options &o, uint32_t flags, const ps_pool *pool, int32_t g) {
    if (o.decode_split_keys && !is_multiple_in(o.decode_split_keys, PS_BLOCK, PS_BLOCK, PS_DEC_MAX_SPLIT))
        return ps_fail(PS_ERR_INVALID_ARGUMENT, "decode_split_keys %d: a multiple of 16 in [16, %d]",
                       o.decode_split_keys, PS_DEC_MAX_SPLIT);
    if (o.prefill_split_keys && !is_multiple_in(o.prefill_split_keys, PS_PRE_TILE, PS_PRE_TILE, PS_PRE_MAX_KEYS))
        return ps_fail(PS_ERR_INVALID_ARGUMENT, "prefill_split_keys %d: a multiple of 64 in [64, %d]",
                       o.prefill_split_keys, PS_PRE_MAX_KEYS);
    if (o.prefix_slice_keys && !is_multiple_in(o.prefix_slice_keys, PS_PRE_TILE, PS_PRE_TILE, PS_PRE_MAX_KEYS))
        return ps_fail(PS_ERR_INVALID_ARGUMENT, "prefix_slice_keys %d: a multiple of 64 in [64, %d]",
                       o.prefix_slice_keys, PS_PRE_MAX_KEYS);
    if (o.decode_waves != 0 && o.decode_waves != 4 && o.decode_waves != 8 && o.decode_waves != 16)
        return ps_fail(PS_ERR_INVALID_ARGUMENT, "decode_waves %d: 0, 4, 8 or 16", o.decode_waves);
    if (o.decode_waves == 16 && (pool->head_dim != 64 || pool->dtype == PS_F32))
        return ps_fail(PS_ERR_INVALID_ARGUMENT, "decode_waves 16 needs head_dim 64 and 16-bit data");
    if (o.prefix_min_seqs < 0 || o.prefix_min_seqs == 1 || o.prefix_min_keys < 0 ||
        (o.prefix_min_keys > 0 && o.prefix_min_keys < PS_BLOCK))
        return ps_fail(PS_ERR_INVALID_ARGUMENT, "prefix_min_seqs must be 0 or >= 2, prefix_min_keys 0 or >= 16");
    for (int i = 0; i < 2; ++i)
        if (o.reserved[i] != 0) return ps_fail(PS_ERR_INVALID_ARGUMENT, "reserved option fields must be 0");
    if (o.decode_stream_kv < 0 || o.decode_stream_kv > 2)
        return ps_fail(PS_ERR_INVALID_ARGUMENT, "decode_stream_kv %d: 0, 1 or 2", o.decode_stream_kv);
    if (o.decode_walk_rotation < 0 || o.decode_walk_rotation > 2)
        return ps_fail(PS_ERR_INVALID_ARGUMENT, "decode_walk_rotation %d: 0, 1 or 2", o.decode_walk_rotation);
    if (flags & PS_PLAN_FIXED_SHAPE) {
        if ((flags & 3) == PS_PLAN_ALL_PREFILL || (flags & PS_PLAN_SHARED_PREFIX))
            return ps_fail(PS_ERR_INVALID_ARGUMENT,
                           "PS_PLAN_FIXED_SHAPE runs every sequence on the decode kernel: no "
                           "PS_PLAN_ALL_PREFILL, no PS_PLAN_SHARED_PREFIX");
        if (o.max_seqs < 1 || o.max_tokens < 1 || o.max_query_len < 1 || o.max_decode_items < 0 ||
            o.max_merge_items < 0 || o.max_workspace_rows < 0)
            return ps_fail(PS_ERR_INVALID_ARGUMENT, "fixed shape needs max_seqs, max_tokens, max_query_len >= 1");
        if ((int64_t)g * o.max_query_len > PS_DEC_MAX_ROWS)
            return ps_fail(PS_ERR_INVALID_ARGUMENT,
                           "fixed shape: %d query heads per KV head x max_query_len %d exceeds %d rows", g,
                           o.max_query_len, PS_DEC_MAX_ROWS);
        if ((o.max_decode_items == 0 ? (int64_t)o.max_seqs * pool->num_kv_heads : o.max_decode_items) > INT32_MAX / 2)
            return ps_fail(PS_ERR_INVALID_ARGUMENT, "fixed shape capacity too large");
    }
    return PS_OK;
}

}  // namespace

extern "C" ps_status ps_plan_step(const int32_t *q_lens, const int32_t *num_computed_tokens,
                                  int32_t num_seqs, const int32_t *block_tables,
                                  int32_t block_table_stride, int32_t num_q_heads,
                                  const ps_pool *pool, uint32_t flags, const ps_plan_options *options,
                                  ps_plan **out_plan) {
    const auto t_start = std::chrono::steady_clock::now();
    if (!out_plan) return ps_fail(PS_ERR_INVALID_ARGUMENT, "out_plan is NULL");
    *out_plan = nullptr;
    if (!pool) return ps_fail(PS_ERR_INVALID_ARGUMENT, "pool is NULL");
    if (num_seqs < 0) return ps_fail(PS_ERR_INVALID_ARGUMENT, "num_seqs < 0");
    if (num_seqs > 0 && (!q_lens || !num_computed_tokens || !block_tables))
        return ps_fail(PS_ERR_INVALID_ARGUMENT, "q_lens, num_computed_tokens and block_tables must be non-NULL");
    const uint32_t known = 3u | PS_PLAN_SHARED_PREFIX | PS_PLAN_SEPARATE_LAUNCHES | PS_PLAN_FIXED_SHAPE;
    if ((flags & ~known) != 0 || (flags & 3) == 3)
        return ps_fail(PS_ERR_INVALID_ARGUMENT, "unknown plan flags %u", flags);
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
    if (num_q_heads < 1 || num_q_heads % pool->num_kv_heads != 0)
        return ps_fail(PS_ERR_INVALID_ARGUMENT, "num_q_heads %d is not a positive multiple of num_kv_heads %d",
                       num_q_heads, pool->num_kv_heads);
    if ((num_seqs > 0 || (flags & PS_PLAN_FIXED_SHAPE)) && block_table_stride < 1)
        return ps_fail(PS_ERR_INVALID_ARGUMENT, "block_table_stride %d < 1", block_table_stride);

    const int32_t S = num_seqs;
    const int32_t Hkv = pool->num_kv_heads, D = pool->head_dim, NB = pool->num_blocks;
    const int32_t g = num_q_heads / Hkv;
    const uint32_t route = flags & 3;
    const bool fixed = (flags & PS_PLAN_FIXED_SHAPE) != 0;
    const ps_plan_options opt = options ? *options : ps_plan_options{};
    {
        const ps_status st = check_options(opt, flags, pool, g);
        if (st != PS_OK) return st;
    }

    // ---- per-sequence checks
    int64_t T = 0, n_entries = 0;
    for (int32_t s = 0; s < S; ++s) {
        const int64_t n = q_lens[s], c = num_computed_tokens[s];
        if (n < 1) return ps_fail(PS_ERR_INVALID_ARGUMENT, "q_lens[%d] = %lld < 1", s, (long long)n);
        if (c < 0) return ps_fail(PS_ERR_INVALID_ARGUMENT, "num_computed_tokens[%d] = %lld < 0", s, (long long)c);
        const int64_t ctx = c + n;
        if (ctx > (int64_t)block_table_stride * PS_BLOCK)
            return ps_fail(PS_ERR_INVALID_ARGUMENT,
                           "sequence %d: context %lld needs %lld blocks, table width is %d", s,
                           (long long)ctx, (long long)ceil_div(ctx, PS_BLOCK), block_table_stride);
        if ((int64_t)g * n > INT32_MAX / 2 || ctx > INT32_MAX / 2)
            return ps_fail(PS_ERR_UNSUPPORTED, "sequence %d too long", s);
        if (fixed && n > opt.max_query_len)
            return ps_fail(PS_ERR_INVALID_ARGUMENT, "q_lens[%d] = %lld exceeds the fixed shape's max_query_len %d",
                           s, (long long)n, opt.max_query_len);
        T += n;
        n_entries += ceil_div(ctx, PS_BLOCK);
    }
    if (T > INT32_MAX / 2) return ps_fail(PS_ERR_UNSUPPORTED, "too many tokens (%lld)", (long long)T);
    if (fixed && (S > opt.max_seqs || T > opt.max_tokens))
        return ps_fail(PS_ERR_INVALID_ARGUMENT, "step of %d sequences / %lld tokens exceeds the fixed shape's %d / %d",
                       S, (long long)T, opt.max_seqs, opt.max_tokens);

    // ---- block ids, duplicates within a table, shared blocks: one pass
    // over the table entries the step covers
    if (S >= (1 << 25)) return ps_fail(PS_ERR_UNSUPPORTED, "too many sequences (%d)", S);
    BlockMarks &bm = t_marks;
    try {
        bm.prepare(NB, n_entries);
    } catch (const std::bad_alloc &) {
        return ps_fail(PS_ERR_HOST_MEMORY, "host allocation failed");
    }
    int64_t kv_rows_unique = 0;   // distinct (physical block, token) rows the step reads
    int64_t shared_refs = 0;      // table entries naming a block an earlier table named
    {
        // clears every mark the step's entries may have set (also after an
        // error part way through)
        struct Clear {
            BlockMarks &bm;
            const int32_t *q_lens, *nc, *bt;
            int32_t S, stride, NB;
            int64_t entries;
            ~Clear() {
                bm.clear(NB, entries, [&](auto zero) {
                    for (int32_t s = 0; s < S; ++s) {
                        const int32_t *row = bt + (int64_t)s * stride;
                        const int64_t nblk = ceil_div((int64_t)nc[s] + q_lens[s], PS_BLOCK);
                        for (int64_t b = 0; b < nblk; ++b)
                            if (row[b] >= 0 && row[b] < NB) zero(row[b]);
                    }
                });
            }
        } clear{bm, q_lens, num_computed_tokens, block_tables, S, block_table_stride, NB, n_entries};
        constexpr uint32_t kShared = 1u << 5;
        // one pass over every table entry the step covers, branch-free but
        // for the (rare) errors; `slot` gives the mark of a block id
        auto scan = [&](auto slot, auto prefetch) -> ps_status {
            // (a local copy: the marks' stores cannot alias it, so it stays
            // in a register instead of being reloaded per entry)
            const uint32_t nb = (uint32_t)NB;
            int64_t uniq = 0, again = 0;
            for (int32_t s = 0; s < S; ++s) {
                const int32_t *row = block_tables + (int64_t)s * block_table_stride;
                const int64_t ctx = (int64_t)num_computed_tokens[s] + q_lens[s];
                const int64_t nblk = ceil_div(ctx, PS_BLOCK);
                const uint32_t tag = (uint32_t)(s + 1) << 6;
                constexpr int64_t kAhead = 16;
                for (int64_t b = 0; b < std::min(nblk, kAhead); ++b) prefetch(row[b]);
                // blocks before the last are full (16 tokens, never fewer
                // than a mark holds), the last holds the rest
                const int64_t nfull = nblk - 1;
                auto entry = [&](int64_t b, uint32_t ntok, auto full) -> bool {
                    const int32_t id = row[b];
                    if ((uint32_t)id >= nb) {
                        ps_fail(PS_ERR_INVALID_ARGUMENT, "block_tables[%d][%lld] = %d outside [0, %d)", s,
                                (long long)b, id, NB);
                        return false;
                    }
                    if (b + kAhead < nblk) prefetch(row[b + kAhead]);
                    uint32_t &m = slot(id);
                    const uint32_t m0 = m;
                    if ((m0 >> 6) == (uint32_t)(s + 1)) {
                        ps_fail(PS_ERR_INVALID_ARGUMENT, "block %d appears twice in the table of sequence %d", id, s);
                        return false;
                    }
                    const uint32_t old = m0 & 31u;
                    const uint32_t seen = m0 != 0u;
                    again += seen;
                    if constexpr (decltype(full)::value) {
                        uniq += PS_BLOCK - old;
                        m = tag | (seen << 5) | PS_BLOCK;
                    } else {
                        uniq += ntok > old ? ntok - old : 0;
                        m = tag | (seen << 5) | std::max(ntok, old);
                    }
                    return true;
                };
                for (int64_t b = 0; b < nfull; ++b)
                    if (!entry(b, PS_BLOCK, std::true_type{})) return PS_ERR_INVALID_ARGUMENT;
                if (!entry(nfull, (uint32_t)(ctx - nfull * PS_BLOCK), std::false_type{})) return PS_ERR_INVALID_ARGUMENT;
            }
            kv_rows_unique = uniq;
            shared_refs = again;
            return PS_OK;
        };
        uint32_t *const dense = bm.dense.data();
        const ps_status scanned =
            bm.is_dense ? scan([dense](int32_t id) -> uint32_t & { return dense[(size_t)id]; }, [](int32_t) {})
                        : scan([&](int32_t id) -> uint32_t & { return bm.at(id); },
                               [&](int32_t id) { if ((uint32_t)id < (uint32_t)NB) bm.prefetch(id); });
        if (scanned != PS_OK) return scanned;
        for (int32_t s = 0; s < S; ++s) {
            const int32_t *row = block_tables + (int64_t)s * block_table_stride;
            const int64_t c = num_computed_tokens[s], ctx = c + q_lens[s];
            for (int64_t b = c / PS_BLOCK; b < ceil_div(ctx, PS_BLOCK); ++b)
                if (bm.at(row[b]) & kShared)
                    return ps_fail(PS_ERR_INVALID_ARGUMENT,
                                   "sequence %d writes new tokens into block %d, which other tables share "
                                   "(copy it before writing)", s, row[b]);
        }
    }

    ps_plan *p = new (std::nothrow) ps_plan();
    if (!p) return ps_fail(PS_ERR_HOST_MEMORY, "host allocation failed");
    p->S = S;
    p->T = (int32_t)T;
    p->Hq = num_q_heads;
    p->Hkv = Hkv;
    p->D = D;
    p->dtype = pool->dtype;
    p->num_blocks = NB;
    p->num_layers = pool->num_layers;
    p->bt_stride = S > 0 || fixed ? std::max(1, block_table_stride) : 1;
    p->flags = flags;
    p->fixed = fixed;

    try {
        // ---- work lists
        std::vector<ps_item> dec, pre;
        std::vector<ps_merge> mrg;
        dec.reserve((size_t)S * Hkv);
        std::vector<char> is_dec(S);
        for (int32_t s = 0; s < S; ++s) {
            const int64_t rows = (int64_t)g * q_lens[s];
            is_dec[s] = (route == PS_PLAN_ALL_DECODE) || fixed ||
                        (route == PS_PLAN_DEFAULT && rows <= PS_DEC_MAX_ROWS);
        }
        const int64_t pre_rows = PS_PRE_ROWS;
        const bool mixed_ok = !(flags & PS_PLAN_SEPARATE_LAUNCHES) && pool->dtype != PS_F32;

        // ---- shared prefixes (PS_PLAN_SHARED_PREFIX). Decode sequences
        // whose tables open with the same physical blocks (blocks shared by
        // reference, PageServe "03 Paged KV cache") form a group. Attention
        // over the shared prefix then runs once per group, in prefill-kernel
        // items whose query rows are gathered from every member: each prefix
        // key lies below every member's first query position, so no mask
        // applies. Each member's decode items cover only its keys after the
        // prefix, and the partial softmax states merge like key splits. A
        // member must share at least prefix_min_keys tokens (whole blocks of
        // its cached context) with the group's first sequence, and a group
        // needs prefix_min_seqs members.
        std::vector<int32_t> grp_of(S, -1);
        std::vector<int32_t> grp_lead;
        std::vector<int64_t> grp_keys;
        std::vector<std::vector<int64_t>> grp_bounds;
        if ((flags & PS_PLAN_SHARED_PREFIX) && route == PS_PLAN_DEFAULT) {
            const int64_t min_seqs = opt.prefix_min_seqs ? opt.prefix_min_seqs : 8;
            const int64_t min_blocks = ceil_div(opt.prefix_min_keys ? opt.prefix_min_keys : 256, PS_BLOCK);
            // candidates, sorted by their first min_blocks block ids: runs of
            // equal keys are the groups
            std::vector<int32_t> cand;
            for (int32_t s = 0; s < S; ++s)
                if (is_dec[s] && num_computed_tokens[s] >= min_blocks * PS_BLOCK) cand.push_back(s);
            auto row_of = [&](int32_t s) { return block_tables + (int64_t)s * block_table_stride; };
            auto key_less = [&](int32_t x, int32_t y) {
                const int32_t *a = row_of(x), *b = row_of(y);
                for (int64_t i = 0; i < min_blocks; ++i)
                    if (a[i] != b[i]) return a[i] < b[i];
                return x < y;
            };
            auto key_same = [&](int32_t x, int32_t y) {
                return std::memcmp(row_of(x), row_of(y), sizeof(int32_t) * (size_t)min_blocks) == 0;
            };
            std::sort(cand.begin(), cand.end(), key_less);
            for (size_t a0 = 0; a0 < cand.size();) {
                size_t a1 = a0 + 1;
                while (a1 < cand.size() && key_same(cand[a0], cand[a1])) ++a1;
                if ((int64_t)(a1 - a0) >= min_seqs) {
                    // the group's prefix: the blocks every member shares with
                    // the first one, within every member's cached context
                    const int32_t lead = cand[a0];
                    const int32_t *lrow = row_of(lead);
                    int64_t common = num_computed_tokens[lead] / PS_BLOCK;
                    for (size_t x = a0 + 1; x < a1; ++x) {
                        const int32_t *mrow = row_of(cand[x]);
                        const int64_t lim = std::min<int64_t>(common, num_computed_tokens[cand[x]] / PS_BLOCK);
                        int64_t b = min_blocks;
                        while (b < lim && mrow[b] == lrow[b]) ++b;
                        common = b;
                    }
                    for (size_t x = a0; x < a1; ++x) grp_of[cand[x]] = (int32_t)grp_lead.size();
                    grp_lead.push_back(lead);
                    grp_keys.push_back(common * PS_BLOCK);
                }
                a0 = a1;
            }
            // prefix slices: about 128 prefix items per step (they share the
            // launch with the decode items), none shorter than 256 keys and
            // none longer than a prefill item's staged block list
            grp_bounds.resize(grp_lead.size());
            std::vector<int64_t> grp_rows(grp_lead.size(), 0);
            for (int32_t s = 0; s < S; ++s)
                if (grp_of[s] >= 0) grp_rows[grp_of[s]] += (int64_t)g * q_lens[s];
            for (size_t gi = 0; gi < grp_lead.size(); ++gi) {
                const int64_t chunks = ceil_div(grp_rows[gi], pre_rows) * Hkv;
                const int64_t want = std::max<int64_t>(1, std::min<int64_t>(ceil_div(128, chunks), grp_keys[gi] / 256));
                const int64_t slice = opt.prefix_slice_keys ? opt.prefix_slice_keys
                                                            : round_up(ceil_div(grp_keys[gi], want), PS_PRE_TILE);
                key_splits(grp_keys[gi], std::min<int64_t>(slice, PS_PRE_MAX_KEYS), PS_PRE_TILE, grp_bounds[gi]);
            }
        }
        // decode: a work item covers <= 32 packed rows and a slice of keys.
        // Slices are long (>= 2048 keys): a split costs a merge launch and
        // partial traffic, which only pays off against long contexts; very
        // long steps are cut into about 512 items (two per CU). A fixed
        // shape does not split unless told to.
        int64_t dec_keys = 0, pre_kmax = 0, pre_tiles = 0;
        for (int32_t s = 0; s < S; ++s) {
            const int64_t rows = (int64_t)g * q_lens[s], c = num_computed_tokens[s];
            const int64_t rb = is_dec[s] ? PS_DEC_MAX_ROWS : pre_rows;
            const int64_t pk = grp_of[s] >= 0 ? grp_keys[grp_of[s]] : 0;
            for (int64_t r0 = 0; r0 < rows; r0 += rb) {
                const int64_t r1 = std::min(rows, r0 + rb);
                const int64_t kmax = c + (r1 - 1) / g + 1;
                if (is_dec[s]) dec_keys += (kmax - pk) * Hkv;
                else { pre_kmax = std::max(pre_kmax, kmax); pre_tiles += Hkv; }
            }
        }
        const int64_t dec_split =
            opt.decode_split_keys ? opt.decode_split_keys
            : fixed               ? PS_DEC_MAX_SPLIT
                                  : std::min<int64_t>(PS_DEC_MAX_SPLIT,
                                                      std::max<int64_t>(2048, round_up(ceil_div(dec_keys, 512), 128)));
        // Prefill: aim for three full rounds of resident workgroups (256 CUs
        // x 2 = 512): each (row block, KV head) gets at most 1536 / blocks
        // slices, sized from the longest key range so that no block gets
        // more (a partly filled last round leaves CUs idle). A slice shorter
        // than ~512 keys costs more in partials (a 128-row tile's partials
        // weigh as much as ~500 keys of K/V) than it balances.
        const int64_t pre_slices = std::max<int64_t>(1, 1536 / std::max<int64_t>(1, pre_tiles));
        int64_t pre_auto = pre_tiles >= 512 ? PS_PRE_MAX_KEYS
                                            : std::max<int64_t>(512, round_up(ceil_div(pre_kmax, pre_slices), PS_PRE_TILE));
        // In a mixed launch the decode items keep the chip busy while the
        // prefill items run. Slicing then pays only if an unsliced prefill
        // item would outlast the decode work by far: it costs a merge
        // launch and the partials. Time models measured on MI355X: a
        // 128-row prefill item at ~1.9 TFLOP/s (two per CU), decode K/V
        // reads at ~4 TB/s.
        if (dec_keys > 0 && mixed_ok) {
            const double t_dec = (double)dec_keys * 2.0 * D * elt_bytes(pool->dtype) / 4.0e6;  // us
            const double t_pre = (double)pre_kmax * pre_rows * 4.0 * D / 1.9e6;               // us
            if (t_pre <= 2.0 * t_dec) pre_auto = PS_PRE_MAX_KEYS;
        }
        const int64_t pre_split = std::min<int64_t>(
            PS_PRE_MAX_KEYS, opt.prefill_split_keys ? opt.prefill_split_keys : round_up(pre_auto, PS_PRE_TILE));

        std::vector<int64_t> bounds;
        int64_t ws_rows = 0;
        int32_t dec_rt = 1;
        // gathered rows of each (group, KV head): the prefix items' row maps
        std::vector<std::vector<ps_row>> grows(grp_lead.size() * (size_t)Hkv);
        for (int32_t s = 0; s < S; ++s) {
            const int64_t rows = (int64_t)g * q_lens[s], c = num_computed_tokens[s];
            const bool d = is_dec[s];
            const int64_t rb = d ? PS_DEC_MAX_ROWS : pre_rows;
            const int32_t gi = grp_of[s];
            const int64_t pk = gi >= 0 ? grp_keys[gi] : 0;                          // prefix keys
            const int64_t npk = gi >= 0 ? (int64_t)grp_bounds[gi].size() - 1 : 0;   // prefix slices
            for (int32_t j = 0; j < Hkv; ++j) {
                for (int64_t r0 = 0; r0 < rows; r0 += rb) {
                    const int64_t r1 = std::min(rows, r0 + rb);
                    const int64_t kmax = c + (r1 - 1) / g + 1;
                    key_splits(kmax - pk, d ? dec_split : pre_split, d ? PS_BLOCK : PS_PRE_TILE, bounds);
                    for (int64_t &b : bounds) b += pk;
                    const int64_t ns = (int64_t)bounds.size() - 1;
                    const int64_t nsplit = npk + ns;   // partial sets the merge combines
                    if (d) dec_rt = std::max<int32_t>(dec_rt, (int32_t)ceil_div(r1 - r0, 16));
                    const int64_t base = nsplit > 1 ? ws_rows : -1;
                    if (gi >= 0) {
                        // the prefix slices' partials come first in the row range's block
                        std::vector<ps_row> &gr = grows[(size_t)gi * Hkv + j];
                        for (int64_t r = r0; r < r1; ++r) {
                            ps_row e{};
                            e.seq = s;
                            e.row = (int32_t)r;
                            e.dest = (int32_t)(base + (r - r0));
                            e.stride = (int32_t)(r1 - r0);
                            gr.push_back(e);
                        }
                    }
                    for (int64_t i = 0; i < ns; ++i) {
                        ps_item it{};
                        it.seq = s;
                        it.kv_head = j;
                        it.row_begin = (int32_t)r0;
                        it.row_end = (int32_t)r1;
                        it.key_begin = (int32_t)bounds[i];
                        it.key_end = (int32_t)bounds[i + 1];
                        it.partial_row = nsplit > 1 ? (int32_t)(base + (npk + i) * (r1 - r0)) : -1;
                        it.flags = r1 == rows && i == ns - 1 ? PS_ITEM_WRITES_NEW : 0;
                        (d ? dec : pre).push_back(it);
                    }
                    if (nsplit > 1) {
                        const int64_t mr = ps_merge_rows(D);
                        for (int64_t q0 = r0; q0 < r1; q0 += mr) {
                            ps_merge m{};
                            m.seq = s;
                            m.kv_head = j;
                            m.row_begin = (int32_t)q0;
                            m.row_end = (int32_t)std::min(r1, q0 + mr);
                            m.partial_row = (int32_t)(base + (q0 - r0));
                            m.num_splits = (int32_t)nsplit;
                            m.split_stride = (int32_t)(r1 - r0);
                            mrg.push_back(m);
                        }
                        ws_rows += nsplit * (r1 - r0);
                    }
                }
            }
        }
        // the prefix items: chunks of gathered rows x prefix key slices
        std::vector<ps_row> rmap;
        int32_t n_gathered = 0;
        for (size_t gi = 0; gi < grp_lead.size(); ++gi) {
            for (int32_t j = 0; j < Hkv; ++j) {
                const std::vector<ps_row> &gr = grows[gi * Hkv + j];
                for (size_t c0 = 0; c0 < gr.size(); c0 += (size_t)pre_rows) {
                    const size_t c1 = std::min(gr.size(), c0 + (size_t)pre_rows);
                    const int32_t off = (int32_t)rmap.size();
                    rmap.insert(rmap.end(), gr.begin() + c0, gr.begin() + c1);
                    for (size_t k = 0; k + 1 < grp_bounds[gi].size(); ++k) {
                        ps_item it{};
                        it.seq = grp_lead[gi];
                        it.kv_head = j;
                        it.row_begin = 0;
                        it.row_end = (int32_t)(c1 - c0);
                        it.key_begin = (int32_t)grp_bounds[gi][k];
                        it.key_end = (int32_t)grp_bounds[gi][k + 1];
                        it.partial_row = off;
                        it.flags = PS_ITEM_GATHERED;
                        it.split = (int32_t)k;
                        pre.push_back(it);
                        ++n_gathered;
                    }
                }
            }
        }
        if (ws_rows > INT32_MAX / 2) {
            delete p;
            return ps_fail(PS_ERR_UNSUPPORTED, "split-K workspace too large");
        }
        // Every item's key span fits the block ids its kernel stages in LDS.
        for (const ps_item &it : dec)
            if (it.key_end - it.key_begin > PS_DEC_MAX_SPLIT || it.key_end <= it.key_begin) {
                delete p;
                return ps_fail(PS_ERR_UNSUPPORTED, "decode item of %d keys (internal limit %d)",
                               it.key_end - it.key_begin, PS_DEC_MAX_SPLIT);
            }
        for (const ps_item &it : pre)
            if (it.key_end - it.key_begin > PS_PRE_MAX_KEYS || it.key_end <= it.key_begin) {
                delete p;
                return ps_fail(PS_ERR_UNSUPPORTED, "prefill item of %d keys (internal limit %d)",
                               it.key_end - it.key_begin, PS_PRE_MAX_KEYS);
            }
        // Walk rotation: a decode item starts its walk at a tile that depends
        // on the item's creation index, so that items reading the same
        // blocks do not all ask for the same lines at once. It depends on
        // the step's logical shape only, never on which blocks are shared.
        // Measured on MI355X: 256 sequences behind one shared prefix (512
        // items) -5%, the long-context verify step and the 1.5B mixed step
        // unchanged, 64 short decodes (128 items) +16%; so by default on
        // from 512 decode items (the resident workgroup slots) up.
        p->rotate = opt.decode_walk_rotation == 1 ||
                    (opt.decode_walk_rotation == 0 && !fixed && dec.size() >= 512);
        if (p->rotate)
            for (size_t k = 0; k < dec.size(); ++k) {
                const uint32_t ntiles = (uint32_t)ceil_div(dec[k].key_end - dec[k].key_begin, PS_DEC_TILE);
                dec[k].rot = ntiles > 1 ? (int32_t)((uint32_t)(k * 13) % ntiles) : 0;
            }
        // Longest decode items first (longest-processing-time order): in a
        // launch with more items than resident workgroups the ones that
        // start late are the short ones, and in a mixed launch the longest
        // decode items start next to prefill items. Measured on MI355X: C4
        // -10%, C3 -5%; a decode-only launch whose items all start at once
        // (C2, 128 items) gains nothing and keeps the sequence order.
        // Nothing else depends on the order: merges and partials are
        // addressed by workspace row.
        if (!pre.empty() || dec.size() > 256) {
            // (a stable sort on 8-byte keys, the original index breaking
            // ties, then one pass moving the items)
            std::vector<uint64_t> order(dec.size());
            for (size_t k = 0; k < dec.size(); ++k)
                order[k] = (uint64_t)(uint32_t)(INT32_MAX - (dec[k].key_end - dec[k].key_begin)) << 32 | k;
            std::sort(order.begin(), order.end());
            std::vector<ps_item> sorted(dec.size());
            for (size_t k = 0; k < dec.size(); ++k) sorted[k] = dec[(uint32_t)order[k]];
            dec.swap(sorted);
        }

        // ---- launch shape (fixed: from the capacities alone)
        const int32_t act_dec = (int32_t)dec.size(), act_mrg = (int32_t)mrg.size();
        int64_t cap_dec = act_dec, cap_mrg = act_mrg, cap_ws = ws_rows;
        int64_t cap_S = S, cap_T = T;
        if (fixed) {
            cap_dec = opt.max_decode_items ? opt.max_decode_items : (int64_t)opt.max_seqs * Hkv;
            cap_mrg = opt.max_merge_items;
            cap_ws = opt.max_workspace_rows;
            cap_S = opt.max_seqs;
            cap_T = opt.max_tokens;
            if (act_dec > cap_dec || act_mrg > cap_mrg || ws_rows > cap_ws) {
                delete p;
                return ps_fail(PS_ERR_INVALID_ARGUMENT,
                               "step needs %d decode items, %d merges, %lld partial rows; the fixed shape "
                               "holds %lld, %lld, %lld", act_dec, act_mrg, (long long)ws_rows,
                               (long long)cap_dec, (long long)cap_mrg, (long long)cap_ws);
            }
            dec_rt = (int32_t)ceil_div((int64_t)g * opt.max_query_len, 16);
            ps_item idle{};
            idle.seq = -1;
            dec.resize((size_t)cap_dec, idle);
            ps_merge midle{};
            midle.seq = -1;
            mrg.resize((size_t)cap_mrg, midle);
        }
        p->dec_rt = dec_rt;
        p->ws_rows = cap_ws;
        p->rows_cap = (int32_t)cap_T;
        p->n_dec = (int32_t)dec.size();
        p->n_pre = (int32_t)pre.size();
        p->n_mrg = (int32_t)mrg.size();
        p->n_gathered = n_gathered;
        p->mixed = mixed_ok && p->n_dec > 0 && p->n_pre > 0;
        // few decode items: more waves per item, so a short slice is read in
        // one round trip; many items: 4 waves each fill the chip
        p->dec_waves = opt.decode_waves ? opt.decode_waves : (p->n_dec < 512 ? 8 : 4);
        if (dec_rt == 2 || p->mixed || p->dtype == PS_F32 || D != 64) p->dec_waves = std::min(p->dec_waves, 8);
        if (dec_rt == 2 || p->mixed) p->dec_waves = 4;
        // Cache policy of the decode K/V loads. A step reads each
        // unshared block once; when its decode K/V also exceed the 256 MiB
        // last-level cache, caching them only evicts other data, and
        // non-temporal loads ran 10% faster on MI355X (long-context verify,
        // 1 GiB of K/V). Shared blocks are read again by other sequences in
        // the same step, and smaller steps can still find their K/V cached
        // from the step before: those keep the cached loads. A fixed-shape
        // plan must not change kernels from step to step: cached.
        {
            int64_t dec_kv = 0;
            for (int32_t s = 0; s < S; ++s)
                if (is_dec[s])
                    dec_kv += ((int64_t)num_computed_tokens[s] + q_lens[s]) * Hkv * 2 * D * elt_bytes(pool->dtype);
            p->stream_kv = opt.decode_stream_kv == 1 ||
                           (opt.decode_stream_kv == 0 && !fixed && shared_refs == 0 && dec_kv > ((int64_t)256 << 20));
        }

        // ---- blob layout
        size_t off = 0;
        auto take = [&](size_t bytes) {
            size_t o = off;
            off = ps_align256(off + std::max<size_t>(bytes, 1));
            return o;
        };
        p->off_qsl = take(sizeof(int32_t) * (size_t)(cap_S + 1));
        p->off_nc = take(sizeof(int32_t) * (size_t)cap_S);
        p->off_ctx = take(sizeof(int32_t) * (size_t)cap_S);
        p->off_slot = take(sizeof(int32_t) * (size_t)cap_T);
        p->off_pos = take(sizeof(int32_t) * (size_t)cap_T);
        p->off_bt = take(sizeof(int32_t) * (size_t)cap_S * p->bt_stride);
        p->off_dec = take(sizeof(ps_item) * dec.size());
        p->off_pre = take(sizeof(ps_item) * pre.size());
        p->off_mrg = take(sizeof(ps_merge) * mrg.size());
        p->off_dhead = take(sizeof(int32_t) * 2 * PS_DEC_HEAD_TILES * dec.size());
        p->off_rmap = take(sizeof(ps_row) * rmap.size());
        p->blob.assign(off, 0);

        int32_t *qsl = p->host<int32_t>(p->off_qsl);
        int32_t *nc = p->host<int32_t>(p->off_nc);
        int32_t *ctxl = p->host<int32_t>(p->off_ctx);
        int32_t *slot = p->host<int32_t>(p->off_slot);
        int32_t *posn = p->host<int32_t>(p->off_pos);
        int32_t *bt = p->host<int32_t>(p->off_bt);
        qsl[0] = 0;
        for (int32_t s = 0; s < S; ++s) {
            qsl[s + 1] = qsl[s] + q_lens[s];
            nc[s] = num_computed_tokens[s];
            ctxl[s] = num_computed_tokens[s] + q_lens[s];
            const int32_t *row = block_tables + (int64_t)s * block_table_stride;
            std::memcpy(bt + (int64_t)s * p->bt_stride, row, sizeof(int32_t) * p->bt_stride);
            for (int32_t i = 0; i < q_lens[s]; ++i) {
                const int64_t pos = (int64_t)nc[s] + i;
                slot[qsl[s] + i] = row[pos / PS_BLOCK] * PS_BLOCK + (int32_t)(pos % PS_BLOCK);
                posn[qsl[s] + i] = (int32_t)pos;
            }
        }
        for (int64_t s = S; s < cap_S; ++s) qsl[s + 1] = (int32_t)T;   // fixed shape: unused tail
        for (int64_t t = T; t < cap_T; ++t) slot[t] = -1;               // (skipped by any scatter)
        if (!dec.empty()) std::memcpy(p->host<ps_item>(p->off_dec), dec.data(), sizeof(ps_item) * dec.size());
        if (!pre.empty()) std::memcpy(p->host<ps_item>(p->off_pre), pre.data(), sizeof(ps_item) * pre.size());
        if (!mrg.empty()) std::memcpy(p->host<ps_merge>(p->off_mrg), mrg.data(), sizeof(ps_merge) * mrg.size());
        if (!rmap.empty()) std::memcpy(p->host<ps_row>(p->off_rmap), rmap.data(), sizeof(ps_row) * rmap.size());
        // decode items' first tiles in walk order: tile t covers keys
        // key_begin + 32 u .. +32, u = (t + rot) mod ntiles; a tile's second
        // block past key_end repeats the first (never read). A wave of an
        // item of NW waves takes its first tiles, t = wave and wave + NW,
        // from here: entries from 2 NW on are never read and stay zero.
        int32_t *dh = p->host<int32_t>(p->off_dhead);
        const int32_t head_tiles = std::min<int32_t>(PS_DEC_HEAD_TILES, 2 * p->dec_waves);
        static_assert(PS_DEC_TILE == 2 * PS_BLOCK, "a decode tile spans two blocks");
        for (size_t i = 0; i < (size_t)act_dec; ++i) {
            const ps_item &it = dec[i];
            // (decode slices start on block boundaries)
            const int32_t *blk = block_tables + (int64_t)it.seq * block_table_stride + it.key_begin / PS_BLOCK;
            const int32_t len = it.key_end - it.key_begin;
            const int32_t ntiles = (len + PS_DEC_TILE - 1) / PS_DEC_TILE;
            const int32_t n = std::min<int32_t>(ntiles, head_tiles);
            int32_t *d = dh + i * 2 * PS_DEC_HEAD_TILES;
            int32_t u = it.rot;
            for (int32_t t = 0; t < n; ++t) {
                const int32_t b0 = blk[2 * u];
                d[2 * t] = b0;
                d[2 * t + 1] = PS_DEC_TILE * u + PS_BLOCK < len ? blk[2 * u + 1] : b0;
                u = u + 1 == ntiles ? 0 : u + 1;
            }
        }
        p->kinds.resize(S);
        for (int32_t s = 0; s < S; ++s) p->kinds[s] = !is_dec[s] ? 1 : grp_of[s] >= 0 ? 2 : 0;

        // ---- algorithmic accounting and the planner's choices
        ps_plan_info &I = p->info;
        I.num_seqs = S;
        I.num_tokens = (int32_t)T;
        I.num_q_heads = num_q_heads;
        I.num_kv_heads = Hkv;
        I.head_dim = D;
        I.dtype = pool->dtype;
        I.decode_items = p->n_dec;
        I.prefill_items = p->n_pre;
        I.prefix_items = n_gathered;
        I.prefix_groups = (int32_t)grp_lead.size();
        I.step_fused = p->n_pre == n_gathered && p->n_dec > 0;
        I.merge_items = p->n_mrg;
        I.decode_row_tiles = dec_rt;
        I.flags = (int32_t)flags;
        I.decode_split_keys = (int32_t)dec_split;
        I.prefill_split_keys = (int32_t)pre_split;
        I.decode_waves = p->dec_waves;
        I.mixed_launch = p->mixed;
        I.decode_walk_rotation = p->rotate ? 1 : 0;
        I.decode_stream_kv = p->stream_kv ? 1 : 0;
        I.active_decode_items = act_dec;
        I.active_merge_items = act_mrg;
        I.workspace_rows = cap_ws;
        const int64_t e = elt_bytes(pool->dtype);
        const int64_t row_kv = 2 * (int64_t)D * e;  // K + V bytes of one (token, KV head)
        for (int32_t s = 0; s < S; ++s) {
            const int64_t n = q_lens[s], c = num_computed_tokens[s], ctx = c + n;
            const int64_t kvb = ctx * Hkv * row_kv;
            const double fl = 4.0 * D * num_q_heads * ((double)n * c + 0.5 * (double)n * (n + 1));
            if (is_dec[s]) { I.decode_seqs++; I.kv_bytes_decode += kvb; I.flops_decode += fl; }
            else { I.prefill_seqs++; I.kv_bytes_prefill += kvb; I.flops_prefill += fl; }
            I.table_bytes += 4 * ceil_div(ctx, PS_BLOCK);
        }
        // unique: each physical block once, with the most tokens any sharer reads
        I.kv_bytes_unique = kv_rows_unique * Hkv * row_kv;
        I.q_bytes = T * num_q_heads * D * e;
        I.out_bytes = I.q_bytes;
        I.scatter_bytes = 2 * (T * Hkv * D * e) * 2 + 4 * T;
    } catch (const std::bad_alloc &) {
        delete p;
        return ps_fail(PS_ERR_HOST_MEMORY, "host allocation failed");
    }
    p->info.plan_us = std::chrono::duration<double, std::micro>(std::chrono::steady_clock::now() - t_start).count();
    *out_plan = p;
    return PS_OK;
}

extern "C" ps_status ps_plan_sizes(const ps_plan *plan, size_t *metadata_bytes, size_t *workspace_bytes) {
    if (!plan) return ps_fail(PS_ERR_INVALID_ARGUMENT, "plan is NULL");
    if (metadata_bytes) *metadata_bytes = plan->blob.size();
    if (workspace_bytes) *workspace_bytes = ps_workspace_layout(plan->ws_rows, plan->D).bytes;
    return PS_OK;
}

extern "C" ps_status ps_plan_upload(ps_plan *plan, void *metadata_dev, size_t metadata_bytes, void *stream) {
    if (!plan) return ps_fail(PS_ERR_INVALID_ARGUMENT, "plan is NULL");
    if (!metadata_dev) return ps_fail(PS_ERR_INVALID_ARGUMENT, "metadata_dev is NULL");
    if (((uintptr_t)metadata_dev & 255) != 0)
        return ps_fail(PS_ERR_INVALID_ARGUMENT, "metadata_dev is not 256-byte aligned");
    if (metadata_bytes < plan->blob.size())
        return ps_fail(PS_ERR_INVALID_ARGUMENT, "metadata buffer holds %zu bytes, plan needs %zu",
                       metadata_bytes, plan->blob.size());
    hipError_t e = hipMemcpyAsync(metadata_dev, plan->blob.data(), plan->blob.size(),
                                  hipMemcpyHostToDevice, (hipStream_t)stream);
    if (e != hipSuccess) return ps_fail(PS_ERR_HIP, "hipMemcpyAsync: %s", hipGetErrorString(e));
    plan->dev = metadata_dev;
    return PS_OK;
}

static void fill_arrays(const ps_plan *p, const uint8_t *base, ps_step_arrays *a) {
    a->slot_mapping = reinterpret_cast<const int32_t *>(base + p->off_slot);
    a->block_tables = reinterpret_cast<const int32_t *>(base + p->off_bt);
    a->block_table_stride = p->bt_stride;
    a->query_start_loc = reinterpret_cast<const int32_t *>(base + p->off_qsl);
    a->num_computed_tokens = reinterpret_cast<const int32_t *>(base + p->off_nc);
    a->context_lens = reinterpret_cast<const int32_t *>(base + p->off_ctx);
    a->positions = reinterpret_cast<const int32_t *>(base + p->off_pos);
}

extern "C" ps_status ps_plan_device_arrays(const ps_plan *plan, ps_step_arrays *arrays) {
    if (!plan || !arrays) return ps_fail(PS_ERR_INVALID_ARGUMENT, "plan or arrays is NULL");
    if (!plan->dev) return ps_fail(PS_ERR_INVALID_ARGUMENT, "plan has not been uploaded");
    fill_arrays(plan, static_cast<const uint8_t *>(plan->dev), arrays);
    return PS_OK;
}

extern "C" ps_status ps_plan_host_arrays(const ps_plan *plan, ps_step_arrays *arrays) {
    if (!plan || !arrays) return ps_fail(PS_ERR_INVALID_ARGUMENT, "plan or arrays is NULL");
    fill_arrays(plan, plan->blob.data(), arrays);
    return PS_OK;
}

extern "C" ps_status ps_plan_get_info(const ps_plan *plan, ps_plan_info *info) {
    if (!plan || !info) return ps_fail(PS_ERR_INVALID_ARGUMENT, "plan or info is NULL");
    *info = plan->info;
    return PS_OK;
}

extern "C" ps_status ps_plan_sequence_kernels(const ps_plan *plan, int32_t *kinds, int32_t num_seqs) {
    if (!plan) return ps_fail(PS_ERR_INVALID_ARGUMENT, "plan is NULL");
    if (num_seqs != plan->S) return ps_fail(PS_ERR_INVALID_ARGUMENT, "num_seqs %d, plan has %d", num_seqs, plan->S);
    if (num_seqs > 0 && !kinds) return ps_fail(PS_ERR_INVALID_ARGUMENT, "kinds is NULL");
    if (num_seqs > 0) std::memcpy(kinds, plan->kinds.data(), sizeof(int32_t) * (size_t)num_seqs);
    return PS_OK;
}

extern "C" void ps_plan_destroy(ps_plan *plan) { delete plan; }

// ---------------------------------------------------------------------------
// ps_paged_attention: argument checks against the plan, then the launches.

// Argument checks against the plan and the launch record; *empty is set
// for a step without tokens (nothing to launch).
static ps_status prepare_attention(const void *q, const ps_pool *pool, const int32_t *block_tables,
                                   int32_t block_table_stride, const int32_t *query_start_loc,
                                   const int32_t *num_computed_tokens, const int32_t *context_lens,
                                   void *out, int32_t num_seqs, int32_t num_tokens, int32_t num_q_heads,
                                   float scale, const ps_plan *plan, void *workspace,
                                   size_t workspace_bytes, ps_attn_launch &a, bool *empty) {
    *empty = false;
    if (!plan) return ps_fail(PS_ERR_INVALID_ARGUMENT, "plan is NULL");
    if (!pool) return ps_fail(PS_ERR_INVALID_ARGUMENT, "pool is NULL");
    if (num_seqs != plan->S || num_tokens != plan->T || num_q_heads != plan->Hq)
        return ps_fail(PS_ERR_INVALID_ARGUMENT,
                       "call sizes (S=%d, T=%d, Hq=%d) differ from the plan's (S=%d, T=%d, Hq=%d)",
                       num_seqs, num_tokens, num_q_heads, plan->S, plan->T, plan->Hq);
    if (pool->num_kv_heads != plan->Hkv || pool->head_dim != plan->D || pool->dtype != plan->dtype ||
        pool->num_blocks != plan->num_blocks || pool->num_layers != plan->num_layers ||
        pool->block_size != PS_BLOCK)
        return ps_fail(PS_ERR_INVALID_ARGUMENT, "pool geometry differs from the plan's");
    if (pool->layer < 0 || pool->layer >= pool->num_layers)
        return ps_fail(PS_ERR_INVALID_ARGUMENT, "layer %d outside [0, %d)", pool->layer, pool->num_layers);
    if ((num_seqs > 0 || plan->fixed) && block_table_stride != plan->bt_stride)
        return ps_fail(PS_ERR_INVALID_ARGUMENT, "block_table_stride %d differs from the plan's %d",
                       block_table_stride, plan->bt_stride);
    if (!(scale > 0.0f) || !(scale < 1e30f))
        return ps_fail(PS_ERR_INVALID_ARGUMENT, "scale must be positive and finite");
    const ps_ws_layout wl = ps_workspace_layout(plan->ws_rows, plan->D);
    if (workspace_bytes < wl.bytes)
        return ps_fail(PS_ERR_WORKSPACE_TOO_SMALL, "workspace holds %zu bytes, step needs %zu",
                       workspace_bytes, wl.bytes);
    if (wl.bytes > 0 && (!workspace || ((uintptr_t)workspace & 255)))
        return ps_fail(PS_ERR_INVALID_ARGUMENT, "workspace is NULL or not 256-byte aligned");
    if (!plan->dev) return ps_fail(PS_ERR_INVALID_ARGUMENT, "plan has not been uploaded");
    if (num_tokens == 0 && !plan->fixed) {
        *empty = true;
        return PS_OK;
    }
    if (!q || !out || !pool->k || !pool->v || !block_tables || !query_start_loc ||
        !num_computed_tokens || !context_lens)
        return ps_fail(PS_ERR_INVALID_ARGUMENT, "a device pointer is NULL");

    a = ps_attn_launch{};
    a.q = q;
    a.out = out;
    a.pool_k = pool->k;
    a.pool_v = pool->v;
    a.block_tables = block_tables;
    a.query_start_loc = query_start_loc;
    a.num_computed = num_computed_tokens;
    a.context_lens = context_lens;
    const uint8_t *dev = static_cast<const uint8_t *>(plan->dev);
    a.decode_items = reinterpret_cast<const ps_item *>(dev + plan->off_dec);
    a.prefill_items = reinterpret_cast<const ps_item *>(dev + plan->off_pre);
    a.merges = reinterpret_cast<const ps_merge *>(dev + plan->off_mrg);
    // the items' first block ids are copies of the plan's table: usable only
    // when the call reads that very table
    const int32_t *plan_bt = reinterpret_cast<const int32_t *>(dev + plan->off_bt);
    a.decode_head = reinterpret_cast<const int32_t *>(dev + plan->off_dhead);
    a.head_ok = block_tables == plan_bt;
    a.row_map = reinterpret_cast<const ps_row *>(dev + plan->off_rmap);
    uint8_t *ws = static_cast<uint8_t *>(workspace);
    a.ws_m = wl.bytes ? reinterpret_cast<float *>(ws + wl.off_m) : nullptr;
    a.ws_l = wl.bytes ? reinterpret_cast<float *>(ws + wl.off_l) : nullptr;
    a.ws_acc = wl.bytes ? reinterpret_cast<float *>(ws + wl.off_acc) : nullptr;
    a.layer_offset = (int64_t)pool->layer * pool->num_blocks * PS_BLOCK * pool->num_kv_heads * pool->head_dim;
    a.bt_stride = plan->bt_stride;
    a.num_blocks = plan->num_blocks;
    // a fixed shape's launch must not depend on this step's token count:
    // its q and out hold max_tokens rows
    a.num_tokens = std::max(1, plan->fixed ? plan->rows_cap : num_tokens);
    a.num_q_heads = plan->Hq;
    a.num_kv_heads = plan->Hkv;
    a.head_dim = plan->D;
    a.dtype = plan->dtype;
    a.n_decode = plan->n_dec;
    a.n_prefill = plan->n_pre;
    a.n_merge = plan->n_mrg;
    a.decode_row_tiles = plan->dec_rt;
    a.decode_waves = plan->dec_waves;
    a.mixed = plan->mixed;
    a.stream_kv = plan->stream_kv ? 1 : 0;
    a.scale_log2 = scale * 1.4426950408889634f;
    a.g = plan->Hq / plan->Hkv;
    ps_group_divisor(a.g, &a.g_magic, &a.g_shift);
    a.num_slots = plan->num_blocks * PS_BLOCK;
    return PS_OK;
}

extern "C" ps_status ps_paged_attention(const void *q, const ps_pool *pool,
                                        const int32_t *block_tables, int32_t block_table_stride,
                                        const int32_t *query_start_loc,
                                        const int32_t *num_computed_tokens,
                                        const int32_t *context_lens, void *out,
                                        int32_t num_seqs, int32_t num_tokens, int32_t num_q_heads,
                                        float scale, const ps_plan *plan,
                                        void *workspace, size_t workspace_bytes, void *stream) {
    ps_attn_launch a;
    bool empty;
    const ps_status st = prepare_attention(q, pool, block_tables, block_table_stride, query_start_loc,
                                           num_computed_tokens, context_lens, out, num_seqs, num_tokens,
                                           num_q_heads, scale, plan, workspace, workspace_bytes, a, &empty);
    if (st != PS_OK || empty) return st;
    const int err = ps_launch_attention(a, stream);
    if (err != 0) return ps_fail(PS_ERR_HIP, "attention launch: %s", ps_hip_error_string(err));
    return PS_OK;
}

extern "C" ps_status ps_step(const void *q, const void *k, const void *v, const int32_t *slot_mapping,
                             const ps_pool *pool, const int32_t *block_tables, int32_t block_table_stride,
                             const int32_t *query_start_loc, const int32_t *num_computed_tokens,
                             const int32_t *context_lens, void *out, int32_t num_seqs, int32_t num_tokens,
                             int32_t num_q_heads, float scale, const ps_plan *plan, void *workspace,
                             size_t workspace_bytes, void *stream) {
    ps_attn_launch a;
    bool empty;
    ps_status st = prepare_attention(q, pool, block_tables, block_table_stride, query_start_loc,
                                     num_computed_tokens, context_lens, out, num_seqs, num_tokens,
                                     num_q_heads, scale, plan, workspace, workspace_bytes, a, &empty);
    if (st != PS_OK || empty) return st;
    if (!k || !v || !slot_mapping) return ps_fail(PS_ERR_INVALID_ARGUMENT, "k, v or slot_mapping is NULL");
    if (plan->n_pre == plan->n_gathered && plan->n_dec > 0) {
        // every sequence on the decode kernel (shared-prefix items read
        // only blocks below every member's new tokens): the scatter rides
        // along
        a.fuse_scatter = 1;
        a.k_new = k;
        a.v_new = v;
        a.slot_mapping = slot_mapping;
    } else {
        st = ps_reshape_and_cache(k, v, slot_mapping, num_tokens, pool, stream);
        if (st != PS_OK) return st;
    }
    const int err = ps_launch_attention(a, stream);
    if (err != 0) return ps_fail(PS_ERR_HIP, "step launch: %s", ps_hip_error_string(err));
    return PS_OK;
}

extern "C" ps_status ps_step_no_alloc(const void *q, const void *k, const void *v, const int32_t *slot_mapping,
                                      const ps_pool *pool, const int32_t *block_tables,
                                      int32_t block_table_stride, const int32_t *query_start_loc,
                                      const int32_t *num_computed_tokens, const int32_t *context_lens, void *out,
                                      int32_t num_seqs, int32_t num_tokens, int32_t num_q_heads, float scale,
                                      const ps_plan *plan, void *stream) {
    if (!plan) return ps_fail(PS_ERR_INVALID_ARGUMENT, "plan is NULL");
    const size_t need = ps_workspace_layout(plan->ws_rows, plan->D).bytes;
    if (need > PS_STATIC_WORKSPACE_BYTES)
        return ps_fail(PS_ERR_WORKSPACE_TOO_SMALL,
                       "step needs %zu bytes of split-K workspace, the static workspace holds %zu "
                       "(plan longer key splits)", need, (size_t)PS_STATIC_WORKSPACE_BYTES);
    void *ws = nullptr;
    if (need > 0) {
        const int err = ps_static_workspace(&ws);
        if (err != 0) return ps_fail(PS_ERR_HIP, "static workspace: %s", ps_hip_error_string(err));
    }
    return ps_step(q, k, v, slot_mapping, pool, block_tables, block_table_stride, query_start_loc,
                   num_computed_tokens, context_lens, out, num_seqs, num_tokens, num_q_heads, scale, plan, ws,
                   need, stream);
}
