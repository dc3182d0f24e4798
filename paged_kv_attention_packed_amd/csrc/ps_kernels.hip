// HIP kernels for one packed paged-attention step on gfx950 (CDNA4).
//
//  * ps_scatter_kernel   — writes the step's new K/V rows into the block
//                          pool at their slots (PageServe "03 Paged KV
//                          cache": scatters new K/V into those slots).
//  * ps_decode_kernel    — decode and speculative-verify rows: split-K over
//                          the context, K/V streamed from HBM straight into
//                          MFMA operand registers, online softmax.
//  * ps_prefill_kernel   — prefill chunks: 128 packed rows per workgroup,
//                          64-key K/V tiles gathered through the block table
//                          into LDS, QK^T and PV on MFMA, causal diagonal at
//                          the chunk's offset.
//  * ps_merge_kernel     — log-sum-exp merge of split-K partials.
//
// MFMA mapping (both attention kernels). A wave works on 16-row tiles of
// "packed rows" (query token x head in the KV head's group), so the g query
// heads that share a KV head share each K/V load. Scores are formed
// transposed, S^T = K Q^T, with v_mfma_f32_16x16x32_{f16,bf16} (fp32 data:
// v_mfma_f32_16x16x4f32): lane (c = lane % 16, q = lane / 16) supplies key
// c's d-range [q*D/4, (q+1)*D/4) and receives S^T[keys 4q..4q+3][row c].
// Each lane therefore owns one query row: its softmax state is lane-local
// and only the row max needs a 4-lane exchange. The output is formed as
// O^T = V^T P^T, whose B operand (P^T) is exactly the score fragment a lane
// already holds (two 16-key tiles give the 8 k-slots 4q..4q+3, 16+4q..19+4q);
// the A operand takes V rows of those same 8 keys, lane c holding the
// d-range [c*D/16, (c+1)*D/16) so each V row is one contiguous 8- or 16-byte
// load, and tile t of O^T holds d = (D/16) * row + t.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cstdlib>
#include <mutex>
#include <type_traits>

#include "ps_internal.h"

namespace psk {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kNegInf = -__builtin_huge_valf();

struct TF32 {
    using T = float;
    static constexpr int ELT = 4;
};
struct TF16 {
    using T = _Float16;
    static constexpr int ELT = 2;
};
struct TBF16 {
    using T = __bf16;
    static constexpr int ELT = 2;
};

// fp32 -> storage type, round to nearest even
__device__ inline float cvt_out(float x, TF32) { return x; }
__device__ inline _Float16 cvt_out(float x, TF16) { return (_Float16)x; }
__device__ inline __bf16 cvt_out(float x, TBF16) { return (__bf16)x; }

// two fp32 -> packed pair of 16-bit values (low half = first), round to
// nearest even: one v_cvt_pk_{f16,bf16}_f32
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ inline uint32_t pack2(float x, float y, TF16) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){x, y}, f16x2));
}
__device__ inline uint32_t pack2(float x, float y, TBF16) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){x, y}, bf16x2));
}

__device__ inline f32x4 mfma32(u32x4 a, u32x4 b, f32x4 c, TF16) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}
__device__ inline f32x4 mfma32(u32x4 a, u32x4 b, f32x4 c, TBF16) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
__device__ inline f32x4 mfma4(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Reductions over the 4 lanes l, l^16, l^32, l^48 (one packed row) with
// the gfx950 row-swap permutes: permlane16_swap(x, x) leaves the pair
// {x[l], x[l ^ 16]} in its two results, permlane32_swap the pair
// {x[l], x[l ^ 32]}; both are VALU operations, unlike a ds_bpermute.
__device__ inline void swap_pair16(float x, float &a, float &b) {
    const auto r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(uint32_t, x),
                                                    __builtin_bit_cast(uint32_t, x), false, false);
    const uint32_t r0 = r[0], r1 = r[1];
    a = __builtin_bit_cast(float, r0);
    b = __builtin_bit_cast(float, r1);
}
__device__ inline void swap_pair32(float x, float &a, float &b) {
    const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x),
                                                    __builtin_bit_cast(uint32_t, x), false, false);
    const uint32_t r0 = r[0], r1 = r[1];
    a = __builtin_bit_cast(float, r0);
    b = __builtin_bit_cast(float, r1);
}
// (max(a, b) as the median of a, b and FLT_MAX: the same value unless an
// operand is +inf or NaN, i.e. an overflowed score, whose softmax has no
// finite value either way. fmaxf would first quiet its operands, two more
// VALU ops each time, since the swap results come from integer
// operations; the reduction runs for every row tile of every key tile.)
__device__ inline float max2(float a, float b) { return __builtin_amdgcn_fmed3f(a, b, 3.4028234663852886e38f); }
__device__ inline float xor_max(float x) {
    float a, b;
    swap_pair16(x, a, b);
    swap_pair32(max2(a, b), a, b);
    return max2(a, b);
}
__device__ inline float xor_sum(float x) {
    float a, b;
    swap_pair16(x, a, b);
    swap_pair32(a + b, a, b);
    return a + b;
}

// A vector load; STREAM: marked non-temporal (streamed past the caches' normal
// allocation: for data the step reads once)
template <bool STREAM, class V>
__device__ inline V load_vec(const V *p) {
    if constexpr (STREAM) return __builtin_nontemporal_load(p);
    else return *p;
}

// N consecutive 32-bit words from a 4*N-byte aligned address
template <int N, bool STREAM = false>
__device__ inline void load_words(const void *p, uint32_t (&w)[N]) {
    if constexpr (N == 2) {
        const u32x2 x = load_vec<STREAM>(reinterpret_cast<const u32x2 *>(p));
        w[0] = x[0];
        w[1] = x[1];
    } else {
        static_assert(N % 4 == 0, "word count");
#pragma unroll
        for (int i = 0; i < N / 4; ++i) {
            const u32x4 x = load_vec<STREAM>(reinterpret_cast<const u32x4 *>(p) + i);
            w[4 * i + 0] = x[0];
            w[4 * i + 1] = x[1];
            w[4 * i + 2] = x[2];
            w[4 * i + 3] = x[3];
        }
    }
}

template <class DT, int D>
struct Geo {
    static constexpr int ELT = DT::ELT;
    static constexpr int KU4 = D * ELT / 64;   // 16-byte words of a lane's K (and Q) d-range
    static constexpr int EPL = D / 16;         // V elements a lane takes from each key row
    static constexpr int VW = EPL * ELT / 4;   // ... as 32-bit words
    static constexpr int NT = D / 16;          // 16-wide d tiles of the output
};

// S^T tile (16 keys x 16 rows) = K_frag . Q_frag^T over the full head dim
template <class DT, int D>
__device__ inline f32x4 qk_tile(const u32x4 (&kf)[Geo<DT, D>::KU4], const u32x4 (&qf)[Geo<DT, D>::KU4]) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < Geo<DT, D>::KU4; ++u) {
        if constexpr (DT::ELT == 2) {
            acc = mfma32(kf[u], qf[u], acc, DT{});
        } else {
            const f32x4 kv = __builtin_bit_cast(f32x4, kf[u]);
            const f32x4 qv = __builtin_bit_cast(f32x4, qf[u]);
            acc = mfma4(kv.x, qv.x, acc);
            acc = mfma4(kv.y, qv.y, acc);
            acc = mfma4(kv.z, qv.z, acc);
            acc = mfma4(kv.w, qv.w, acc);
        }
    }
    return acc;
}

// A operand of O^T tile t from 8 V rows (16-bit types): element j = row j's
// element t
template <int VW>
__device__ inline u32x4 v_operand(const uint32_t (&vr)[8][VW], int t) {
    const int w = t >> 1;
    const uint32_t sel = (t & 1) ? 0x07060302u : 0x05040100u;
    u32x4 a;
    a[0] = __builtin_amdgcn_perm(vr[1][w], vr[0][w], sel);
    a[1] = __builtin_amdgcn_perm(vr[3][w], vr[2][w], sel);
    a[2] = __builtin_amdgcn_perm(vr[5][w], vr[4][w], sel);
    a[3] = __builtin_amdgcn_perm(vr[7][w], vr[6][w], sel);
    return a;
}

// Online-softmax update of one row tile from NS raw scores per lane
// (masked scores are -inf). `c` = softmax scale * log2(e); m is the
// reference max in log2 units, l the running denominator; on return sv
// holds exp2(c * s - m). The reference only moves when some row's max
// grows by more than 2^8 (then the accumulators are rescaled): the
// numerator and denominator always share one reference, so the result is
// the same softmax, with probabilities bounded by 256, and steady-state
// tiles skip the rescale entirely. All row tiles of the wave share one
// decision, so the rescale is a single uniform branch.
constexpr float kLazyRescale = 8.f;

// SUM = false: the caller accumulates the row sums itself (the prefill
// kernel does it on MFMA, as an extra all-ones column tile of o).
template <int RT, int NS, int NT, bool SUM = true>
__device__ inline void softmax_update(float (&sv)[RT][NS], float c, float (&m)[RT], float (&l)[RT],
                                      f32x4 (&o)[RT][NT]) {
    float tmax[RT];
    bool grow = false;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        float x = kNegInf;
#pragma unroll
        for (int e = 0; e < NS; ++e) x = fmaxf(x, sv[rt][e]);
        tmax[rt] = xor_max(x) * c;
        grow = grow || tmax[rt] > m[rt] + kLazyRescale;
    }
    if (__any(grow)) {  // one wave-uniform decision for all row tiles
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            const float mnew = fmaxf(m[rt], tmax[rt]);
            const float alpha = fast_exp2(m[rt] - (mnew == kNegInf ? 0.f : mnew));
            l[rt] *= alpha;
            m[rt] = mnew;
#pragma unroll
            for (int t = 0; t < NT; ++t) o[rt][t] *= alpha;
        }
    }
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        const float muse = m[rt] == kNegInf ? 0.f : m[rt];
        float psum = 0.f;
#pragma unroll
        for (int e = 0; e < NS; ++e) {
            sv[rt][e] = fast_exp2(__builtin_fmaf(sv[rt][e], c, -muse));
            if constexpr (SUM) psum += sv[rt][e];
        }
        if constexpr (SUM) l[rt] += psum;
    }
}

// r / g for 0 <= r < 2^31 (g = num_q_heads / num_kv_heads): a multiply
// and a shift with constants the host derived.
__device__ inline int div_g(const ps_attn_launch &a, int r) {
    return (int)(((uint64_t)(uint32_t)r * a.g_magic) >> a.g_shift);
}

// Packed token `local` of a sequence whose first token is qs0, clamped
// into [0, num_tokens): with arrays that keep the call's contract the
// clamp changes nothing; with others every access stays inside q, out, k
// and v.
__device__ inline int tok_index(const ps_attn_launch &a, int qs0, int local) {
    return min(max(qs0 + local, 0), a.num_tokens - 1);
}

// A block id read from the call's table, clamped into the pool.
__device__ inline int64_t clamp_blk(const ps_attn_launch &a, int32_t id) {
    return (int64_t)min((uint32_t)id, (uint32_t)(a.num_blocks - 1));
}

// What a work item needs about its sequence, from the call's own arrays:
// first packed row, tokens already in the pool, context length.
struct SeqInfo {
    int qs0, nc, ctx;
};
__device__ inline SeqInfo seq_info(const ps_attn_launch &a, int s) {
    return SeqInfo{a.query_start_loc[s], a.num_computed[s], a.context_lens[s]};
}

// Which query row a lane's packed row stands for, its visibility limit and
// its Q fragment.
// A row past the item's end (r >= row_end) loads the item's last row
// instead and gets lim = -1: where its keys are masked it sees none, where
// they are not its results are finite and never stored. Loading it
// unconditionally keeps the loads out of a branch whose other side would
// write the same registers, which would make the compiler wait for them
// (and for everything issued before them) on the spot.
// A row sees key tau iff tau <= nc + (its token) and tau < ctx.
template <class DT, int D>
__device__ inline void load_q_row(const ps_attn_launch &a, int r, int row_end, int g, int kv_head,
                                  const SeqInfo &si, int q4, u32x4 (&qf)[Geo<DT, D>::KU4], int &lim) {
    const bool ok = r < row_end;
    const int rr = ok ? r : row_end - 1;
    const int tok = div_g(a, rr);
    const int h = kv_head * g + (rr - tok * g);
    lim = ok ? min(si.nc + tok, si.ctx - 1) : -1;
    const typename DT::T *qp =
        static_cast<const typename DT::T *>(a.q) + ((int64_t)tok_index(a, si.qs0, tok) * a.num_q_heads + h) * D;
#pragma unroll
    for (int u = 0; u < Geo<DT, D>::KU4; ++u)
        qf[u] = *reinterpret_cast<const u32x4 *>(qp + (u * 4 + q4) * (16 / DT::ELT));
}

// ---------------------------------------------------------------------------
// Waits. A bare s_barrier with explicit s_waitcnt: a fenced barrier would
// also wait for global loads still in flight.

template <int N>
__device__ inline void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// all waves reach this point with their LDS reads complete
__device__ inline void lds_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// ---------------------------------------------------------------------------
// KV scatter: one thread per 16 bytes of a token's K (and V) row.

__global__ __launch_bounds__(256) void ps_scatter_kernel(const u32x4 *__restrict__ k,
                                                         const u32x4 *__restrict__ v,
                                                         const int32_t *__restrict__ slots,
                                                         int64_t total, int32_t row_words,
                                                         u32x4 *__restrict__ pk, u32x4 *__restrict__ pv,
                                                         int32_t num_slots) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= total) return;
    const int64_t t = i / row_words;
    const int32_t w = (int32_t)(i - t * row_words);
    const int32_t slot = slots[t];
    if ((uint32_t)slot >= (uint32_t)num_slots) return;
    const int64_t dst = (int64_t)slot * row_words + w;
    pk[dst] = k[i];
    pv[dst] = v[i];
}

// ---------------------------------------------------------------------------
// Block copy (copy-on-write, swap out / in): one workgroup per (pair,
// layer) moves that layer's K and V block, 16 bytes per thread per step.

__global__ __launch_bounds__(256) void ps_copy_blocks_kernel(const u32x4 *__restrict__ sk,
                                                             const u32x4 *__restrict__ sv,
                                                             u32x4 *__restrict__ dk, u32x4 *__restrict__ dv,
                                                             const int32_t *__restrict__ src_ids,
                                                             const int32_t *__restrict__ dst_ids,
                                                             int32_t num_layers, int32_t src_blocks,
                                                             int32_t dst_blocks, int32_t block_words) {
    const int pair = blockIdx.x / num_layers;
    const int layer = blockIdx.x - pair * num_layers;
    const int32_t s = src_ids[pair], d = dst_ids[pair];
    if ((uint32_t)s >= (uint32_t)src_blocks || (uint32_t)d >= (uint32_t)dst_blocks) return;
    const int64_t so = ((int64_t)layer * src_blocks + s) * block_words;
    const int64_t do_ = ((int64_t)layer * dst_blocks + d) * block_words;
    for (int w = threadIdx.x; w < block_words; w += 256) {
        const u32x4 a = sk[so + w];
        const u32x4 b = sv[so + w];
        dk[do_ + w] = a;
        dv[do_ + w] = b;
    }
}

// ---------------------------------------------------------------------------
// Decode / verify attention. One workgroup = one work item (sequence, KV
// head, <= RT*16 packed rows, key slice). Its 4 waves take 32-key tiles of
// the slice round-robin, each double-buffering the next tile's K/V in
// registers, then merge their softmax states through LDS.

// one 16-byte global -> LDS DMA per lane; lane l lands at lds + 16 * l
// Issued as inline asm: the compiler cannot tell which LDS bytes a DMA in
// flight will write, so for the builtin (or an asm that clobbers memory) it
// waits for every DMA in flight, the next tiles' too, before each LDS read.
// Ordering is explicit instead: wait_vmcnt for this thread's DMAs, then
// lds_barrier (whose asm does clobber memory) for everyone's. m0 holds the
// LDS destination; nothing else on gfx950 reads it.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"  // m0 is a reserved register: the clobber is the point
template <bool STREAM = false>
__device__ inline void dma16(const void *src, uint8_t *lds) {
#if defined(__HIP_DEVICE_COMPILE__)
    const uint32_t off = __builtin_amdgcn_readfirstlane(
        (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t *)lds);
    if constexpr (STREAM)
        asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off nt" ::"v"(src), "s"(off) : "m0");
    else
        asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(off) : "m0");
#endif
}
// Same, addressed as a scalar base plus a 32-bit per-lane byte offset.
template <bool STREAM = false>
__device__ inline void dma16_sv(const void *base, uint32_t voff, uint32_t lds_off) {
#if defined(__HIP_DEVICE_COMPILE__)
    if constexpr (STREAM)
        asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1 nt" ::"v"(voff), "s"(base), "s"(lds_off) : "m0");
    else
        asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(base), "s"(lds_off) : "m0");
#endif
}
#pragma clang diagnostic pop

// 16-byte chunk position of `chunk` in key row `row`: XOR-swizzled so that
// the operand reads of a tile do not pile onto a few LDS banks.
//
// 256-byte (and longer) rows: chunk ^ f(row), f(r) = (r ^ 2r) mod 16, an
// invertible XOR-linear map of row % 16. Three read shapes use these rows:
// one chunk of 16 rows per 16 lanes (K operands, ds_read_b128), 8 bytes of
// 2 adjacent chunks of 4 adjacent rows per 16 lanes (V operands, transposing
// reads) and whole rows per 16 lanes (V rows of the decode kernel). gfx950's
// lane-to-bank pairing for these reads is not documented; timed on MI355X
// (one 64-row tile read over and over, 4 workgroups per CU), this f runs all
// three at 440-490 B/ns per CU, where the row-XOR keys tried besides it
// (r, (r mod 8) << 1 with bit 3 in bit 0, no swizzle, and others) leave at
// least one of them at 290-300 or below.
template <int ROWB>
__device__ inline int swz(int chunk, int row) {
    if constexpr (ROWB >= 256) return chunk ^ ((row ^ (row << 1)) & 15);
    else return chunk ^ ((row >> 1) & 7);  // 128-byte rows: two rows share 256 bytes
}

// NW waves per workgroup: more waves cover a short key slice in one round
// trip (each wave takes every NW-th 32-key tile); the register budget
// allows 2 waves per SIMD up to 8 waves and 4 per SIMD at 16.
template <class DT, int D, int RT, int NW>
struct DecodeLds {
    float o[NW][RT * 16][D];   // per-wave partial outputs, merged at the end
    float m[NW][RT * 16];
    float l[NW][RT * 16];
    int32_t bt[PS_DEC_MAX_SPLIT / PS_BLOCK];  // the item's block ids
};

// STREAM: the item's K/V loads from the pool are non-temporal (the planner's
// choice for steps that read each block once and more than the caches hold).
// FUSE: the launch may carry the fused scatter (a.fuse_scatter); without it
// the scatter's code and registers are compiled out.
template <class DT, int D, int RT, int NW, bool STREAM, bool FUSE = true>
__device__ __forceinline__ void decode_item(const ps_attn_launch a, int item, DecodeLds<DT, D, RT, NW> &sh) {
    using G = Geo<DT, D>;
    using T = typename DT::T;
    constexpr int ELT = G::ELT, KU4 = G::KU4, VW = G::VW, NT = G::NT, EPL = G::EPL;
    constexpr int ROWS = RT * 16;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: keeps tile math scalar
    // The item, the block ids of the wave's first tiles and the launch's
    // arguments, all needed before the first K/V load: the empty asm takes
    // them as operands, so their scalar loads are issued together and
    // waited for once instead of at first uses scattered over the prologue
    // (scalar loads return out of order: every wait is a wait for all).
    // It comes after the loads: a volatile asm counts as a possible memory
    // write, and loads after it would not be scalar loads.
    const ps_item it = a.decode_items[item];
    const int2 *head = reinterpret_cast<const int2 *>(a.decode_head) + (int64_t)item * PS_DEC_HEAD_TILES;
    const int2 hid0 = head[wave];
    const int2 hid1 = head[min(wave + NW, PS_DEC_HEAD_TILES - 1)];
    asm volatile("" ::"s"(it.seq), "s"(it.kv_head), "s"(it.row_begin), "s"(it.row_end), "s"(it.key_begin),
                 "s"(it.key_end), "s"(it.partial_row), "s"(it.flags), "s"(it.rot), "s"(hid0.x), "s"(hid0.y),
                 "s"(hid1.x), "s"(hid1.y), "s"(a.pool_k), "s"(a.pool_v), "s"(a.layer_offset),
                 "s"(a.block_tables), "s"(a.bt_stride), "s"(a.q), "s"(a.k_new), "s"(a.v_new),
                 "s"(a.num_kv_heads), "s"(a.g), "s"(a.g_magic), "s"(a.query_start_loc), "s"(a.num_computed),
                 "s"(a.context_lens), "s"(a.head_ok));
    if (it.seq < 0) return;   // an idle item of a fixed-shape launch
    const int c = lane & 15, q4 = lane >> 4;
    const int s = it.seq, j = it.kv_head;
    const int g = a.g;
    // the sequence's offsets, from the call's arrays
    const SeqInfo si = seq_info(a, s);
    const int qs0 = si.qs0, nc = max(si.nc, 0);
    const int32_t *bt = a.block_tables + (int64_t)s * a.bt_stride;
    const int64_t rs = (int64_t)a.num_kv_heads * D;  // elements from one slot to the next
    const T *kp = static_cast<const T *>(a.pool_k) + a.layer_offset + (int64_t)j * D;
    const T *vp = static_cast<const T *>(a.pool_v) + a.layer_offset + (int64_t)j * D;
    const int kb = it.key_begin, ke = it.key_end;
    // fused scatter: this step's keys (positions nc..) come from the inputs,
    // key position p from packed token qs0 + p - nc
    const bool fused = FUSE && a.fuse_scatter != 0;
    const T *kn = static_cast<const T *>(fused ? a.k_new : a.pool_k) + (int64_t)j * D;
    const T *vn = static_cast<const T *>(fused ? a.v_new : a.pool_v) + (int64_t)j * D;
    const int new_lo = fused ? nc : INT32_MAX;   // keys in [new_lo, ke) are read from kn / vn
    auto new_row = [&](int pos) { return (int64_t)tok_index(a, qs0, pos - nc); };

    // The item's block ids go to LDS once: every tile after a wave's first
    // reads its two ids there instead of waiting on a scalar load from the
    // table. The staging loads are issued before the first tile's, so
    // waiting for them does not wait for K/V.
    // A second tile in flight fits the registers for one row tile (except
    // fp32 rows of 128), and for two row tiles of 16-bit rows of 64.
    constexpr bool DOUBLE_BUFFER = (RT == 1 && !(ELT == 4 && D == 128)) || (RT == 2 && ELT == 2 && D == 64);
    // Short items (no wave gets a tile past the ones it takes from the
    // table) skip the staging and its barrier.
    int32_t *const sbt = sh.bt;
    constexpr int SPT = (PS_DEC_MAX_SPLIT / PS_BLOCK + 64 * NW - 1) / (64 * NW);
    const int nb = (ke - kb + PS_BLOCK - 1) / PS_BLOCK;
    const bool staged = (ke - kb + PS_DEC_TILE - 1) / PS_DEC_TILE > (DOUBLE_BUFFER ? 2 : 1) * NW;
    const int32_t *btk = bt + (kb >> 4);
    int32_t stg[SPT] = {};
    if (staged) {
#pragma unroll
        for (int i = 0; i < SPT; ++i) stg[i] = btk[min(tid + i * 64 * NW, nb - 1)];
    }

    // Fused scatter: the item holding the sequence's last keys (last row
    // range, last key slice) copies this step's K/V rows of its KV head
    // into their slots; no item of this launch reads those slots from the
    // pool. A thread's first 16-byte word and its slot are loaded here,
    // ahead of the K/V tiles, and stored after the tiles: the copy then
    // adds no load latency to the item's end.
    constexpr int WPR = D * ELT / 16;   // 16-byte words per head row
    const bool writer = fused && (it.flags & PS_ITEM_WRITES_NEW);
    const int n_new = max(ke - nc, 0);
    const int sc_units = writer ? 2 * n_new * WPR : 0;
    const int64_t rw16 = rs * ELT / 16;   // 16-byte words from one slot (or token) to the next
    auto sc_word = [&](int w, const u32x4 *&src, int &i, int &cw, int &which) {
        which = w >= n_new * WPR;   // K words first, then V (w < sc_units)
        const int r2 = w - which * n_new * WPR;
        i = r2 / WPR;
        cw = r2 - i * WPR;
        src = reinterpret_cast<const u32x4 *>(which ? vn : kn) + (int64_t)tok_index(a, qs0, i) * rw16 + cw;
    };
    u32x4 sc_data = {0u, 0u, 0u, 0u};
    int32_t sc_slot = -1;
    int sc_cw = 0, sc_which = 0;
    if (tid < sc_units) {
        const u32x4 *src;
        int i;
        sc_word(tid, src, i, sc_cw, sc_which);
        sc_slot = a.slot_mapping[tok_index(a, qs0, i)];
        sc_data = *src;
    }

    u32x4 qf[RT][KU4];
    int lim[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
        load_q_row<DT, D>(a, it.row_begin + rt * 16 + c, it.row_end, g, j, si, q4, qf[rt], lim[rt]);

    float m[RT], l[RT];
    f32x4 o[RT][NT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        m[rt] = kNegInf;
        l[rt] = 0.f;
#pragma unroll
        for (int t = 0; t < NT; ++t) o[rt][t] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    constexpr int NBUF = DOUBLE_BUFFER ? 2 : 1;
    u32x4 kf[NBUF][2][KU4];
    uint32_t vr[NBUF][8][VW];

    // K/V of walk-order tile t, keys [k0, k0 + 32): two pool blocks. Block
    // ids are read with scalar loads (t is wave-uniform), so the vector
    // loads never wait on each other: a wave's first tiles from the item's
    // head ids (they need nothing but the item's index), later ones from
    // LDS. A block's address is a scalar base plus a lane offset fixed for
    // the whole item, so the loads take no vector address arithmetic. Rows
    // of an existing block past key_end are loaded (they are in bounds) and
    // zeroed or masked at use.
    const int64_t rsb = rs * ELT;                     // bytes from one slot (or token) to the next
    const uint32_t koff = (uint32_t)(c * rsb + 16 * q4);   // + 64 u: the lane's K words
    uint32_t voff[4];                                  // V row 4 q4 + i of a block, the lane's words
#pragma unroll
    for (int i = 0; i < 4; ++i) voff[i] = (uint32_t)((4 * q4 + i) * rsb + EPL * c * ELT);
    const char *kpool = reinterpret_cast<const char *>(kp), *vpool = reinterpret_cast<const char *>(vp);
    const char *knew = reinterpret_cast<const char *>(kn), *vnew = reinterpret_cast<const char *>(vn);
    auto load_tile = [&](auto bufc, int t, int k0, auto from_lds) {
        constexpr int buf = decltype(bufc)::value;
        const bool has1 = k0 + 16 < ke;
        int64_t blk0, blk1;
        if constexpr (decltype(from_lds)::value) {
            const int li = (k0 - kb) >> 4;
            blk0 = clamp_blk(a, __builtin_amdgcn_readfirstlane(sbt[li]));
            blk1 = has1 ? clamp_blk(a, __builtin_amdgcn_readfirstlane(sbt[li + 1])) : blk0;
        } else if (a.head_ok && t < PS_DEC_HEAD_TILES) {   // t is wave or wave + NW
            const int2 ids = t == wave ? hid0 : hid1;
            blk0 = ids.x;
            blk1 = ids.y;
        } else {
            blk0 = clamp_blk(a, bt[k0 >> 4]);
            blk1 = has1 ? clamp_blk(a, bt[(k0 >> 4) + 1]) : blk0;
        }
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
            const int kbk = k0 + sb * 16;                // the block's first key
            const int64_t blk = sb ? blk1 : blk0;
            const char *kb_pool = kpool + blk * 16 * rsb, *vb_pool = vpool + blk * 16 * rsb;
            if (kbk + 16 <= new_lo) {
                // every row from the pool: scalar base + fixed lane offset
                if (sb == 0 || has1) {
#pragma unroll
                    for (int u = 0; u < KU4; ++u)
                        kf[buf][sb][u] = load_vec<STREAM>(reinterpret_cast<const u32x4 *>(kb_pool + koff + 64 * u));
                } else {
#pragma unroll
                    for (int u = 0; u < KU4; ++u) kf[buf][sb][u] = u32x4{0u, 0u, 0u, 0u};
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) load_words<VW, STREAM>(vb_pool + voff[i], vr[buf][sb * 4 + i]);
            } else {
                // the block holds keys of this step: rows in [new_lo, ke)
                // come from k_new / v_new (key position p is packed token
                // qs0 + p - nc, whose row has the same stride as a pool slot)
                if (sb == 0 || has1) {
                    const int pos = kbk + c;
                    const char *src = pos >= new_lo && pos < ke ? knew + new_row(pos) * rsb + 16 * q4
                                                                : kb_pool + koff;
#pragma unroll
                    for (int u = 0; u < KU4; ++u)
                        kf[buf][sb][u] = load_vec<STREAM>(reinterpret_cast<const u32x4 *>(src + 64 * u));
                } else {
#pragma unroll
                    for (int u = 0; u < KU4; ++u) kf[buf][sb][u] = u32x4{0u, 0u, 0u, 0u};
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int pos = kbk + 4 * q4 + i;
                    const char *src = pos >= new_lo && pos < ke ? vnew + new_row(pos) * rsb + EPL * c * ELT
                                                                : vb_pool + voff[i];
                    load_words<VW, STREAM>(src, vr[buf][sb * 4 + i]);
                }
            }
        }
    };

    // keys below vis_all are visible to every row of the item (the first
    // row's query sits at position nc + row_begin / g)
    const int vis_all = min(min(ke, si.ctx), nc + div_g(a, it.row_begin) + 1);
    auto compute_tile = [&](auto bufc, int k0) {
        constexpr int buf = decltype(bufc)::value;
        float pv[RT][8];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            f32x4 sacc[2];
#pragma unroll
            for (int sb = 0; sb < 2; ++sb) sacc[sb] = qk_tile<DT, D>(kf[buf][sb], qf[rt]);
#pragma unroll
            for (int sb = 0; sb < 2; ++sb)
#pragma unroll
                for (int i = 0; i < 4; ++i) pv[rt][sb * 4 + i] = sacc[sb][i];
        }
        if (k0 + PS_DEC_TILE > vis_all) {
            // a tile on the causal diagonal or at the slice's end
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                const int vis = min(ke - 1, lim[rt]) - k0 - 4 * q4;
#pragma unroll
                for (int sb = 0; sb < 2; ++sb)
#pragma unroll
                    for (int i = 0; i < 4; ++i) pv[rt][sb * 4 + i] = sb * 16 + i <= vis ? pv[rt][sb * 4 + i] : kNegInf;
            }
        }
        softmax_update(pv, a.scale_log2, m, l, o);
        if (k0 + PS_DEC_TILE > ke) {
            // V rows at or past key_end may be stale (even NaN) and P = 0
            // there would not cancel them
            const int vlim = ke - k0 - 4 * q4;
#pragma unroll
            for (int jj = 0; jj < 8; ++jj) {
                const bool ok = (jj >> 2) * 16 + (jj & 3) < vlim;
#pragma unroll
                for (int w = 0; w < VW; ++w) vr[buf][jj][w] = ok ? vr[buf][jj][w] : 0u;
            }
        }
        if constexpr (DT::ELT == 2) {
            u32x4 pb[RT];
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int e = 0; e < 4; ++e) pb[rt][e] = pack2(pv[rt][2 * e], pv[rt][2 * e + 1], DT{});
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                const u32x4 av = v_operand<VW>(vr[buf], t);
#pragma unroll
                for (int rt = 0; rt < RT; ++rt) o[rt][t] = mfma32(av, pb[rt], o[rt][t], DT{});
            }
        } else {
#pragma unroll
            for (int jj = 0; jj < 8; ++jj)
#pragma unroll
                for (int t = 0; t < NT; ++t) {
                    const float av = __builtin_bit_cast(float, vr[buf][jj][t]);
#pragma unroll
                    for (int rt = 0; rt < RT; ++rt) o[rt][t] = mfma4(av, pv[rt][jj], o[rt][t]);
                }
        }
    };

    using B0 = std::integral_constant<int, 0>;
    using B1 = std::integral_constant<int, 1>;
    using FromTable = std::false_type;
    using FromLds = std::true_type;
    const int ntiles = (ke - kb + PS_DEC_TILE - 1) / PS_DEC_TILE;
    // With the walk-rotation plan option an item starts its walk over the
    // key range at an item-dependent tile (it.rot, 0 otherwise), so that
    // items sharing prefix blocks do not all ask for the same lines at once
    // (softmax order is free; the order is a fixed function of the item).
    const int rot = it.rot;
    auto key0 = [&](int t) {
        int u = t + rot;
        u -= u >= ntiles ? ntiles : 0;
        return kb + u * PS_DEC_TILE;
    };
    int ti = wave;
    // A wave's first tiles (one, or two with a second buffer) take their
    // ids from the table; they are in flight while the staged ids are
    // written. Waiting for the staging loads there waits for those tiles
    // too, which costs little: they were issued together.
    if (ti < ntiles) load_tile(B0{}, ti, key0(ti), FromTable{});
    if constexpr (DOUBLE_BUFFER)
        if (ti + NW < ntiles) load_tile(B1{}, ti + NW, key0(ti + NW), FromTable{});
    if (staged) {
#pragma unroll
        for (int i = 0; i < SPT; ++i)
            if (tid + i * 64 * NW < nb) sbt[tid + i * 64 * NW] = stg[i];
        lds_barrier();
    }
    // Two row tiles of 16-bit rows of 128 leave no registers for a second
    // tile in flight. Their wave's region of the LDS merge buffer (idle
    // until the wave's last tile, 16 KiB: K and V of one tile) takes it
    // instead: tile ti + NW is DMA'd there while tile ti is computed, then
    // read into the registers. Rows sit as in the prefill ring (16-byte
    // chunks XOR-swizzled by row), so the fragment reads are conflict free.
    constexpr bool LDS_SLOT = !DOUBLE_BUFFER && ELT == 2 && D == 128;
    static_assert(!LDS_SLOT || sizeof(sh.o[0]) == 2 * PS_DEC_TILE * D * ELT, "slot size");
    uint8_t *const slot = reinterpret_cast<uint8_t *>(&sh.o[wave][0][0]);
    const uint32_t slot_lds = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t *)slot;
    // DMA of the tile at k0 (blocks b0, b1): instruction i moves rows
    // 4 (i % 8) .. +3 of K (i < 8) or V, lane l row + l / 16, position l % 16
    auto dma_tile = [&](int k0, int64_t b0, int64_t b1) {
        const int p = lane & 15;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int kv = i >> 3;
            const int rr = (i & 7) * 4 + (lane >> 4);       // row of the tile
            const int64_t blk = (i & 7) >= 4 ? b1 : b0;      // compile-time choice
            const int chunk = swz<D * ELT>(p, rr) * (16 / ELT);
            const T *pool = kv ? vp : kp;
            if (k0 + PS_DEC_TILE <= new_lo) {
                // the block base is wave-uniform; say so, for the scalar operand
                const uint64_t base = (uint64_t)(uintptr_t)(pool + blk * 16 * rs);
                // (readfirstlane returns int: widen through uint32_t, or the
                // low half would sign-extend over the high one)
                const uint64_t ubase =
                    ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(base >> 32)) << 32) |
                    (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)base);
                dma16_sv<STREAM>(reinterpret_cast<const void *>(ubase), (uint32_t)(((rr & 15) * (int)rs + chunk) * ELT),
                         slot_lds + i * 1024);
            } else {
                const int pos = k0 + rr;
                const T *src = pos >= new_lo && pos < ke ? (kv ? vn : kn) + new_row(pos) * rs + chunk
                                                         : pool + (blk * 16 + (rr & 15)) * rs + chunk;
                dma16<STREAM>(src, slot + i * 1024);
            }
        }
    };
    // the slot's tile into the registers of buffer 0, as load_tile leaves them
    auto read_slot = [&]() {
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
            const int r = sb * 16 + c;
#pragma unroll
            for (int u = 0; u < KU4; ++u)
                kf[0][sb][u] = *reinterpret_cast<const u32x4 *>(slot + r * (D * ELT) +
                                                                swz<D * ELT>(u * 4 + q4, r) * 16);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int rv = sb * 16 + 4 * q4 + i;
                const u32x4 x = *reinterpret_cast<const u32x4 *>(slot + PS_DEC_TILE * (D * ELT) +
                                                                 rv * (D * ELT) + swz<D * ELT>(c, rv) * 16);
#pragma unroll
                for (int w = 0; w < 4; ++w) vr[0][sb * 4 + i][w] = x[w];
            }
        }
    };
    if constexpr (!DOUBLE_BUFFER && !LDS_SLOT) {
        // the other resident waves cover the load latency
        for (; ti < ntiles; ti += NW) {
            if (ti != wave) load_tile(B0{}, ti, key0(ti), FromLds{});
            compute_tile(B0{}, key0(ti));
        }
    }
    if constexpr (LDS_SLOT) {
        if (ti + NW < ntiles) {
            // the wave's second tile: ids from the head (or the table)
            const int t1 = ti + NW, k1 = key0(t1);
            int64_t b0, b1;
            if (a.head_ok && t1 < PS_DEC_HEAD_TILES) {
                b0 = hid1.x;
                b1 = hid1.y;
            } else {
                b0 = clamp_blk(a, bt[k1 >> 4]);
                b1 = k1 + 16 < ke ? clamp_blk(a, bt[(k1 >> 4) + 1]) : b0;
            }
            dma_tile(k1, b0, b1);
        }
        for (; ti < ntiles; ti += NW) {
            if (ti != wave) {
                // the DMA of this tile (the only vector memory operation in
                // flight) has landed; the asm fences keep the compiler from
                // moving LDS reads across the waits
                wait_vmcnt<0>();
                asm volatile("" ::: "memory");
                read_slot();
                __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the slot is read
                asm volatile("" ::: "memory");
                if (ti + NW < ntiles) {
                    const int kn2 = key0(ti + NW);
                    const int li = (kn2 - kb) >> 4;
                    const int64_t b0 = clamp_blk(a, __builtin_amdgcn_readfirstlane(sbt[li]));
                    const int64_t b1 = kn2 + 16 < ke ? clamp_blk(a, __builtin_amdgcn_readfirstlane(sbt[li + 1])) : b0;
                    dma_tile(kn2, b0, b1);
                }
            }
            compute_tile(B0{}, key0(ti));
        }
    }
    if constexpr (DOUBLE_BUFFER) {
        // tile ti + 2 NW streams into the buffer tile ti has just released
        while (ti < ntiles) {
            compute_tile(B0{}, key0(ti));
            if (ti + 2 * NW < ntiles) load_tile(B0{}, ti + 2 * NW, key0(ti + 2 * NW), FromLds{});
            ti += NW;
            if (ti >= ntiles) break;
            compute_tile(B1{}, key0(ti));
            if (ti + 2 * NW < ntiles) load_tile(B1{}, ti + 2 * NW, key0(ti + 2 * NW), FromLds{});
            ti += NW;
        }
    }

    // ---- fused scatter: the stores (words past the first 64 NW come
    // from a plain copy loop)
    if (sc_units > 0) {
        u32x4 *pk = reinterpret_cast<u32x4 *>(const_cast<T *>(kp));
        u32x4 *pv = reinterpret_cast<u32x4 *>(const_cast<T *>(vp));
        if (tid < sc_units && (uint32_t)sc_slot < (uint32_t)a.num_slots)
            (sc_which ? pv : pk)[(int64_t)sc_slot * rw16 + sc_cw] = sc_data;
        for (int w = tid + 64 * NW; w < sc_units; w += 64 * NW) {
            const u32x4 *src;
            int i, cw, which;
            sc_word(w, src, i, cw, which);
            const int32_t slot = a.slot_mapping[tok_index(a, qs0, i)];
            if ((uint32_t)slot >= (uint32_t)a.num_slots) continue;
            (which ? pv : pk)[(int64_t)slot * rw16 + cw] = *src;
        }
    }

    // The staging registers stay allocated up to here: reused earlier,
    // they would make the first tile's compute wait (at the join of the
    // staged and unstaged paths) for every load in flight.
#pragma unroll
    for (int i = 0; i < SPT; ++i) asm volatile("" ::"v"(stg[i]));

    // ---- merge the waves' states
    // A wave's partial O goes to its LDS region lane-major: entry
    // cb = (rt * 4 + i) * NT + t of every lane (row rt * 16 + c, column
    // EPL * (4 q4 + i) + t) sits at cb * 64 + lane. Each store, and each
    // read below, then covers 64 consecutive words: no bank conflicts
    // (row-major, the 16 lanes of one column would all hit one bank).
    constexpr int NE = RT * 4 * NT;   // entries per lane
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        l[rt] = xor_sum(l[rt]);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int t = 0; t < NT; ++t) (&sh.o[wave][0][0])[((rt * 4 + i) * NT + t) * 64 + lane] = o[rt][t][i];
        if (q4 == 0) {
            sh.m[wave][rt * 16 + c] = m[rt];
            sh.l[wave][rt * 16 + c] = l[rt];
        }
    }
    __syncthreads();

    // Thread (wave, lane) finishes entries [wave * EPT, wave * EPT + EPT)
    // of the lane's position: one row tile rt0, columns d0 .. d0 + EPT - 1
    // (EPL = NT, so column EPL * (4 q4 + i) + t is 4 NT q4 + cb mod 4 NT).
    constexpr int EPT = NE / NW;   // output elements per thread (>= 1)
    static_assert(EPT >= 1 && NE % NW == 0 && (4 * NT) % EPT == 0, "waves do not split the entries");
    static_assert(EPL == NT && NE * 64 == ROWS * D, "entry layout");
    const int cb0 = wave * EPT;
    const int row = cb0 / (4 * NT) * 16 + c, d0 = 4 * NT * q4 + cb0 % (4 * NT);
    const int r = it.row_begin + row;
    if (r >= it.row_end) return;
    float mw[NW], M = kNegInf;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        mw[w] = sh.m[w][row];
        M = fmaxf(M, mw[w]);
    }
    const float muse = M == kNegInf ? 0.f : M;
    float L = 0.f, acc[EPT];
#pragma unroll
    for (int e = 0; e < EPT; ++e) acc[e] = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        const float f = fast_exp2(mw[w] - muse);
        L += sh.l[w][row] * f;
#pragma unroll
        for (int e = 0; e < EPT; ++e) acc[e] += (&sh.o[w][0][0])[(cb0 + e) * 64 + lane] * f;
    }
    if (it.partial_row < 0) {
        const int tok = div_g(a, r);
        const int h = j * g + (r - tok * g);
        T *op = static_cast<T *>(a.out) + ((int64_t)tok_index(a, qs0, tok) * a.num_q_heads + h) * D + d0;
        const float inv = 1.f / L;
#pragma unroll
        for (int e = 0; e < EPT; ++e) op[e] = cvt_out(acc[e] * inv, DT{});
    } else {
        const int64_t pr = (int64_t)it.partial_row + row;
#pragma unroll
        for (int e = 0; e < EPT; ++e) a.ws_acc[pr * D + d0 + e] = acc[e];
        if (d0 == 0) {
            a.ws_m[pr] = M;
            a.ws_l[pr] = L;
        }
    }
}

template <class DT, int D, int RT, int NW, bool STREAM>
__global__ __launch_bounds__(64 * NW, NW >= 16 ? 4 : 2) void ps_decode_kernel(const ps_attn_launch a) {
    __shared__ DecodeLds<DT, D, RT, NW> L;
    decode_item<DT, D, RT, NW, STREAM>(a, blockIdx.x, L);
}

// ---------------------------------------------------------------------------
// Prefill-chunk attention. One workgroup = 128 packed rows (4 waves x 32)
// of one sequence and KV head over a key slice. K and V tiles (64 keys for
// 16-bit data, 32 for fp32) are gathered through the block table straight
// into LDS with global_load_lds_dwordx4 (no register staging) into a
// two-stage ring, so the next tile streams in while the current one is
// consumed. 16-byte chunks of each key row are XOR-swizzled by the row
// (swz), which keeps the per-key K fragment reads and the transposing V
// reads off each other's LDS banks without padding (the DMA writes whole
// 1 KiB lines). Hand-offs use a bare s_barrier with explicit s_waitcnt,
// since a fenced barrier would also wait for the tile still in flight.


// 4 16-bit values per lane, transposed within each 16-lane group: lane i
// receives element i % 4 of the 8-byte loads issued by lanes 4e + i / 4,
// e = 0..3
__device__ inline u32x2 lds_read_tr16(const uint8_t *p) {
#if defined(__HIP_DEVICE_COMPILE__)
    typedef short s16x4 __attribute__((ext_vector_type(4)));
    const s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4 *)(p));
    return __builtin_bit_cast(u32x2, r);
#else
    (void)p;
    return u32x2{0u, 0u};
#endif
}

// `bytes` bytes starting at byte `off` of swizzled LDS row `row`
template <int ROWB, int VW>
__device__ inline void lds_row_words(const uint8_t *rowp, int row, int off, uint32_t (&w)[VW]) {
    if constexpr (VW == 2) {
        const u32x2 x = *reinterpret_cast<const u32x2 *>(rowp + swz<ROWB>(off >> 4, row) * 16 + (off & 15));
        w[0] = x[0];
        w[1] = x[1];
    } else {
#pragma unroll
        for (int i = 0; i < VW / 4; ++i) {
            const u32x4 x = *reinterpret_cast<const u32x4 *>(rowp + swz<ROWB>((off >> 4) + i, row) * 16);
            w[4 * i + 0] = x[0];
            w[4 * i + 1] = x[1];
            w[4 * i + 2] = x[2];
            w[4 * i + 3] = x[3];
        }
    }
}

// TK: keys per tile; OCC: waves per SIMD the register budget is sized for
// (1: 512 registers, accumulators may live in AGPRs; 2: 256 registers)
template <class DT, int D, int TK>
struct PrefillLds {
    static constexpr int STAGEB = 2 * TK * D * DT::ELT;  // one ring stage: K tile, then V tile
    __attribute__((aligned(1024))) uint8_t ring0[STAGEB];
    __attribute__((aligned(1024))) uint8_t ring1[STAGEB];
    int32_t bt[PS_PRE_MAX_KEYS / PS_BLOCK];  // the item's block ids
};

template <class DT, int D, int TK, int RPW>
__device__ __forceinline__ void prefill_item(const ps_attn_launch a, int item, PrefillLds<DT, D, TK> &sh) {
    using G = Geo<DT, D>;
    using T = typename DT::T;
    constexpr int ELT = G::ELT, KU4 = G::KU4, VW = G::VW, NT = G::NT, EPL = G::EPL;
    constexpr int RT = RPW / 16;  // 16-row MFMA tiles per wave
    constexpr int NSB = TK / 16;
    constexpr int ROWB = D * ELT;          // LDS bytes per key row
    constexpr int CPR = ROWB / 16;         // 16-byte chunks per row
    constexpr int TILEB = TK * ROWB;       // one K (or V) tile
    constexpr int STAGEB = 2 * TILEB;      // K then V
    constexpr int NLD = STAGEB / 4096;     // 16-byte DMA loads per thread per stage
    static_assert(CPR >= 8 && TILEB % 4096 == 0, "tile geometry");
    static_assert(2 * RPW * D * ELT <= STAGEB, "output staging fits the ring");

    static_assert(PrefillLds<DT, D, TK>::STAGEB == STAGEB, "stage size");
    uint8_t *const ring0 = sh.ring0;
    uint8_t *const ring1 = sh.ring1;
    auto stage = [&](auto sc) -> uint8_t * { return decltype(sc)::value == 0 ? ring0 : ring1; };
    int32_t *const sbt = sh.bt;

    const ps_item it = a.prefill_items[item];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int c = lane & 15, q4 = lane >> 4;
    const int s = it.seq, j = it.kv_head;
    const int g = a.g;
    // the sequence's offsets, from the call's arrays (a gathered item's
    // rows name their own sequences)
    const SeqInfo si = seq_info(a, s);
    const int qs0 = si.qs0, nc = si.nc;
    const int32_t *bt = a.block_tables + (int64_t)s * a.bt_stride;
    const int64_t rs = (int64_t)a.num_kv_heads * D;
    const T *kp = static_cast<const T *>(a.pool_k) + a.layer_offset + (int64_t)j * D;
    const T *vp = static_cast<const T *>(a.pool_v) + a.layer_offset + (int64_t)j * D;
    const int kb = it.key_begin, ke = it.key_end;
    // byte offset of pool block b (b < 2^31, 16 rows of at most 1 MiB)
    const uint32_t bstride = (uint32_t)(PS_BLOCK * rs * ELT);
    auto blk_bytes = [&](int64_t b) { return (uint64_t)(uint32_t)b * bstride; };

    const int wr0 = it.row_begin + wave * RPW;
    const bool active = wr0 < it.row_end;
    const int wr_last = min(wr0 + RPW, it.row_end) - 1;
    // A gathered item (shared-prefix pass) takes its rows from the row map;
    // every key of its range is visible to all of them.
    const bool gathered = (it.flags & PS_ITEM_GATHERED) != 0;
    constexpr int kAllVisible = INT32_MAX / 2;
    // smallest and largest visibility limits among the wave's rows
    const int lim_lo = gathered ? kAllVisible : min(nc + div_g(a, wr0), si.ctx - 1);
    const int lim_hi = gathered ? kAllVisible : min(nc + div_g(a, wr_last), si.ctx - 1);


    // 16-bit data: o carries one more tile, the row sums of P, formed on
    // MFMA against an all-ones V tile (rescaled with o, and summed over the
    // same rounded P as the numerator)
    constexpr int NTL = ELT == 2 ? NT + 1 : NT;
    float m[RT], l[RT];
    f32x4 o[RT][NTL];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        m[rt] = kNegInf;
        l[rt] = 0.f;
#pragma unroll
        for (int t = 0; t < NTL; ++t) o[rt][t] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    // DMA the K/V tile of keys [k0, k0 + TK) into ring stage `stage`. Block
    // ids are scalar loads; keys of blocks past key_end re-read the tile's
    // first block (in bounds) and are masked or zeroed at use.
    constexpr int RPI = 4096 / ROWB;  // key rows one DMA instruction covers
    static_assert(RPI >= 8 && (RPI <= 16 || RPI == 32), "rows per DMA instruction");
    const int trow = tid / CPR;        // this thread's row within such a group
    const int tpos = tid % CPR;        // and its 16-byte position in that row
    // The tile's block ids: one LDS read of NSB consecutive entries (the
    // tile starts a multiple of NSB entries in; entries past the item's
    // blocks are read but not used), issued before the wait that precedes
    // the DMA so that its latency hides under that wait.
    using IdVec = int32_t __attribute__((ext_vector_type(NSB)));
    auto read_ids = [&](int k0) -> IdVec { return *reinterpret_cast<const IdVec *>(sbt + ((k0 - kb) >> 4)); };
    auto issue_tile = [&](auto stagec, int k0, IdVec ids) {
        uint8_t *const ring = stage(stagec);
        int64_t blk[NSB];
        blk[0] = clamp_blk(a, __builtin_amdgcn_readfirstlane(ids[0]));
#pragma unroll
        for (int b = 1; b < NSB; ++b)
            blk[b] = (k0 + 16 * b < ke) ? clamp_blk(a, __builtin_amdgcn_readfirstlane(ids[b])) : blk[0];
#pragma unroll
        for (int i = 0; i < NLD; ++i) {
            const int r0 = (i * RPI) % TK;  // first key row of instruction i (compile-time)
            const int kv = (i * RPI) / TK;  // K or V (compile-time)
            const int key = r0 + trow;
            int64_t b = blk[r0 >> 4];
            if constexpr (RPI == 32) b = (trow >> 4) ? blk[(r0 >> 4) + 1] : b;
            const int inblk = (key & 15) * (int)rs + swz<ROWB>(tpos, key) * (16 / ELT);
            // (block ids and the block stride fit 32 bits: one 32x32 -> 64
            // multiply per block)
            const char *bbase = reinterpret_cast<const char *>(kv ? vp : kp) + blk_bytes(b);
            if constexpr (RPI == 32) {  // one instruction spans two blocks: per-lane address
                dma16(reinterpret_cast<const T *>(bbase) + inblk, ring + i * 4096 + wave * 1024);
            } else {  // scalar block base, loop-invariant lane offset, scalar LDS slot
                const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t *)ring;
                dma16_sv(bbase, (uint32_t)inblk * ELT, lds0 + i * 4096 + wave * 1024);
            }
        }
    };

    using S0 = std::integral_constant<int, 0>;
    using S1 = std::integral_constant<int, 1>;
    // Tile 0's DMA goes out first, with its block ids read straight from the
    // table (scalar loads), so that its latency overlaps the Q rows' and the
    // staged ids' instead of following them.
    const int ntiles = (ke - kb + TK - 1) / TK;
    if (ntiles > 0) {
        const int32_t *btk = bt + (kb >> 4);
        IdVec id0;
#pragma unroll
        for (int b = 0; b < NSB; ++b) id0[b] = kb + 16 * b < ke ? btk[b] : 0;  // (unused past key_end)
        issue_tile(S0{}, kb, id0);
    }

    u32x4 qf[RT][KU4];
    int lim[RT];
    ps_row grow[RT];   // gathered rows' map entries
    if (!gathered) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
            load_q_row<DT, D>(a, wr0 + rt * 16 + c, it.row_end, g, j, si, q4, qf[rt], lim[rt]);
    } else {
        // (as in load_q_row: a row past the end reads the last row's map
        // entry and query, unconditionally, and is never stored); all map
        // entries first, then their sequences' first rows, then the
        // queries they name
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            const int r = wr0 + rt * 16 + c;
            grow[rt] = a.row_map[it.partial_row + (r < it.row_end ? r : it.row_end - 1)];
            lim[rt] = r < it.row_end ? kAllVisible : -1;
        }
        int gqs[RT];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) gqs[rt] = a.query_start_loc[grow[rt].seq];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            const int tok = div_g(a, grow[rt].row);
            const int h = j * g + (grow[rt].row - tok * g);
            const T *qp = static_cast<const T *>(a.q) + ((int64_t)tok_index(a, gqs[rt], tok) * a.num_q_heads + h) * D;
#pragma unroll
            for (int u = 0; u < KU4; ++u) qf[rt][u] = *reinterpret_cast<const u32x4 *>(qp + (u * 4 + q4) * (16 / ELT));
        }
    }

    // Block ids of the item's key range go to LDS once: inside the ring
    // they could only be vector loads, and waiting for those would also
    // wait for the tile in flight. Q is waited for here for the same
    // reason, and so is tile 0, issued together with them.
    for (int i = tid; i < (ke - kb + PS_BLOCK - 1) / PS_BLOCK; i += 256) sbt[i] = bt[(kb >> 4) + i];
    wait_vmcnt<0>();
    __syncthreads();

    // The all-ones A operand of the row-sum MFMAs, held in VGPRs for the
    // whole item (the empty asm makes it opaque): as a constant, the
    // compiler rebuilt it from SGPRs with two 64-bit moves at every use.
    constexpr uint32_t one2 = std::is_same<DT, TBF16>::value ? 0x3F803F80u : 0x3C003C00u;
    u32x4 ones = {one2, one2, one2, one2};
    if constexpr (ELT == 2) asm volatile("" : "+v"(ones));
    auto compute_tile = [&](auto stagec, int k0) {
        const uint8_t *ksm = stage(stagec);
        const uint8_t *vsm = ksm + TILEB;
        const bool full = (k0 + TK <= ke) && (k0 + TK - 1 <= lim_lo);
        // The MFMA runs go at raised wave priority: with two waves per SIMD,
        // the one in its softmax then issues around the other's matrix
        // work instead of the two contending (2-3% on long chunks).
        f32x4 sacc[RT][NSB];
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int sb = 0; sb < NSB; ++sb) {
            u32x4 kf[KU4];
            const uint8_t *kr = ksm + (sb * 16 + c) * ROWB;
#pragma unroll
            for (int u = 0; u < KU4; ++u) kf[u] = *reinterpret_cast<const u32x4 *>(kr + swz<ROWB>(u * 4 + q4, sb * 16 + c) * 16);
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) sacc[rt][sb] = qk_tile<DT, D>(kf, qf[rt]);
        }
        __builtin_amdgcn_s_setprio(0);
        // 16-bit data: the V operands of the first 32-key half are read
        // here, ahead of the softmax (they do not depend on P), so that
        // their LDS latency hides under its VALU work; the softmax's
        // rescale branch keeps the compiler from sinking them to their use.
        // A operand of O^T tile t straight from LDS with transposing reads:
        // lane (c, q4) gets V[keys 4q4..4q4+3 and 16+4q4..19+4q4][d = 16t +
        // c]; in the group the source lane j reads row (j / 4) of the key
        // quad, d quad (j % 4).
        const int j16 = lane & 15;
        const int vtrow = 4 * q4 + (j16 >> 2);
        const int tbyte = (j16 & 3) * 8;  // within a 32-byte d tile
        auto v_half = [&](int h, u32x4 (&av)[NT]) {
            const int r0 = 32 * h + vtrow, r1 = r0 + 16;
            const uint8_t *v0 = vsm + r0 * ROWB, *v1 = vsm + r1 * ROWB;
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                const int b = t * 32 + tbyte;
                const u32x2 lo = lds_read_tr16(v0 + swz<ROWB>(b >> 4, r0) * 16 + (b & 15));
                const u32x2 hi = lds_read_tr16(v1 + swz<ROWB>(b >> 4, r1) * 16 + (b & 15));
                av[t] = u32x4{lo[0], lo[1], hi[0], hi[1]};
            }
        };
        u32x4 av0[ELT == 2 ? NT : 1];
        if constexpr (ELT == 2) {
            // (V rows past key_end were zeroed in LDS before this tile)
            v_half(0, av0);
        }
        float pv[RT][4 * NSB];
        if (full) {  // (wave-uniform) every key of the tile is visible to every row
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int sb = 0; sb < NSB; ++sb)
#pragma unroll
                    for (int i = 0; i < 4; ++i) pv[rt][sb * 4 + i] = sacc[rt][sb][i];
        } else {
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                // key k0 + sb*16 + 4*q4 + i is visible iff sb*16 + i <= vis
                const int vis = min(ke - 1, lim[rt]) - k0 - 4 * q4;
#pragma unroll
                for (int sb = 0; sb < NSB; ++sb)
#pragma unroll
                    for (int i = 0; i < 4; ++i) pv[rt][sb * 4 + i] = sb * 16 + i <= vis ? sacc[rt][sb][i] : kNegInf;
            }
        }
        softmax_update<RT, 4 * NSB, NTL, ELT != 2>(pv, a.scale_log2, m, l, o);
        __builtin_amdgcn_s_setprio(1);
        // P.V over 32-key halves
        if constexpr (ELT == 2) {
#pragma unroll
            for (int h = 0; h < NSB / 2; ++h) {
                u32x4 pb[RT];
#pragma unroll
                for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        pb[rt][e] = pack2(pv[rt][8 * h + 2 * e], pv[rt][8 * h + 2 * e + 1], DT{});
                u32x4 av[NT];
                if (h == 0) {
#pragma unroll
                    for (int t = 0; t < NT; ++t) av[t] = av0[t];
                } else {
                    v_half(h, av);
                }
#pragma unroll
                for (int t = 0; t < NT; ++t) {
#pragma unroll
                    for (int rt = 0; rt < RT; ++rt) o[rt][t] = mfma32(av[t], pb[rt], o[rt][t], DT{});
                }
#pragma unroll
                for (int rt = 0; rt < RT; ++rt) o[rt][NTL - 1] = mfma32(ones, pb[rt], o[rt][NTL - 1], DT{});
            }
            __builtin_amdgcn_s_setprio(0);
            return;
        }
#pragma unroll
        for (int h = 0; h < NSB / 2; ++h) {
            uint32_t vr[8][VW];
#pragma unroll
            for (int jj = 0; jj < 8; ++jj) {
                const int key = (2 * h + (jj >> 2)) * 16 + 4 * q4 + (jj & 3);
                lds_row_words<ROWB, VW>(vsm + key * ROWB, key, EPL * c * ELT, vr[jj]);
                if (k0 + TK > ke) {  // rows past key_end hold whatever the pool had
                    const bool ok = key < ke - k0;
#pragma unroll
                    for (int w = 0; w < VW; ++w) vr[jj][w] = ok ? vr[jj][w] : 0u;
                }
            }
            if constexpr (ELT == 2) {
                u32x4 pb[RT];
#pragma unroll
                for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        pb[rt][e] = pack2(pv[rt][8 * h + 2 * e], pv[rt][8 * h + 2 * e + 1], DT{});
#pragma unroll
                for (int t = 0; t < NT; ++t) {
                    const u32x4 av = v_operand<VW>(vr, t);
#pragma unroll
                    for (int rt = 0; rt < RT; ++rt) o[rt][t] = mfma32(av, pb[rt], o[rt][t], DT{});
                }
            } else {
#pragma unroll
                for (int jj = 0; jj < 8; ++jj)
#pragma unroll
                    for (int t = 0; t < NT; ++t) {
                        const float av = __builtin_bit_cast(float, vr[jj][t]);
#pragma unroll
                        for (int rt = 0; rt < RT; ++rt) o[rt][t] = mfma4(av, pv[rt][8 * h + jj], o[rt][t]);
                    }
            }
        }
        __builtin_amdgcn_s_setprio(0);
    };

    // Tile ti sits in stage ti % 2; the tile after it streams in while it
    // is consumed. One barrier per tile: once every thread's loads of tile
    // ti have landed, every wave has also finished tile ti - 1, so its
    // stage takes tile ti + 1.
    // Past the end a step re-reads its own tile instead of branching around
    // the issue: a branch here would make the compiler wait for the tiles
    // in flight before every LDS read.
    auto step = [&](auto cur, auto ahead, int ti, int ntiles) {
        const int k0 = kb + ti * TK;
        const int kn = ti + 1 < ntiles ? k0 + TK : k0;
        const IdVec ids = read_ids(kn);
        wait_vmcnt<0>();                // this thread's loads of tile ti have landed
        lds_barrier();                  // ... and every other thread's
        issue_tile(ahead, kn, ids);
        if constexpr (ELT == 2) {
            // The last tile of the slice: V rows past key_end hold whatever
            // the pool had (even NaN), and a zero weight would not cancel
            // them. Zero them in LDS (whole rows: the swizzle stays inside
            // a row), so the P.V loop needs no masks.
            if (k0 + TK > ke) {
                uint8_t *vz = stage(cur) + TILEB;
                const int first = ke - k0;
                for (int x = tid; x < (TK - first) * CPR; x += 256)
                    reinterpret_cast<u32x4 *>(vz + (first + x / CPR) * ROWB)[x % CPR] = u32x4{0u, 0u, 0u, 0u};
                lds_barrier();
            }
        }
        if (active && k0 <= lim_hi) compute_tile(cur, k0);
    };
    for (int ti = 0; ti < ntiles; ti += 2) {
        step(S0{}, S1{}, ti, ntiles);
        if (ti + 1 < ntiles) step(S1{}, S0{}, ti + 1, ntiles);
    }

    wait_vmcnt<0>();  // the last, unused tile must land before the ring is reused
    __syncthreads();
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        if constexpr (ELT == 2) l[rt] = o[rt][NTL - 1][0];  // every entry holds the row's sum
        else l[rt] = xor_sum(l[rt]);
    }

    if (gathered || it.partial_row >= 0) {
        if (!active) return;
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            const int r = wr0 + rt * 16 + c;
            if (r >= it.row_end) continue;
            const int64_t pr = gathered ? (int64_t)grow[rt].dest + (int64_t)it.split * grow[rt].stride
                                        : (int64_t)it.partial_row + (r - it.row_begin);
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                if constexpr (ELT == 2) {  // tile t row 4q4 + i holds d = 16t + 4q4 + i
                    *reinterpret_cast<f32x4 *>(a.ws_acc + pr * D + t * 16 + 4 * q4) = o[rt][t];
                } else {                   // ... d = EPL (4q4 + i) + t
#pragma unroll
                    for (int i = 0; i < 4; ++i) a.ws_acc[pr * D + EPL * (4 * q4 + i) + t] = o[rt][t][i];
                }
            }
            if (q4 == 0) {
                a.ws_m[pr] = m[rt];
                a.ws_l[pr] = l[rt];
            }
        }
        return;
    }

    // final output: normalise, round, transpose through LDS, write rows.
    // Chunk ch (16 bytes) of staged row `row` sits at ch ^ (row mod OCPR):
    // the 16 lanes that hold one column of a row tile then store to 16
    // different chunks (unswizzled, a row is 256 bytes and all 16 would
    // hit one bank).
    constexpr int OCPR = D * ELT / 16;   // 16-byte chunks per output row
    static_assert((OCPR & (OCPR - 1)) == 0, "chunks per row: a power of two");
    uint8_t *const sob = (wave < 2 ? ring0 : ring1) + (wave & 1) * RPW * D * ELT;
    auto staged = [&](int row, int byte) { return sob + row * (D * ELT) + (((byte >> 4) ^ (row & (OCPR - 1))) << 4) + (byte & 15); };
    if (active) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            const float inv = l[rt] > 0.f ? 1.f / l[rt] : 0.f;
            const int row = rt * 16 + c;
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                if constexpr (ELT == 2) {   // d = 16t + 4q4 .. +3: one 8-byte store
                    const u32x2 w = {pack2(o[rt][t][0] * inv, o[rt][t][1] * inv, DT{}),
                                     pack2(o[rt][t][2] * inv, o[rt][t][3] * inv, DT{})};
                    *reinterpret_cast<u32x2 *>(staged(row, (16 * t + 4 * q4) * ELT)) = w;
                } else {
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        *reinterpret_cast<T *>(staged(row, (EPL * (4 * q4 + i) + t) * ELT)) = cvt_out(o[rt][t][i] * inv, DT{});
                }
            }
        }
    }
    __syncthreads();
    if (!active) return;
    for (int x = lane; x < RPW * OCPR; x += 64) {
        const int row = x / OCPR, ch = x - row * OCPR;
        const int r = wr0 + row;
        if (r >= it.row_end) continue;
        const int tok = div_g(a, r);
        const int h = j * g + (r - tok * g);
        uint8_t *dst = static_cast<uint8_t *>(a.out) + (((int64_t)tok_index(a, qs0, tok) * a.num_q_heads + h) * D) * ELT;
        reinterpret_cast<u32x4 *>(dst)[ch] = *reinterpret_cast<const u32x4 *>(staged(row, ch * 16));
    }
}

template <class DT, int D, int TK, int OCC, int RPW>
__global__ __launch_bounds__(256, OCC) void ps_prefill_kernel(const ps_attn_launch a) {
    __shared__ PrefillLds<DT, D, TK> L;
    prefill_item<DT, D, TK, RPW>(a, blockIdx.x, L);
}

// Decode and prefill items of one step in a single launch, so that the
// memory-bound decode items and the MFMA-bound prefill items share the
// CUs instead of running one kernel after the other. Block b < 2 min(nd,
// np) alternates decode / prefill items, the remaining blocks take what is
// left. Decode items run 4 waves. Workgroups go to the 8 XCDs round-robin
// by block index, so in the alternating part the decode items run on the
// even XCDs and the prefill items on the odd ones: the prefill items,
// which read the same keys (one chunk's context, or a shared prefix),
// then share four L2s. Mappings that give every XCD both kinds (runs of 8
// or 256 blocks) measured 0-3% slower.
// When prefill items outnumber decode items two to one or more, the
// decode items are instead spread evenly over the launch in rounds of 8
// blocks (one block per XCD; whole rounds of one kind, in Bresenham
// proportion; the last nd % 8 and np % 8 items close the launch). Then
// every round of resident items keeps some HBM reads running under the
// MFMA work, instead of all of them running in the first rounds (C5 -1%;
// with fewer prefill items it is slower: C3 +2%, C4 +17%).
template <class DT, int D, int RT, bool STREAM, bool FUSE>
__global__ __launch_bounds__(256, 2) void ps_mixed_kernel(const ps_attn_launch a) {
    __shared__ union {
        DecodeLds<DT, D, RT, 4> d;
        PrefillLds<DT, D, PS_PRE_TILE> p;
    } L;
    const int nd = a.n_decode, np = a.n_prefill, m = min(nd, np);
    const int b = blockIdx.x;
    bool dec;
    int idx;
    if (np >= 2 * nd) {
        const int nd8 = nd >> 3, np8 = np >> 3, R = nd8 + np8;
        if (b < 8 * R) {
            const int r = b >> 3, x = b & 7;
            const int before = (int)((int64_t)r * nd8 / R), upto = (int)((int64_t)(r + 1) * nd8 / R);
            dec = upto > before;
            idx = (dec ? before : r - before) * 8 + x;
        } else {
            const int bb = b - 8 * R, dr = nd - 8 * nd8;
            dec = bb < dr;
            idx = dec ? 8 * nd8 + bb : 8 * np8 + (bb - dr);
        }
    } else {
        dec = b < 2 * m ? (b & 1) == 0 : nd > np;
        idx = b < 2 * m ? b >> 1 : m + (b - 2 * m);
    }
    if (dec) {
        // Decode waves run at the prefill waves' MFMA level throughout,
        // above their softmax phases: the few instructions between a decode
        // wave's loads then issue promptly and keep its loads flowing.
        __builtin_amdgcn_s_setprio(1);
        decode_item<DT, D, RT, 4, STREAM, FUSE>(a, idx, L.d);
    } else {
        prefill_item<DT, D, PS_PRE_TILE, 32>(a, idx, L.p);
    }
}

// ---------------------------------------------------------------------------
// Split-K merge: out = sum_i acc_i 2^(m_i - M) / sum_i l_i 2^(m_i - M),
// M = max_i m_i. One workgroup per chunk of rows of one split set; each
// thread owns 4 consecutive elements of one row.

template <class DT, int D>
__global__ __launch_bounds__(256) void ps_merge_kernel(const ps_attn_launch a) {
    using T = typename DT::T;
    const ps_merge mg = a.merges[blockIdx.x];
    if (mg.seq < 0) return;   // an idle merge of a fixed-shape launch
    const int qs0 = a.query_start_loc[mg.seq];
    const int row = threadIdx.x / (D / 4), d0 = (threadIdx.x % (D / 4)) * 4;
    const int r = mg.row_begin + row;
    if (r >= mg.row_end) return;
    const int g = a.g;
    const int64_t p0 = (int64_t)mg.partial_row + row;
    const int ns = mg.num_splits;
    float M = kNegInf, L = 0.f;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    constexpr int MS = 8;
    if (ns <= MS) {
        // Every split's (m, l, acc) in one batch of loads, so the merge
        // waits for memory once. Slots past the split count re-read split
        // 0 (in bounds, finite) and take a zero weight: the sums are the
        // same, term for term, as in the loop below.
        float mv[MS], lv[MS];
        f32x4 av[MS];
#pragma unroll
        for (int sp = 0; sp < MS; ++sp) {
            const int64_t pr = p0 + (int64_t)(sp < ns ? sp : 0) * mg.split_stride;
            mv[sp] = a.ws_m[pr];
            lv[sp] = a.ws_l[pr];
            av[sp] = *reinterpret_cast<const f32x4 *>(a.ws_acc + pr * D + d0);
        }
#pragma unroll
        for (int sp = 0; sp < MS; ++sp) M = sp < ns ? fmaxf(M, mv[sp]) : M;
        const float muse = M == kNegInf ? 0.f : M;
#pragma unroll
        for (int sp = 0; sp < MS; ++sp) {
            const float f = sp < ns ? fast_exp2(mv[sp] - muse) : 0.f;
            L += lv[sp] * f;
            acc += av[sp] * f;
        }
    } else {
        for (int sp = 0; sp < ns; ++sp) M = fmaxf(M, a.ws_m[p0 + (int64_t)sp * mg.split_stride]);
        const float muse = M == kNegInf ? 0.f : M;
        for (int sp = 0; sp < ns; ++sp) {
            const int64_t pr = p0 + (int64_t)sp * mg.split_stride;
            const float f = fast_exp2(a.ws_m[pr] - muse);
            L += a.ws_l[pr] * f;
            acc += *reinterpret_cast<const f32x4 *>(a.ws_acc + pr * D + d0) * f;
        }
    }
    const int tok = div_g(a, r);
    const int h = mg.kv_head * g + (r - tok * g);
    T *op = static_cast<T *>(a.out) + ((int64_t)tok_index(a, qs0, tok) * a.num_q_heads + h) * D + d0;
    const float inv = 1.f / L;
#pragma unroll
    for (int e = 0; e < 4; ++e) op[e] = cvt_out(acc[e] * inv, DT{});
}

// ---------------------------------------------------------------------------
// Launchers

}  // namespace psk

namespace psk {

// Launches of one attention call. Kernel shapes: decode items of one row
// tile run 4, 8 or 16 waves (the plan's choice), of two row tiles 4 waves;
// prefill items 4 waves of 32 rows over 64-key tiles (32-key tiles for
// fp32) in a two-stage LDS ring; a step with both kinds runs them in one
// launch unless the plan asks for two.
template <class DT, int D>
hipError_t launch_attention_t(const ps_attn_launch &a, hipStream_t st) {
    if constexpr (DT::ELT == 2) {
        if (a.n_decode > 0 && a.n_prefill > 0 && a.mixed) {
            const dim3 grid(a.n_decode + a.n_prefill), block(256);
            // (a mixed launch fuses the scatter only next to shared-prefix
            // items, so most mixed launches take the variant without it)
            auto mixed = [&](auto rtc, auto streamc, auto fusec) {
                hipLaunchKernelGGL((ps_mixed_kernel<DT, D, decltype(rtc)::value, decltype(streamc)::value,
                                                    decltype(fusec)::value>), grid, block, 0, st, a);
            };
            using R1 = std::integral_constant<int, 1>;
            using R2 = std::integral_constant<int, 2>;
            auto by_fuse = [&](auto rtc, auto streamc) {
                if (a.fuse_scatter) mixed(rtc, streamc, std::true_type{});
                else mixed(rtc, streamc, std::false_type{});
            };
            auto by_stream = [&](auto rtc) {
                if (a.stream_kv) by_fuse(rtc, std::true_type{});
                else by_fuse(rtc, std::false_type{});
            };
            if (a.decode_row_tiles == 2) by_stream(R2{});
            else by_stream(R1{});
            if (a.n_merge > 0)
                hipLaunchKernelGGL((ps_merge_kernel<DT, D>), dim3(a.n_merge), dim3(256), 0, st, a);
            return hipGetLastError();
        }
    }
    if (a.n_decode > 0) {
        auto decode = [&](auto streamc) {
            constexpr bool STREAM = decltype(streamc)::value;
            if (a.decode_row_tiles == 2) {
                hipLaunchKernelGGL((ps_decode_kernel<DT, D, 2, 4, STREAM>), dim3(a.n_decode), dim3(256), 0, st, a);
            } else if (a.decode_waves >= 16 && D == 64 && DT::ELT == 2) {
                if constexpr (D == 64 && DT::ELT == 2)  // 16 waves fit the register budget only here
                    hipLaunchKernelGGL((ps_decode_kernel<DT, D, 1, 16, STREAM>), dim3(a.n_decode), dim3(1024), 0, st, a);
            } else if (a.decode_waves >= 8) {
                hipLaunchKernelGGL((ps_decode_kernel<DT, D, 1, 8, STREAM>), dim3(a.n_decode), dim3(512), 0, st, a);
            } else {
                hipLaunchKernelGGL((ps_decode_kernel<DT, D, 1, 4, STREAM>), dim3(a.n_decode), dim3(256), 0, st, a);
            }
        };
        if (a.stream_kv) decode(std::true_type{});
        else decode(std::false_type{});
    }
    if (a.n_prefill > 0) {
        const dim3 grid(a.n_prefill), block(256);
        if constexpr (DT::ELT == 4)
            hipLaunchKernelGGL((ps_prefill_kernel<DT, D, PS_PRE_TILE / 2, 2, 32>), grid, block, 0, st, a);
        else
            hipLaunchKernelGGL((ps_prefill_kernel<DT, D, PS_PRE_TILE, 2, 32>), grid, block, 0, st, a);
    }
    if (a.n_merge > 0)
        hipLaunchKernelGGL((ps_merge_kernel<DT, D>), dim3(a.n_merge), dim3(256), 0, st, a);
    return hipGetLastError();
}

template <class DT>
hipError_t launch_attention_d(const ps_attn_launch &a, hipStream_t st) {
    return a.head_dim == 64 ? launch_attention_t<DT, 64>(a, st) : launch_attention_t<DT, 128>(a, st);
}

}  // namespace psk

using namespace psk;

int ps_launch_attention(const ps_attn_launch &a, void *stream) {
    hipStream_t st = static_cast<hipStream_t>(stream);
    hipError_t e;
    switch (a.dtype) {
        case PS_F32: e = launch_attention_d<TF32>(a, st); break;
        case PS_F16: e = launch_attention_d<TF16>(a, st); break;
        default: e = launch_attention_d<TBF16>(a, st); break;
    }
    return (int)e;
}

// ---------------------------------------------------------------------------
// Static split-K workspace of ps_step_no_alloc: one array per GPU, held
// until the process ends. In host code `scratch` only names the symbol; its
// device address comes from hipGetSymbolAddress, looked up once per device
// with that device current, and only that address is handed to kernels.

static __device__ __align__(256) uint8_t scratch[PS_STATIC_WORKSPACE_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
void *g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];
}  // namespace

int ps_static_workspace(void **ptr) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return (int)e;
    if (dev < 0 || dev >= kMaxDevices) return (int)hipErrorInvalidDevice;
    std::call_once(g_scratch_once[dev], [dev] {
        void *p = nullptr;
        g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        g_scratch_ptr[dev] = p;
    });
    if (g_scratch_err[dev] != hipSuccess) return (int)g_scratch_err[dev];
    *ptr = g_scratch_ptr[dev];
    return 0;
}

int ps_launch_scatter(const void *k, const void *v, const int32_t *slot_mapping, int32_t num_tokens,
                      const ps_pool *pool, void *stream) {
    const int elt = pool->dtype == PS_F32 ? 4 : 2;
    const int64_t row_bytes = (int64_t)pool->num_kv_heads * pool->head_dim * elt;
    const int32_t row_words = (int32_t)(row_bytes / 16);
    const int64_t total = (int64_t)num_tokens * row_words;
    const int64_t layer_bytes = (int64_t)pool->num_blocks * PS_BLOCK * row_bytes;
    u32x4 *pk = reinterpret_cast<u32x4 *>(static_cast<uint8_t *>(pool->k) + pool->layer * layer_bytes);
    u32x4 *pv = reinterpret_cast<u32x4 *>(static_cast<uint8_t *>(pool->v) + pool->layer * layer_bytes);
    const int64_t blocks = (total + 255) / 256;
    hipLaunchKernelGGL(ps_scatter_kernel, dim3((unsigned)blocks), dim3(256), 0,
                       static_cast<hipStream_t>(stream), static_cast<const u32x4 *>(k),
                       static_cast<const u32x4 *>(v), slot_mapping, total, row_words, pk, pv,
                       pool->num_blocks * PS_BLOCK);
    return (int)hipGetLastError();
}

int ps_launch_copy_blocks(const ps_pool *src, const ps_pool *dst, const int32_t *src_blocks,
                          const int32_t *dst_blocks, int32_t num_pairs, void *stream) {
    const int elt = src->dtype == PS_F32 ? 4 : 2;
    const int32_t block_words = (int32_t)((int64_t)PS_BLOCK * src->num_kv_heads * src->head_dim * elt / 16);
    hipLaunchKernelGGL(ps_copy_blocks_kernel, dim3((unsigned)(num_pairs * src->num_layers)), dim3(256), 0,
                       static_cast<hipStream_t>(stream), static_cast<const u32x4 *>(src->k),
                       static_cast<const u32x4 *>(src->v), static_cast<u32x4 *>(dst->k),
                       static_cast<u32x4 *>(dst->v), src_blocks, dst_blocks, src->num_layers,
                       src->num_blocks, dst->num_blocks, block_words);
    return (int)hipGetLastError();
}

const char *ps_hip_error_string(int err) { return hipGetErrorString((hipError_t)err); }
