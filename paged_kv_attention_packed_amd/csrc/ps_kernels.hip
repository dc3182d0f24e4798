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

#include <type_traits>

#include "ps_internal.h"

namespace {

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

// two fp32 -> packed pair of 16-bit values (low half = first)
__device__ inline uint32_t pack2(float x, float y, TF16) {
    return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)x) |
           ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)y) << 16);
}
__device__ inline uint32_t pack2(float x, float y, TBF16) {
    return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)x) |
           ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)y) << 16);
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

__device__ inline float xor_max(float x) {
    x = fmaxf(x, __shfl_xor(x, 16));
    return fmaxf(x, __shfl_xor(x, 32));
}
__device__ inline float xor_sum(float x) {
    x += __shfl_xor(x, 16);
    return x + __shfl_xor(x, 32);
}

// N consecutive 32-bit words from a 4*N-byte aligned address
template <int N>
__device__ inline void load_words(const void *p, uint32_t (&w)[N]) {
    if constexpr (N == 2) {
        const u32x2 x = *reinterpret_cast<const u32x2 *>(p);
        w[0] = x[0];
        w[1] = x[1];
    } else {
        static_assert(N % 4 == 0, "word count");
#pragma unroll
        for (int i = 0; i < N / 4; ++i) {
            const u32x4 x = reinterpret_cast<const u32x4 *>(p)[i];
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

// Online-softmax update of one row tile for 8*NSB scores already in
// log2 units; returns the probabilities in pv.
template <int NS>
__device__ inline void softmax_update(float (&sv)[NS], float &m, float &l, float &alpha) {
    float tmax = kNegInf;
#pragma unroll
    for (int e = 0; e < NS; ++e) tmax = fmaxf(tmax, sv[e]);
    tmax = xor_max(tmax);
    const float mnew = fmaxf(m, tmax);
    const float muse = mnew == kNegInf ? 0.f : mnew;
    alpha = fast_exp2(m - muse);
    float psum = 0.f;
#pragma unroll
    for (int e = 0; e < NS; ++e) {
        sv[e] = fast_exp2(sv[e] - muse);
        psum += sv[e];
    }
    l = l * alpha + psum;
    m = mnew;
}

// Which query row a lane's packed row stands for, its visibility limit and
// its Q fragment.
template <class DT, int D>
__device__ inline void load_q_row(const ps_attn_launch &a, int r, int row_end, int g, int kv_head,
                                  int qs0, int nc, int q4, u32x4 (&qf)[Geo<DT, D>::KU4], int &lim) {
    if (r < row_end) {
        const int tok = r / g;
        const int h = kv_head * g + (r - tok * g);
        lim = nc + tok;
        const typename DT::T *qp =
            static_cast<const typename DT::T *>(a.q) + ((int64_t)(qs0 + tok) * a.num_q_heads + h) * D;
#pragma unroll
        for (int u = 0; u < Geo<DT, D>::KU4; ++u)
            qf[u] = *reinterpret_cast<const u32x4 *>(qp + (u * 4 + q4) * (16 / DT::ELT));
    } else {
        lim = -1;
#pragma unroll
        for (int u = 0; u < Geo<DT, D>::KU4; ++u) qf[u] = u32x4{0u, 0u, 0u, 0u};
    }
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
// Decode / verify attention. One workgroup = one work item (sequence, KV
// head, <= RT*16 packed rows, key slice). Its 4 waves take 32-key tiles of
// the slice round-robin, each double-buffering the next tile's K/V in
// registers, then merge their softmax states through LDS.

template <class DT, int D, int RT>
__global__ __launch_bounds__(256, 2) void ps_decode_kernel(const ps_attn_launch a) {
    using G = Geo<DT, D>;
    using T = typename DT::T;
    constexpr int ELT = G::ELT, KU4 = G::KU4, VW = G::VW, NT = G::NT, EPL = G::EPL;
    constexpr int ROWS = RT * 16;

    __shared__ float sm_o[PS_DEC_WAVES][ROWS][D];
    __shared__ float sm_m[PS_DEC_WAVES][ROWS];
    __shared__ float sm_l[PS_DEC_WAVES][ROWS];

    const ps_item it = a.decode_items[blockIdx.x];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: keeps tile math scalar
    const int c = lane & 15, q4 = lane >> 4;
    const int s = it.seq, j = it.kv_head;
    const int g = a.num_q_heads / a.num_kv_heads;
    const int qs0 = a.query_start_loc[s], nc = a.num_computed[s];
    const int32_t *bt = a.block_tables + (int64_t)s * a.bt_stride;
    const int64_t rs = (int64_t)a.num_kv_heads * D;  // elements from one slot to the next
    const T *kp = static_cast<const T *>(a.pool_k) + a.layer_offset + (int64_t)j * D;
    const T *vp = static_cast<const T *>(a.pool_v) + a.layer_offset + (int64_t)j * D;
    const int kb = it.key_begin, ke = it.key_end;

    u32x4 qf[RT][KU4];
    int lim[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
        load_q_row<DT, D>(a, it.row_begin + rt * 16 + c, it.row_end, g, j, qs0, nc, q4, qf[rt], lim[rt]);

    float m[RT], l[RT];
    f32x4 o[RT][NT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        m[rt] = kNegInf;
        l[rt] = 0.f;
#pragma unroll
        for (int t = 0; t < NT; ++t) o[rt][t] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    constexpr bool DOUBLE_BUFFER = RT == 1;
    constexpr int NBUF = DOUBLE_BUFFER ? 2 : 1;
    u32x4 kf[NBUF][2][KU4];
    uint32_t vr[NBUF][8][VW];

    // K/V of keys [k0, k0 + 32): two pool blocks. Block ids are read with
    // scalar loads (k0 is wave-uniform), so the vector loads never wait on
    // each other. Rows of an existing block past key_end are loaded (they
    // are in bounds) and zeroed or masked at use.
    auto load_tile = [&](auto bufc, int k0) {
        constexpr int buf = decltype(bufc)::value;
        const bool has1 = k0 + 16 < ke;
        const int64_t blk0 = bt[k0 >> 4];
        const int64_t blk1 = has1 ? (int64_t)bt[(k0 >> 4) + 1] : blk0;
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
            const int64_t blk = sb ? blk1 : blk0;
            if (sb == 0 || has1) {
                const T *p = kp + (blk * 16 + c) * rs;
#pragma unroll
                for (int u = 0; u < KU4; ++u)
                    kf[buf][sb][u] = *reinterpret_cast<const u32x4 *>(p + (u * 4 + q4) * (16 / ELT));
            } else {
#pragma unroll
                for (int u = 0; u < KU4; ++u) kf[buf][sb][u] = u32x4{0u, 0u, 0u, 0u};
            }
        }
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
            const int64_t blk = (jj >> 2) ? blk1 : blk0;
            load_words<VW>(vp + (blk * 16 + 4 * q4 + (jj & 3)) * rs + EPL * c, vr[buf][jj]);
        }
    };

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
                for (int i = 0; i < 4; ++i) {
                    const int key = k0 + sb * 16 + 4 * q4 + i;
                    const float x = sacc[sb][i] * a.scale_log2;
                    pv[rt][sb * 4 + i] = (key < ke && key <= lim[rt]) ? x : kNegInf;
                }
            float alpha;
            softmax_update(pv[rt], m[rt], l[rt], alpha);
#pragma unroll
            for (int t = 0; t < NT; ++t) o[rt][t] *= alpha;
        }
        if (k0 + PS_DEC_TILE > ke) {
            // ragged tile: V rows at or past key_end may be stale (even NaN)
            // and P = 0 there would not cancel them
#pragma unroll
            for (int jj = 0; jj < 8; ++jj) {
                const bool ok = k0 + (jj >> 2) * 16 + 4 * q4 + (jj & 3) < ke;
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
    const int ntiles = (ke - kb + PS_DEC_TILE - 1) / PS_DEC_TILE;
    int ti = wave;
    if constexpr (!DOUBLE_BUFFER) {
        // two row tiles leave no registers for a second tile in flight;
        // the other resident waves cover the load latency
        for (; ti < ntiles; ti += PS_DEC_WAVES) {
            load_tile(B0{}, kb + ti * PS_DEC_TILE);
            compute_tile(B0{}, kb + ti * PS_DEC_TILE);
        }
    }
    if constexpr (DOUBLE_BUFFER) {
        if (ti < ntiles) load_tile(B0{}, kb + ti * PS_DEC_TILE);
        while (ti < ntiles) {
            if (ti + PS_DEC_WAVES < ntiles) load_tile(B1{}, kb + (ti + PS_DEC_WAVES) * PS_DEC_TILE);
            compute_tile(B0{}, kb + ti * PS_DEC_TILE);
            ti += PS_DEC_WAVES;
            if (ti >= ntiles) break;
            if (ti + PS_DEC_WAVES < ntiles) load_tile(B0{}, kb + (ti + PS_DEC_WAVES) * PS_DEC_TILE);
            compute_tile(B1{}, kb + ti * PS_DEC_TILE);
            ti += PS_DEC_WAVES;
        }
    }

    // ---- merge the 4 waves' states
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        l[rt] = xor_sum(l[rt]);
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) sm_o[wave][rt * 16 + c][EPL * (4 * q4 + i) + t] = o[rt][t][i];
        if (q4 == 0) {
            sm_m[wave][rt * 16 + c] = m[rt];
            sm_l[wave][rt * 16 + c] = l[rt];
        }
    }
    __syncthreads();

    constexpr int EPT = ROWS * D / 256;  // output elements per thread
    const int e0 = tid * EPT;
    const int row = e0 / D, d0 = e0 % D;
    const int r = it.row_begin + row;
    if (r >= it.row_end) return;
    float mw[PS_DEC_WAVES], M = kNegInf;
#pragma unroll
    for (int w = 0; w < PS_DEC_WAVES; ++w) {
        mw[w] = sm_m[w][row];
        M = fmaxf(M, mw[w]);
    }
    const float muse = M == kNegInf ? 0.f : M;
    float L = 0.f, acc[EPT];
#pragma unroll
    for (int e = 0; e < EPT; ++e) acc[e] = 0.f;
#pragma unroll
    for (int w = 0; w < PS_DEC_WAVES; ++w) {
        const float f = fast_exp2(mw[w] - muse);
        L += sm_l[w][row] * f;
#pragma unroll
        for (int e = 0; e < EPT; ++e) acc[e] += sm_o[w][row][d0 + e] * f;
    }
    if (it.partial_row < 0) {
        const int tok = r / g;
        const int h = j * g + (r - tok * g);
        T *op = static_cast<T *>(a.out) + ((int64_t)(qs0 + tok) * a.num_q_heads + h) * D + d0;
        const float inv = 1.f / L;
#pragma unroll
        for (int e = 0; e < EPT; ++e) op[e] = cvt_out(acc[e] * inv, DT{});
    } else {
        const int64_t pr = (int64_t)it.partial_row + row;
#pragma unroll
        for (int e = 0; e < EPT; ++e) {
            const int d = d0 + e;
            a.ws_acc[pr * D + (d % EPL) * 16 + d / EPL] = acc[e];
        }
        if (d0 == 0) {
            a.ws_m[pr] = M;
            a.ws_l[pr] = L;
        }
    }
}

// ---------------------------------------------------------------------------
// Prefill-chunk attention. One workgroup = 128 packed rows (4 waves x 32)
// of one sequence and KV head over a key slice. 64-key K and V tiles are
// gathered through the block table into LDS (rows padded by 16 bytes so the
// per-key fragment reads are bank-conflict free), the next tile's loads are
// in flight in registers while the current one is consumed.

template <class DT, int D>
__global__ __launch_bounds__(256, 2) void ps_prefill_kernel(const ps_attn_launch a) {
    using G = Geo<DT, D>;
    using T = typename DT::T;
    constexpr int ELT = G::ELT, KU4 = G::KU4, VW = G::VW, NT = G::NT, EPL = G::EPL;
    constexpr int RT = PS_PRE_ROWS_PER_WAVE / 16;
    constexpr int TK = PS_PRE_TILE;
    constexpr int ROWB = D * ELT + 16;        // LDS bytes per key row (padded)
    constexpr int CPR = D * ELT / 16;         // 16-byte chunks per key row
    constexpr int CPT = 2 * TK * CPR / 256;   // chunks per thread per K+V tile
    constexpr int NSB = TK / 16;

    __shared__ __attribute__((aligned(16))) uint8_t smem[2 * TK * ROWB];
    uint8_t *const ksm = smem;
    uint8_t *const vsm = smem + TK * ROWB;

    const ps_item it = a.prefill_items[blockIdx.x];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int c = lane & 15, q4 = lane >> 4;
    const int s = it.seq, j = it.kv_head;
    const int g = a.num_q_heads / a.num_kv_heads;
    const int qs0 = a.query_start_loc[s], nc = a.num_computed[s];
    const int32_t *bt = a.block_tables + (int64_t)s * a.bt_stride;
    const int64_t rs = (int64_t)a.num_kv_heads * D;
    const T *kp = static_cast<const T *>(a.pool_k) + a.layer_offset + (int64_t)j * D;
    const T *vp = static_cast<const T *>(a.pool_v) + a.layer_offset + (int64_t)j * D;
    const int kb = it.key_begin, ke = it.key_end;

    const int wr0 = it.row_begin + wave * PS_PRE_ROWS_PER_WAVE;
    const bool active = wr0 < it.row_end;
    const int wr_last = min(wr0 + PS_PRE_ROWS_PER_WAVE, it.row_end) - 1;
    const int lim_lo = nc + wr0 / g;      // smallest visibility limit among the wave's rows
    const int lim_hi = nc + wr_last / g;  // largest

    u32x4 qf[RT][KU4];
    int lim[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
        load_q_row<DT, D>(a, wr0 + rt * 16 + c, it.row_end, g, j, qs0, nc, q4, qf[rt], lim[rt]);

    float m[RT], l[RT];
    f32x4 o[RT][NT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        m[rt] = kNegInf;
        l[rt] = 0.f;
#pragma unroll
        for (int t = 0; t < NT; ++t) o[rt][t] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    u32x4 pf[CPT];
    // one K+V tile = 4 pool blocks; their ids are scalar loads (k0 is
    // uniform). Chunks of blocks past key_end read block 0 of the tile
    // (always in bounds) and, like rows past key_end, are zeroed when the
    // tile is stored to LDS, so the loads never wait on each other.
    auto load_tile = [&](int k0) {
        int64_t blk[NSB];
        blk[0] = bt[k0 >> 4];
#pragma unroll
        for (int b = 1; b < NSB; ++b) blk[b] = (k0 + 16 * b < ke) ? (int64_t)bt[(k0 >> 4) + b] : blk[0];
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            const int x = tid + i * 256;
            const int kv = x / (TK * CPR);
            const int rem = x - kv * (TK * CPR);
            const int key = rem / CPR, ch = rem - key * CPR;
            int64_t b = blk[0];
#pragma unroll
            for (int q = 1; q < NSB; ++q) b = (key >> 4) == q ? blk[q] : b;
            const T *src = (kv ? vp : kp) + (b * 16 + (key & 15)) * rs;
            pf[i] = reinterpret_cast<const u32x4 *>(src)[ch];
        }
    };
    auto store_tile = [&](int k0) {
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            const int x = tid + i * 256;
            const int kv = x / (TK * CPR);
            const int rem = x - kv * (TK * CPR);
            const int key = rem / CPR, ch = rem - key * CPR;
            *reinterpret_cast<u32x4 *>((kv ? vsm : ksm) + key * ROWB + ch * 16) =
                (k0 + key < ke) ? pf[i] : u32x4{0u, 0u, 0u, 0u};
        }
    };

    auto compute_tile = [&](int k0) {
        const bool full = (k0 + TK <= ke) && (k0 + TK - 1 <= lim_lo);
        f32x4 sacc[RT][NSB];
#pragma unroll
        for (int sb = 0; sb < NSB; ++sb) {
            u32x4 kf[KU4];
            const uint8_t *kr = ksm + (sb * 16 + c) * ROWB + q4 * 16;
#pragma unroll
            for (int u = 0; u < KU4; ++u) kf[u] = *reinterpret_cast<const u32x4 *>(kr + u * 64);
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) sacc[rt][sb] = qk_tile<DT, D>(kf, qf[rt]);
        }
        float pv[RT][4 * NSB];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
#pragma unroll
            for (int sb = 0; sb < NSB; ++sb)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float x = sacc[rt][sb][i] * a.scale_log2;
                    if (!full) {
                        const int key = k0 + sb * 16 + 4 * q4 + i;
                        x = (key < ke && key <= lim[rt]) ? x : kNegInf;
                    }
                    pv[rt][sb * 4 + i] = x;
                }
            float alpha;
            softmax_update(pv[rt], m[rt], l[rt], alpha);
#pragma unroll
            for (int t = 0; t < NT; ++t) o[rt][t] *= alpha;
        }
        // P.V over two 32-key halves
#pragma unroll
        for (int h = 0; h < NSB / 2; ++h) {
            uint32_t vr[8][VW];
#pragma unroll
            for (int jj = 0; jj < 8; ++jj) {
                const int key = (2 * h + (jj >> 2)) * 16 + 4 * q4 + (jj & 3);
                load_words<VW>(vsm + key * ROWB + EPL * c * ELT, vr[jj]);
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
    };

    const int ntiles = (ke - kb + TK - 1) / TK;
    if (ntiles > 0) load_tile(kb);
    for (int ti = 0; ti < ntiles; ++ti) {
        const int k0 = kb + ti * TK;
        __syncthreads();
        store_tile(k0);
        __syncthreads();
        if (ti + 1 < ntiles) load_tile(k0 + TK);
        if (active && k0 <= lim_hi) compute_tile(k0);
    }

#pragma unroll
    for (int rt = 0; rt < RT; ++rt) l[rt] = xor_sum(l[rt]);

    if (it.partial_row >= 0) {
        if (!active) return;
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            const int r = wr0 + rt * 16 + c;
            if (r >= it.row_end) continue;
            const int64_t pr = (int64_t)it.partial_row + (r - it.row_begin);
#pragma unroll
            for (int t = 0; t < NT; ++t) *reinterpret_cast<f32x4 *>(a.ws_acc + pr * D + t * 16 + 4 * q4) = o[rt][t];
            if (q4 == 0) {
                a.ws_m[pr] = m[rt];
                a.ws_l[pr] = l[rt];
            }
        }
        return;
    }

    // final output: normalise, round, transpose through LDS, write rows
    __syncthreads();
    T *so = reinterpret_cast<T *>(smem) + wave * PS_PRE_ROWS_PER_WAVE * D;
    if (active) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            const float inv = l[rt] > 0.f ? 1.f / l[rt] : 0.f;
#pragma unroll
            for (int t = 0; t < NT; ++t)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    so[(rt * 16 + c) * D + EPL * (4 * q4 + i) + t] = cvt_out(o[rt][t][i] * inv, DT{});
        }
    }
    __syncthreads();
    if (!active) return;
    const uint8_t *sob = reinterpret_cast<const uint8_t *>(so);
    for (int x = lane; x < PS_PRE_ROWS_PER_WAVE * CPR; x += 64) {
        const int row = x / CPR, ch = x - row * CPR;
        const int r = wr0 + row;
        if (r >= it.row_end) continue;
        const int tok = r / g;
        const int h = j * g + (r - tok * g);
        uint8_t *dst = static_cast<uint8_t *>(a.out) + (((int64_t)(qs0 + tok) * a.num_q_heads + h) * D) * ELT;
        reinterpret_cast<u32x4 *>(dst)[ch] = *reinterpret_cast<const u32x4 *>(sob + row * D * ELT + ch * 16);
    }
}

// ---------------------------------------------------------------------------
// Split-K merge: out = sum_i acc_i 2^(m_i - M) / sum_i l_i 2^(m_i - M).

template <class DT, int D>
__global__ __launch_bounds__(256) void ps_merge_kernel(const ps_attn_launch a) {
    using T = typename DT::T;
    constexpr int EPL = D / 16;
    constexpr int CH = 8;
    const ps_merge mg = a.merges[blockIdx.x];
    const int rows = mg.row_end - mg.row_begin;
    const int g = a.num_q_heads / a.num_kv_heads;
    const int qs0 = a.query_start_loc[mg.seq];
    for (int u = threadIdx.x; u < rows * (D / CH); u += 256) {
        const int row = u / (D / CH), d0 = (u - row * (D / CH)) * CH;
        float M = kNegInf;
        for (int sp = 0; sp < mg.num_splits; ++sp)
            M = fmaxf(M, a.ws_m[(int64_t)mg.partial_row + (int64_t)sp * rows + row]);
        const float muse = M == kNegInf ? 0.f : M;
        float L = 0.f, acc[CH];
#pragma unroll
        for (int e = 0; e < CH; ++e) acc[e] = 0.f;
        for (int sp = 0; sp < mg.num_splits; ++sp) {
            const int64_t pr = (int64_t)mg.partial_row + (int64_t)sp * rows + row;
            const float f = fast_exp2(a.ws_m[pr] - muse);
            L += a.ws_l[pr] * f;
            const float *ap = a.ws_acc + pr * D;
#pragma unroll
            for (int e = 0; e < CH; ++e) {
                const int d = d0 + e;
                acc[e] += ap[(d % EPL) * 16 + d / EPL] * f;
            }
        }
        const int r = mg.row_begin + row;
        const int tok = r / g;
        const int h = mg.kv_head * g + (r - tok * g);
        T *op = static_cast<T *>(a.out) + ((int64_t)(qs0 + tok) * a.num_q_heads + h) * D + d0;
        const float inv = 1.f / L;
#pragma unroll
        for (int e = 0; e < CH; ++e) op[e] = cvt_out(acc[e] * inv, DT{});
    }
}

// ---------------------------------------------------------------------------
// Launchers

template <class DT, int D>
hipError_t launch_attention_t(const ps_attn_launch &a, hipStream_t st) {
    if (a.n_decode > 0) {
        if (a.decode_row_tiles == 1)
            hipLaunchKernelGGL((ps_decode_kernel<DT, D, 1>), dim3(a.n_decode), dim3(256), 0, st, a);
        else
            hipLaunchKernelGGL((ps_decode_kernel<DT, D, 2>), dim3(a.n_decode), dim3(256), 0, st, a);
    }
    if (a.n_prefill > 0)
        hipLaunchKernelGGL((ps_prefill_kernel<DT, D>), dim3(a.n_prefill), dim3(256), 0, st, a);
    if (a.n_merge > 0)
        hipLaunchKernelGGL((ps_merge_kernel<DT, D>), dim3(a.n_merge), dim3(256), 0, st, a);
    return hipGetLastError();
}

template <class DT>
hipError_t launch_attention_d(const ps_attn_launch &a, hipStream_t st) {
    return a.head_dim == 64 ? launch_attention_t<DT, 64>(a, st) : launch_attention_t<DT, 128>(a, st);
}

}  // namespace

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

const char *ps_hip_error_string(int err) { return hipGetErrorString((hipError_t)err); }
