// Rotary position embedding fused with the KV scatter, for gfx950.
//
// The Qwen2 forward pass rotates q and k by their token positions before
// attention (tinyserve README, "Highlights"); in a packed step every token
// carries an explicit position and a slot (PageServe "01 Scheduler loop",
// Pack). One pass over the step's new rows does both: q is rotated into
// q_out, k is rotated straight into its pool slot and v is copied there,
// so the rotated k never makes a round trip through HBM.
//
// Rotation: the pair (x[j], x[j + D/2]) turns by a = pos * theta^(-2j/D).
// The angle is an fp64 product (the frequency comes from the host in fp64)
// and cos / sin are taken in fp64, since at positions of 10^5 and beyond an
// fp32 angle alone would be off by more than a bf16 ulp; the rotation
// itself is fp32 and the result is rounded to the storage type.
//
// Work split: a workgroup of 256 threads owns as many tokens as keep every
// thread at <= 2 units, a unit being a 16-byte chunk at d and its partner
// at d + D/2 of one q or k head (eight threads cover the two 128-byte
// halves of a bf16 head of 128), or one 16-byte word of a v row. A thread
// issues all of its loads up front, then computes up to two of the
// tokens' (cos, sin) pairs into LDS while those loads are in flight, and
// only then rotates and stores: one memory round trip per thread, with
// the fp64 angle math hidden under it. A token with more than 512 units
// (e.g. 64 query heads of 128) takes a workgroup of its own, whose
// threads finish the units past the first 512 one at a time. q_out may
// alias q: a thread reads and writes only its own chunks, reads first.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ps_internal.h"

namespace psr {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

struct RF32 { static constexpr int ELT = 4; };
struct RF16 { static constexpr int ELT = 2; };
struct RBF16 { static constexpr int ELT = 2; };

// 16 bytes -> elements as fp32
__device__ inline void unpack(u32x4 w, float *x, RF32) {
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = __builtin_bit_cast(float, (uint32_t)w[i]);
}
__device__ inline void unpack(u32x4 w, float *x, RF16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t u = w[i];
        x[2 * i] = (float)__builtin_bit_cast(_Float16, (uint16_t)(u & 0xffffu));
        x[2 * i + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(u >> 16));
    }
}
__device__ inline void unpack(u32x4 w, float *x, RBF16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t u = w[i];
        x[2 * i] = __builtin_bit_cast(float, u << 16);
        x[2 * i + 1] = __builtin_bit_cast(float, u & 0xffff0000u);
    }
}

// fp32 elements -> 16 bytes, round to nearest even
__device__ inline u32x4 pack(const float *y, RF32) {
    u32x4 w;
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = __builtin_bit_cast(uint32_t, y[i]);
    return w;
}
__device__ inline u32x4 pack(const float *y, RF16) {
    u32x4 w;
#pragma unroll
    for (int i = 0; i < 4; ++i)
        w[i] = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)y[2 * i]) |
               ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)y[2 * i + 1]) << 16);
    return w;
}
__device__ inline u32x4 pack(const float *y, RBF16) {
    u32x4 w;
#pragma unroll
    for (int i = 0; i < 4; ++i)
        w[i] = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)y[2 * i]) |
               ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)y[2 * i + 1]) << 16);
    return w;
}

// Units a thread owns: a unit is one (head, 16-byte chunk) pair of a q or k
// row to rotate, or one 16-byte word of a v row to copy.
constexpr int kUnitsPerThread = 2;
// Angles a thread computes: tokens_per_wg * D / 2 <= 512.
constexpr int kAnglesPerThread = 2;

template <class DT, int D>
__global__ __launch_bounds__(256) void ps_rope_cache_kernel(const ps_rope_launch a) {
    constexpr int HALF = D / 2;
    constexpr int CH = 16 / DT::ELT;   // elements per 16-byte chunk
    constexpr int HC = HALF / CH;      // chunks per half row
    constexpr int ROW_W = D / CH;      // 16-byte words per head row
    __shared__ float2 cs[kAnglesPerThread * 256];

    const int tpb = a.tokens_per_wg;
    const int64_t t0 = (int64_t)blockIdx.x * tpb;
    const int n_tok = (int)min<int64_t>(tpb, a.num_tokens - t0);
    const int Hq = a.num_q_heads, Hkv = a.num_kv_heads;
    const int q_units = Hq * HC;
    const int rot_units = (Hq + Hkv) * HC;
    const int v_words = Hkv * ROW_W;
    const int per_tok = rot_units + v_words;
    const int n_units = n_tok * per_tok;
    const int n_angles = n_tok * HALF;

    // 1. positions first, so that the angle math below can start while the
    //    data loads are still in flight. Loads are branch-free: indexes are
    //    clamped into range and the unused results ignored, so that no
    //    load waits on another at a control-flow join.
    int32_t pos[kAnglesPerThread];
    double freq[kAnglesPerThread];
#pragma unroll
    for (int i = 0; i < kAnglesPerThread; ++i) {
        const int idx = min((int)threadIdx.x + 256 * i, n_angles - 1);
        pos[i] = a.positions[t0 + idx / HALF];
        freq[i] = a.inv_freq[idx % HALF];
    }

    // 2. every load of this thread's first units
    const u32x4 *q = static_cast<const u32x4 *>(a.q);
    const u32x4 *k = static_cast<const u32x4 *>(a.k);
    const u32x4 *v = static_cast<const u32x4 *>(a.v);
    // unit u of the workgroup: its source words, kind, destination word
    // and first angle
    auto describe = [&](int u, const u32x4 *&src, int &hi_off, int64_t &t, int &kind, int64_t &dst, int &cbase) {
        const int tok = u / per_tok;
        const int r = u - tok * per_tok;
        t = t0 + tok;
        const bool rot = r < rot_units;
        const int head = r / HC;
        const int c = r - head * HC;
        const bool isq = head < Hq;
        const int64_t qw = (t * Hq + head) * ROW_W + c;
        const int64_t kw = (t * Hkv + (head - Hq)) * ROW_W + c;
        const int64_t vw = t * v_words + (r - rot_units);
        src = rot ? (isq ? q + qw : k + kw) : v + vw;
        hi_off = rot ? HC : 0;
        kind = rot ? (isq ? 1 : 2) : 3;
        dst = rot ? (isq ? qw : (int64_t)(head - Hq) * ROW_W + c) : (int64_t)(r - rot_units);
        cbase = tok * HALF + c * CH;
    };
    u32x4 lo[kUnitsPerThread], hi[kUnitsPerThread];
    int32_t slot[kUnitsPerThread];
    int kind[kUnitsPerThread];      // 0 none, 1 q, 2 k, 3 v
    int64_t dst[kUnitsPerThread];   // word index of the destination (k, v: within the slot row)
    int cbase[kUnitsPerThread];     // first angle of the chunk in cs
#pragma unroll
    for (int i = 0; i < kUnitsPerThread; ++i) {
        const int u0 = threadIdx.x + 256 * i;
        const u32x4 *src;
        int hi_off;
        int64_t t;
        describe(min(u0, n_units - 1), src, hi_off, t, kind[i], dst[i], cbase[i]);
        slot[i] = a.slots[t];
        lo[i] = src[0];
        hi[i] = src[hi_off];
        kind[i] = u0 >= n_units ? 0 : kind[i];
    }

    // 3. cos / sin of this workgroup's angles (fp64), shared through LDS
#pragma unroll
    for (int i = 0; i < kAnglesPerThread; ++i) {
        const int idx = threadIdx.x + 256 * i;
        if (idx < n_angles) {
            double sd, cd;
            sincos((double)pos[i] * freq[i], &sd, &cd);
            cs[idx] = make_float2((float)cd, (float)sd);
        }
    }
    __syncthreads();

    // 4. rotate and store
    u32x4 *q_out = static_cast<u32x4 *>(a.q_out);
    u32x4 *pk = static_cast<u32x4 *>(a.pool_k);
    u32x4 *pv = static_cast<u32x4 *>(a.pool_v);
    const uint32_t num_slots = (uint32_t)a.num_slots;
    auto finish = [&](int kd, int32_t sl, int64_t dw, int cb, u32x4 w_lo, u32x4 w_hi) {
        if (kd == 0) return;
        if (kd != 1 && (uint32_t)sl >= num_slots) return;
        if (kd == 3) {
            pv[(int64_t)sl * v_words + dw] = w_lo;
            return;
        }
        float x1[CH], x2[CH], y1[CH], y2[CH];
        unpack(w_lo, x1, DT{});
        unpack(w_hi, x2, DT{});
#pragma unroll
        for (int e = 0; e < CH; ++e) {
            const float2 f = cs[cb + e];
            y1[e] = x1[e] * f.x - x2[e] * f.y;
            y2[e] = x2[e] * f.x + x1[e] * f.y;
        }
        u32x4 *o = kd == 1 ? q_out + dw : pk + (int64_t)sl * v_words + dw;
        o[0] = pack(y1, DT{});
        o[HC] = pack(y2, DT{});
    };
#pragma unroll
    for (int i = 0; i < kUnitsPerThread; ++i) finish(kind[i], slot[i], dst[i], cbase[i], lo[i], hi[i]);

    // 5. a token of more units than two per thread (many heads) is one
    //    workgroup's alone; its remaining units go one by one
    for (int u = threadIdx.x + 256 * kUnitsPerThread; u < n_units; u += 256) {
        const u32x4 *src;
        int hi_off, kd, cb;
        int64_t t, dw;
        describe(u, src, hi_off, t, kd, dw, cb);
        const int32_t sl = a.slots[t];
        const u32x4 w_lo = src[0], w_hi = src[hi_off];
        finish(kd, sl, dw, cb, w_lo, w_hi);
    }
}

template <class DT, int D>
hipError_t launch_t(ps_rope_launch a, hipStream_t st) {
    constexpr int CH = 16 / DT::ELT;
    const int per_tok = (a.num_q_heads + a.num_kv_heads) * (D / 2 / CH) + a.num_kv_heads * (D / CH);
    int tpb = kUnitsPerThread * 256 / per_tok;
    tpb = tpb < 1 ? 1 : tpb;
    tpb = tpb > kAnglesPerThread * 256 / (D / 2) ? kAnglesPerThread * 256 / (D / 2) : tpb;
    a.tokens_per_wg = tpb;
    const unsigned grid = (unsigned)((a.num_tokens + tpb - 1) / tpb);
    hipLaunchKernelGGL((ps_rope_cache_kernel<DT, D>), dim3(grid), dim3(256), 0, st, a);
    return hipGetLastError();
}

template <class DT>
hipError_t launch_d(const ps_rope_launch &a, hipStream_t st) {
    return a.head_dim == 64 ? launch_t<DT, 64>(a, st) : launch_t<DT, 128>(a, st);
}

}  // namespace psr

int ps_launch_rope_cache(const ps_rope_launch &a, void *stream) {
    hipStream_t st = static_cast<hipStream_t>(stream);
    switch (a.dtype) {
        case PS_F32: return (int)psr::launch_d<psr::RF32>(a, st);
        case PS_F16: return (int)psr::launch_d<psr::RF16>(a, st);
        default: return (int)psr::launch_d<psr::RBF16>(a, st);
    }
}
