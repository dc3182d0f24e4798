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
// Work split: a workgroup of 256 threads owns 512 / D tokens, so that its
// tokens' D/2 angles each come to one thread. Each thread computes one
// (cos, sin) pair into LDS; then every head of those tokens is handled 16
// bytes per half-row per thread: a thread loads the chunk at d and the
// chunk at d + D/2, rotates, and stores both (eight threads cover the two
// 128-byte halves of a bf16 head of 128). V rows move as 16-byte words.

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

template <class DT, int D>
__global__ __launch_bounds__(256) void ps_rope_cache_kernel(const ps_rope_launch a) {
    constexpr int HALF = D / 2;
    constexpr int CH = 16 / DT::ELT;   // elements per 16-byte chunk
    constexpr int HC = HALF / CH;      // chunks per half row
    constexpr int TPB = 512 / D;       // tokens per workgroup: TPB * HALF = 256 angles
    __shared__ float2 cs[TPB][HALF];

    const int t0 = blockIdx.x * TPB;
    const int n_tok = min(TPB, a.num_tokens - t0);
    {
        const int tok = threadIdx.x / HALF, j = threadIdx.x % HALF;
        float c = 1.f, s = 0.f;
        if (tok < n_tok) {
            const double ang = (double)a.positions[t0 + tok] * a.inv_freq[j];
            double sd, cd;
            sincos(ang, &sd, &cd);
            c = (float)cd;
            s = (float)sd;
        }
        cs[tok][j] = make_float2(c, s);
    }
    __syncthreads();

    const int Hq = a.num_q_heads, Hkv = a.num_kv_heads;
    const int rot_units = (Hq + Hkv) * HC;    // (head, chunk) pairs to rotate per token
    const int v_words = Hkv * D / CH;         // 16-byte words of one token's V row
    const int per_tok = rot_units + v_words;
    const u32x4 *q = static_cast<const u32x4 *>(a.q);
    u32x4 *q_out = static_cast<u32x4 *>(a.q_out);
    const u32x4 *k = static_cast<const u32x4 *>(a.k);
    const u32x4 *v = static_cast<const u32x4 *>(a.v);
    u32x4 *pk = static_cast<u32x4 *>(a.pool_k);
    u32x4 *pv = static_cast<u32x4 *>(a.pool_v);
    constexpr int ROW_W = D / CH;             // 16-byte words per head row

    for (int u = threadIdx.x; u < n_tok * per_tok; u += 256) {
        const int tok = u / per_tok;
        const int r = u - tok * per_tok;
        const int64_t t = t0 + tok;
        if (r < rot_units) {
            const int head = r / HC, c = r - head * HC;
            const u32x4 *src;
            u32x4 *dst;
            if (head < Hq) {
                src = q + (t * Hq + head) * ROW_W;
                dst = q_out + (t * Hq + head) * ROW_W;
            } else {
                const int32_t slot = a.slots[t];
                if ((uint32_t)slot >= (uint32_t)a.num_slots) continue;
                src = k + (t * Hkv + (head - Hq)) * ROW_W;
                dst = pk + ((int64_t)slot * Hkv + (head - Hq)) * ROW_W;
            }
            const u32x4 lo = src[c], hi = src[HC + c];
            float x1[CH], x2[CH], y1[CH], y2[CH];
            unpack(lo, x1, DT{});
            unpack(hi, x2, DT{});
#pragma unroll
            for (int e = 0; e < CH; ++e) {
                const float2 f = cs[tok][c * CH + e];
                y1[e] = x1[e] * f.x - x2[e] * f.y;
                y2[e] = x2[e] * f.x + x1[e] * f.y;
            }
            dst[c] = pack(y1, DT{});
            dst[HC + c] = pack(y2, DT{});
        } else {
            const int32_t slot = a.slots[t];
            if ((uint32_t)slot >= (uint32_t)a.num_slots) continue;
            const int w = r - rot_units;
            pv[(int64_t)slot * v_words + w] = v[t * v_words + w];
        }
    }
}

template <class DT, int D>
hipError_t launch_t(const ps_rope_launch &a, hipStream_t st) {
    constexpr int TPB = 512 / D;
    const unsigned grid = (unsigned)((a.num_tokens + TPB - 1) / TPB);
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
