// Rejection-sampling verification of speculative drafts, for gfx950.
//
// A verify round of sequence s scores [last, d_0 .. d_{k-1}] in one packed
// pass; the target's distributions p_0..p_k and the proposer's q_0..q_{k-1}
// then decide how many drafts survive and which token follows (tinyserve
// README "How it works", Speculative decoding; PageServe "06 Development
// history", Next steps). Draft d_i is kept while u_i * q_i(d_i) < p_i(d_i)
// (fp64: the product of an fp64 uniform and an fp32 probability); at the
// first rejection the next token is drawn from max(p_i - q_i, 0), else from
// p_k after the last draft.
//
// Draws are inverse-CDF lookups on fixed-point weights
// floor(clamp(w, 0, 1) * 2^40): integer running sums are exact, so the
// result does not depend on how the vocabulary is split across threads.
//
// Two launches:
//  * ps_spec_sums_kernel  — grid (sequence, 4096-entry vocab chunk): every
//    workgroup derives the sequence's first rejection from k gathered
//    probabilities (chunk 0 records it), then sums its chunk of the row the
//    draw comes from: the residual (reading p_j and q_j) or p_k. One pass
//    over at most two vocab rows per sequence: this is the HBM-bound part.
//  * ps_spec_select_kernel — one workgroup per sequence: reads the
//    decision and the chunk sums in one round trip, finds the chunk that
//    holds the draw and rescans only that chunk. A residual without mass
//    (the draw then comes from p_j) takes a slow whole-row path here.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ps_internal.h"

namespace pss {

constexpr int kThreads = 256;
constexpr int kPerThread = PS_SPEC_CHUNK / kThreads;   // 16 entries

__device__ inline uint64_t fixed_weight(double w) {
    if (!(w > 0.0)) return 0;
    if (w > 1.0) w = 1.0;
    return (uint64_t)(w * 1099511627776.0);   // 2^40
}

__device__ inline uint64_t uniform53(double v) {
    const uint64_t top = (1ull << 53) - 1;
    if (!(v > 0.0)) return 0;
    if (v >= 1.0) return top;
    const uint64_t x = (uint64_t)(v * 9007199254740992.0);   // 2^53
    return x > top ? top : x;
}

// floor(u53 * total / 2^53) for u53 < 2^53, total < 2^63
__device__ inline uint64_t scale53(uint64_t u53, uint64_t total) {
    const uint64_t hi = __umul64hi(u53, total);
    const uint64_t lo = u53 * total;
    return (hi << 11) | (lo >> 53);
}

// Weight of vocab entry t of the row being drawn from: the residual
// max(p - q, 0) when q is given, else p.
__device__ inline uint64_t weight(float p, const float *qrow, int64_t t) {
    if (qrow) {
        const double r = (double)p - (double)qrow[t];
        return fixed_weight(r > 0.0 ? r : 0.0);
    }
    return fixed_weight((double)p);
}

struct Decision {
    int64_t d0;   // first draft row of the sequence
    int32_t k;    // drafts
    int32_t j;    // drafts kept (index of the first rejection, or k)
    bool bad;
};

// The first rejection of sequence s, computed by every wave for itself:
// lane i looks at draft base + i. Every draft token is range-checked, also
// after the first rejection, so that a malformed sequence is flagged as a
// whole.
__device__ inline Decision decide(const ps_spec_launch &a, int s) {
    Decision r;
    const int lane = threadIdx.x & 63;
    const int32_t b0 = a.starts[s], b1 = a.starts[s + 1];
    r.d0 = b0;
    r.k = b1 - b0;
    r.j = r.k;
    r.bad = b0 < 0 || b1 < b0 || b1 > a.total_drafts;
    if (r.bad) return r;
    const int64_t V = a.vocab;
    for (int base = 0; base < r.k; base += 64) {
        const int i = base + lane;
        bool rej = false, badtok = false;
        if (i < r.k) {
            const int32_t d = a.tokens[r.d0 + i];
            badtok = d < 0 || d >= a.vocab;
            if (!badtok) {
                const double p = a.target[(r.d0 + s + i) * V + d];
                const double q = a.draft[(r.d0 + i) * V + d];
                rej = !(a.accept_u[r.d0 + i] * q < p);
            }
        }
        if (__any(badtok)) {
            r.bad = true;
            return r;
        }
        const uint64_t m = __ballot(rej);
        if (m && r.j == r.k) r.j = base + __builtin_ctzll(m);
    }
    return r;
}

__device__ inline uint64_t shfl_up_u64(uint64_t x, int off) {
    const uint32_t lo = __shfl_up((uint32_t)x, off, 64);
    const uint32_t hi = __shfl_up((uint32_t)(x >> 32), off, 64);
    return ((uint64_t)hi << 32) | lo;
}
__device__ inline uint64_t shfl_xor_u64(uint64_t x, int m) {
    const uint32_t lo = __shfl_xor((uint32_t)x, m, 64);
    const uint32_t hi = __shfl_xor((uint32_t)(x >> 32), m, 64);
    return ((uint64_t)hi << 32) | lo;
}

// Exclusive scan of one uint64 per thread over the workgroup; also returns
// the workgroup total. wave_tot is 4 entries of LDS.
__device__ inline uint64_t block_exclusive_scan(uint64_t x, uint64_t *wave_tot, uint64_t &total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    uint64_t inc = x;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const uint64_t y = shfl_up_u64(inc, off);
        if (lane >= off) inc += y;
    }
    if (lane == 63) wave_tot[wave] = inc;
    __syncthreads();
    uint64_t before = 0;
    total = 0;
#pragma unroll
    for (int w = 0; w < kThreads / 64; ++w) {
        const uint64_t t = wave_tot[w];
        before += w < wave ? t : 0;
        total += t;
    }
    __syncthreads();
    return before + inc - x;
}

template <bool VEC>
__device__ inline void load4(const float *row, int64_t idx, int64_t V, float *out) {
    if (VEC && idx + 3 < V) {
        const float4 f = *reinterpret_cast<const float4 *>(row + idx);
        out[0] = f.x;
        out[1] = f.y;
        out[2] = f.z;
        out[3] = f.w;
    } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) out[e] = idx + e < V ? row[idx + e] : 0.f;
    }
}

template <bool VEC>
__global__ __launch_bounds__(kThreads) void ps_spec_sums_kernel(const ps_spec_launch a) {
    const int s = blockIdx.x;
    const int chunk = blockIdx.y;
    __shared__ uint64_t red[kThreads / 64];
    const Decision dc = decide(a, s);
    if (chunk == 0 && threadIdx.x == 0) {
        a.decisions[2 * s] = dc.j;
        a.decisions[2 * s + 1] = dc.bad ? 1 : 0;
    }
    uint64_t *out = a.chunk_sums + (int64_t)s * a.n_chunks + chunk;
    if (dc.bad) {
        if (threadIdx.x == 0) *out = 0;
        return;
    }
    // the row the draw comes from: the residual after a rejection, else p_k
    const int64_t V = a.vocab;
    const float *prow = a.target + (dc.d0 + s + dc.j) * V;
    const float *qrow = dc.j < dc.k ? a.draft + (dc.d0 + dc.j) * V : nullptr;
    uint64_t sum = 0;
#pragma unroll
    for (int m = 0; m < kPerThread / 4; ++m) {
        // coalesced: consecutive threads take consecutive 16-byte groups
        const int64_t idx = (int64_t)chunk * PS_SPEC_CHUNK + m * (kThreads * 4) + threadIdx.x * 4;
        float p[4], q[4];
        load4<VEC>(prow, idx, V, p);
        if (qrow) load4<VEC>(qrow, idx, V, q);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            uint64_t w;
            if (qrow) {
                const double r = (double)p[e] - (double)q[e];
                w = fixed_weight(r > 0.0 ? r : 0.0);
            } else {
                w = fixed_weight((double)p[e]);
            }
            sum += idx + e < V ? w : 0;
        }
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) sum += shfl_xor_u64(sum, m);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0) red[wave] = sum;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint64_t t = 0;
#pragma unroll
        for (int w = 0; w < kThreads / 64; ++w) t += red[w];
        *out = t;
    }
}

struct SelectLds {
    uint64_t wave_tot[kThreads / 64];
    uint64_t found[2];   // chunk, running sum before it
    int32_t token;
};

// Chunk `chunk` of the row (weights of p, or of max(p - q, 0) with q):
// thread t owns entries [16t, 16t + 16); the token whose running sum
// first exceeds `local` goes to L.token. Returns the chunk's total.
__device__ inline uint64_t find_in_chunk(const float *prow, const float *qrow, int64_t V, int64_t chunk,
                                         uint64_t local, SelectLds &L) {
    const int64_t t0 = chunk * PS_SPEC_CHUNK + (int64_t)threadIdx.x * kPerThread;
    uint64_t w[kPerThread];
    uint64_t sum = 0;
#pragma unroll
    for (int e = 0; e < kPerThread; ++e) {
        const int64_t t = t0 + e;
        w[e] = t < V ? weight(prow[t], qrow, t) : 0;
        sum += w[e];
    }
    uint64_t ctot;
    const uint64_t cbefore = block_exclusive_scan(sum, L.wave_tot, ctot);
    if (cbefore <= local && local < cbefore + sum) {
        uint64_t run = cbefore;
        int32_t tok = -1;
#pragma unroll
        for (int e = 0; e < kPerThread; ++e) {
            run += w[e];
            if (tok < 0 && run > local) tok = (int32_t)(t0 + e);
        }
        L.token = tok;
    }
    __syncthreads();
    return ctot;
}

// Rare path: a rejection whose residual has no mass at the draw's
// resolution draws from p_j instead. One workgroup sums the whole row,
// then walks it chunk by chunk.
__device__ inline int32_t draw_whole_row(const float *prow, int64_t V, int nc, double v, SelectLds &L) {
    uint64_t mine = 0;
    for (int c = 0; c < nc; ++c) {
        const int64_t t0 = (int64_t)c * PS_SPEC_CHUNK + (int64_t)threadIdx.x * kPerThread;
#pragma unroll
        for (int e = 0; e < kPerThread; ++e)
            mine += t0 + e < V ? fixed_weight((double)prow[t0 + e]) : 0;
    }
    uint64_t total;
    block_exclusive_scan(mine, L.wave_tot, total);
    if (total == 0) return -1;
    const uint64_t target = scale53(uniform53(v), total);
    uint64_t run = 0;
    for (int c = 0; c < nc; ++c) {
        if (threadIdx.x == 0) L.token = -1;
        __syncthreads();
        const uint64_t ctot = find_in_chunk(prow, nullptr, V, c, target - run, L);
        if (target < run + ctot) return L.token;
        run += ctot;
    }
    return -1;
}

__global__ __launch_bounds__(kThreads) void ps_spec_select_kernel(const ps_spec_launch a) {
    const int s = blockIdx.x;
    __shared__ SelectLds L;
    if (threadIdx.x == 0) {
        L.found[0] = L.found[1] = 0;   // published by the scans' barriers
        L.token = -1;
    }
    // independent loads: the first pass's decision, the chunk sums, the rows
    const int32_t j = a.decisions[2 * s];
    const bool bad = a.decisions[2 * s + 1] != 0;
    const int32_t b0 = a.starts[s], b1 = a.starts[s + 1];
    const uint64_t *sums = a.chunk_sums + (int64_t)s * a.n_chunks;
    const int nc = a.n_chunks;
    const int per = (nc + kThreads - 1) / kThreads;
    const int c0 = min(nc, (int)threadIdx.x * per), c1 = min(nc, c0 + per);
    uint64_t mine = 0;
    for (int c = c0; c < c1; ++c) mine += sums[c];
    if (bad) {
        if (threadIdx.x == 0) a.num_accepted[s] = a.next_token[s] = -1;
        return;
    }
    const int32_t k = b1 - b0;
    const int64_t V = a.vocab;
    const float *prow = a.target + ((int64_t)b0 + s + j) * V;
    const float *qrow = j < k ? a.draft + ((int64_t)b0 + j) * V : nullptr;
    uint64_t total;
    const uint64_t before = block_exclusive_scan(mine, L.wave_tot, total);
    int32_t tok;
    if (total == 0) {
        tok = qrow ? draw_whole_row(prow, V, nc, a.sample_u[s], L) : -1;
    } else {
        const uint64_t target = scale53(uniform53(a.sample_u[s]), total);
        // the chunk holding the draw
        if (before <= target && target < before + mine) {
            uint64_t run = before;
            for (int c = c0; c < c1; ++c) {
                if (target < run + sums[c]) {
                    L.found[0] = (uint64_t)c;
                    L.found[1] = run;
                    break;
                }
                run += sums[c];
            }
        }
        __syncthreads();
        const int64_t chunk = min((int64_t)L.found[0], (int64_t)nc - 1);
        find_in_chunk(prow, qrow, V, chunk, target - L.found[1], L);
        tok = L.token;
    }
    if (threadIdx.x == 0) {
        a.num_accepted[s] = j;
        a.next_token[s] = tok;
    }
}

}  // namespace pss

int ps_launch_spec_verify(const ps_spec_launch &a, bool vec, void *stream) {
    hipStream_t st = static_cast<hipStream_t>(stream);
    const dim3 grid1((unsigned)a.num_seqs, (unsigned)a.n_chunks);
    if (vec)
        hipLaunchKernelGGL(pss::ps_spec_sums_kernel<true>, grid1, dim3(pss::kThreads), 0, st, a);
    else
        hipLaunchKernelGGL(pss::ps_spec_sums_kernel<false>, grid1, dim3(pss::kThreads), 0, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return (int)e;
    hipLaunchKernelGGL(pss::ps_spec_select_kernel, dim3((unsigned)a.num_seqs), dim3(pss::kThreads), 0, st, a);
    return (int)hipGetLastError();
}
