// Router: logits l = x W_r^T + b, then a wavefront per token selects the
// k largest logits (ties -> lowest expert index) and forms the softmax gates.
//
// The pages say only that each token is routed to k experts per layer and that the
// routing changes from token to token (dothoosh.com FreeToken article, "FreeToken
// architecture and the sparsity puzzle" and mechanism 2); the softmax-over-selected
// gating and the tie rule are this library's stated reading.
#include "common.h"
#include "kernels.h"

namespace moe {

// ------------------------------------------------------------------------------------------------
// Logits, decode shape: one wavefront per expert row of W_r, all tokens of the batch.
// The row (d elements) is streamed once with 16-byte loads; tokens are taken TG at a time.
// ------------------------------------------------------------------------------------------------
template <typename A> struct vec16;
template <> struct vec16<float> {
    static constexpr int N = 4;
    __device__ __forceinline__ static void load(const float* p, float* v) {
        float4 q = *reinterpret_cast<const float4*>(p);
        v[0] = q.x; v[1] = q.y; v[2] = q.z; v[3] = q.w;
    }
};
template <> struct vec16<uint16_t> {
    static constexpr int N = 8;
    __device__ __forceinline__ static void load(const uint16_t* p, float* v) {
        uint4 q = *reinterpret_cast<const uint4*>(p);
        v[0] = bf16_lo(q.x); v[1] = bf16_hi(q.x); v[2] = bf16_lo(q.y); v[3] = bf16_hi(q.y);
        v[4] = bf16_lo(q.z); v[5] = bf16_hi(q.z); v[6] = bf16_lo(q.w); v[7] = bf16_hi(q.w);
    }
};

template <typename A, int TG>
__global__ void __launch_bounds__(256) route_logits_gemv(const A* __restrict__ x, const A* __restrict__ wr,
                                                         const float* __restrict__ b, float* __restrict__ logits,
                                                         int T, int d, int E) {
    constexpr int V = vec16<A>::N;
    const int e = blockIdx.x * 4 + wave_id();
    if (e >= E) return;
    const int lane = lane_id();
    const A* w = wr + (int64_t)e * d;
    const float bias = b ? b[e] : 0.0f;
    for (int t0 = 0; t0 < T; t0 += TG) {
        float acc[TG];
#pragma unroll
        for (int q = 0; q < TG; ++q) acc[q] = 0.0f;
        for (int i = lane * V; i < d; i += MOE_WAVE * V) {
            float wv[V];
            vec16<A>::load(w + i, wv);
#pragma unroll
            for (int q = 0; q < TG; ++q) {
                if (t0 + q < T) {
                    float xv[V];
                    vec16<A>::load(x + (int64_t)(t0 + q) * d + i, xv);
#pragma unroll
                    for (int v = 0; v < V; ++v) acc[q] = fmaf(wv[v], xv[v], acc[q]);
                }
            }
        }
#pragma unroll
        for (int q = 0; q < TG; ++q) {
            float s = wave_sum(acc[q]);
            if (lane == 0 && t0 + q < T) logits[(int64_t)(t0 + q) * E + e] = s + bias;
        }
    }
}

// ------------------------------------------------------------------------------------------------
// Top-k + gates: one wavefront per token.  Lane l holds the EPL logits of experts l*EPL ..
// l*EPL+EPL-1 as order-preserving 32-bit keys (NaN lowest, -0 equal to +0); k rounds of a
// wave-wide max, ties to the lowest expert, pick the experts in selection order.
// With `part` (the router GEMM's ks K-split partial sums, ks x [T, E]) the logits are formed
// here first -- the partials added in split order, then the bias -- and stored to `logits`.
// ------------------------------------------------------------------------------------------------
template <int EPL>
__global__ void __launch_bounds__(256) route_topk(const float* __restrict__ logits_in, const float* __restrict__ part,
                                                  int ks, const float* __restrict__ bias,
                                                  float* __restrict__ logits_out, int T, int E, int k,
                                                  uint32_t no_renorm, int32_t* __restrict__ idx_out,
                                                  float* __restrict__ w_out, int32_t* __restrict__ idx_out2) {
    __shared__ float s_row[4][EPL * MOE_WAVE];
    const int wv = wave_id();
    const int t = blockIdx.x * 4 + wv;
    if (t >= T) return;
    const int lane = lane_id();
    float* l = s_row[wv];
    uint32_t key[EPL];
    if (part) {
        // every split's values loaded at once (ks <= ROUTER_MAX_SPLIT), then added in split order
        const int64_t n = (int64_t)T * E;
        float pv[ROUTER_MAX_SPLIT][EPL];
#pragma unroll
        for (int q = 0; q < ROUTER_MAX_SPLIT; ++q)
#pragma unroll
            for (int j = 0; j < EPL; ++j) {
                const int e = lane * EPL + j;
                pv[q][j] = (q < ks && e < E) ? part[(int64_t)q * n + (int64_t)t * E + e] : 0.0f;
            }
        float v[EPL];
#pragma unroll
        for (int j = 0; j < EPL; ++j) {
            v[j] = 0.0f;
#pragma unroll
            for (int q = 0; q < ROUTER_MAX_SPLIT; ++q)
                if (q < ks) v[j] += pv[q][j];
        }
#pragma unroll
        for (int j = 0; j < EPL; ++j) {
            const int e = lane * EPL + j;
            if (e < E) {
                const float lv = v[j] + (bias ? bias[e] : 0.0f);
                logits_out[(int64_t)t * E + e] = lv;
                l[e] = lv;
            }
        }
    } else {
#pragma unroll
        for (int j = 0; j < EPL; ++j) {
            const int e = lane * EPL + j;
            if (e < E) l[e] = logits_in[(int64_t)t * E + e];
        }
    }
#pragma unroll
    for (int j = 0; j < EPL; ++j) {
        const int e = lane * EPL + j;
        key[j] = (e < E) ? sel_ord(l[e]) : 0u;
    }
    const int my_sel = wave_topk<EPL>(key, k);
    // Gates: exp(l - m) with m the first (largest) selected logit.
    const float m = l[__builtin_amdgcn_readlane(my_sel, 0)];
    const float term = (lane < k) ? expf(l[my_sel] - m) : 0.0f;
    float den;
    if (no_renorm) {
        float sum = 0.0f;
#pragma unroll
        for (int j = 0; j < EPL; ++j) {
            const int e = lane * EPL + j;
            if (e < E) sum += expf(l[e] - m);
        }
        den = wave_sum(sum);
    } else {
        den = wave_sum(term);
    }
    if (lane < k) {
        idx_out[(int64_t)t * k + lane] = my_sel;
        w_out[(int64_t)t * k + lane] = term / den;
        if (idx_out2) idx_out2[(int64_t)t * k + lane] = my_sel;
    }
}

// ------------------------------------------------------------------------------------------------
// Host launchers
// ------------------------------------------------------------------------------------------------
hipError_t launch_route_logits(int act_dtype, const void* x, const void* wr, const float* b, float* logits,
                               int T, int d, int E, hipStream_t st) {
    dim3 grid((E + 3) / 4), block(256);
    if (act_dtype == 0)
        hipLaunchKernelGGL((route_logits_gemv<float, 8>), grid, block, 0, st, (const float*)x, (const float*)wr, b,
                           logits, T, d, E);
    else
        hipLaunchKernelGGL((route_logits_gemv<uint16_t, 8>), grid, block, 0, st, (const uint16_t*)x,
                           (const uint16_t*)wr, b, logits, T, d, E);
    return hipGetLastError();
}

hipError_t launch_route_topk(const float* logits, int T, int E, int k, bool no_renorm, int32_t* idx, float* w,
                             int32_t* idx2, hipStream_t st, const RouterPartials* rp) {
    dim3 grid((T + 3) / 4), block(256);
    const uint32_t nr = no_renorm ? 1u : 0u;
    const float* part = rp ? rp->part : nullptr;
    const int ks = rp ? rp->ks : 1;
    const float* bias = rp ? rp->bias : nullptr;
    float* lout = rp ? rp->logits : nullptr;
#define MOE_TOPK(EPLV) \
    hipLaunchKernelGGL((route_topk<EPLV>), grid, block, 0, st, logits, part, ks, bias, lout, T, E, k, nr, idx, w, idx2)
    if (E <= 64) MOE_TOPK(1);
    else if (E <= 128) MOE_TOPK(2);
    else if (E <= 256) MOE_TOPK(4);
    else if (E <= 512) MOE_TOPK(8);
    else MOE_TOPK(16);
#undef MOE_TOPK
    return hipGetLastError();
}

}  // namespace moe
