// Decode path of the whole layer (T <= 32 tokens, T*E <= 8192) in three launches.
//
// At decode a token touches only its k experts (FreeToken/dothoosh, "Architecture and the
// sparsity puzzle": 13B of 284B parameters per token), so the layer is a stream of a few
// experts' weight rows from HBM and everything else is latency.  The launches are arranged so
// that no workgroup ever waits for another one inside a kernel:
//
//   dec_logits  one wavefront per (router row, token) computes a logit (with the residual
//               stack, every wavefront also RMS-normalises its token itself and the first
//               workgroup of each token stores the normalised input for the FFN kernels).
//   dec_w13     every workgroup first redoes the routing from the logits in LDS -- top-k and
//               gates per token, grouping by expert into a slot table (expert, first sorted
//               position, pairs, token mask) -- then computes its share of
//               a[pos, j] = silu(Wg_e[j] . x_t) * (Wu_e[j] . x_t) in fp32.  The shared
//               expert's items come first and their rows are pulled into L2 during the
//               routing, which does not decide them.  Workgroup 0 also
//               publishes the routing (top-k, slot table, per-position gate) for the down
//               kernel and the caller.
//   dec_w2c     down projection fused with the combine: a workgroup owns R output rows of
//               every token; its 8 wavefronts split the slots, each adds g * (W2_e[i] . a) for
//               its slots, and the 8 partial sums are added in wavefront order through LDS --
//               a fixed order, so results are deterministic and need no atomics.
//   dec_w2c1    the same for a single token: the workgroup's (slot, row) units are cut into 8
//               contiguous ranges, one per wavefront, so no wavefront makes two round trips.
#include <map>
#include <mutex>
#include <tuple>

#include "common.h"
#include "kernels.h"
#include "wchunk.h"

namespace moe {

constexpr int DEC_MAX_T = 32;
constexpr int DEC_MAX_TE = 8192;  // logits held in LDS by every gate/up workgroup

template <typename A> struct rvec;
template <> struct rvec<float> {
    static constexpr int N = 4;
    __device__ __forceinline__ static void load(const float* p, float* v) {
        float4 q = *reinterpret_cast<const float4*>(p);
        v[0] = q.x; v[1] = q.y; v[2] = q.z; v[3] = q.w;
    }
};
template <> struct rvec<uint16_t> {
    static constexpr int N = 8;
    __device__ __forceinline__ static void load(const uint16_t* p, float* v) {
        uint4 q = *reinterpret_cast<const uint4*>(p);
        v[0] = bf16_lo(q.x); v[1] = bf16_hi(q.x); v[2] = bf16_lo(q.y); v[3] = bf16_hi(q.y);
        v[4] = bf16_lo(q.z); v[5] = bf16_hi(q.z); v[6] = bf16_lo(q.w); v[7] = bf16_hi(q.w);
    }
};

// ------------------------------------------------------------------------------------------------
// dec_logits
// ------------------------------------------------------------------------------------------------
struct DecLogitsArgs {
    const void* x;   // [T, d] act dtype, or (prenorm) the fp32 residual stream h [T, d]
    const void* wr;  // [E, d] act dtype
    const float* b;  // [E] or NULL
    float* logits;   // [T, E]
    void* xn;        // prenorm: normalised input (act dtype), written by workgroup 0
    int T, d, E, prenorm;
};

// One wavefront per (router row, token): grid = (E, T) of one-wavefront workgroups.  Every load of a pass (up to 8
// 16-byte chunks of the row and of the token per lane) is issued before any arithmetic, so a
// wavefront waits for one round trip per pass.  With the residual stack (prenorm) each
// wavefront first takes its token's RMS from h (fp32) and reads x = bf16(h * inv_rms), the value
// the FFN kernels read; the workgroups of column 0 store that normalised input.
template <typename A>
__device__ __forceinline__ float dot_chunk(uint4 w, uint4 x);
template <>
__device__ __forceinline__ float dot_chunk<uint16_t>(uint4 w, uint4 x) {
    float a = 0.0f;
    a = fmaf(bf16_lo(w.x), bf16_lo(x.x), a); a = fmaf(bf16_hi(w.x), bf16_hi(x.x), a);
    a = fmaf(bf16_lo(w.y), bf16_lo(x.y), a); a = fmaf(bf16_hi(w.y), bf16_hi(x.y), a);
    a = fmaf(bf16_lo(w.z), bf16_lo(x.z), a); a = fmaf(bf16_hi(w.z), bf16_hi(x.z), a);
    a = fmaf(bf16_lo(w.w), bf16_lo(x.w), a); a = fmaf(bf16_hi(w.w), bf16_hi(x.w), a);
    return a;
}
template <>
__device__ __forceinline__ float dot_chunk<float>(uint4 w, uint4 x) {
    float a = 0.0f;
    a = fmaf(__uint_as_float(w.x), __uint_as_float(x.x), a);
    a = fmaf(__uint_as_float(w.y), __uint_as_float(x.y), a);
    a = fmaf(__uint_as_float(w.z), __uint_as_float(x.z), a);
    a = fmaf(__uint_as_float(w.w), __uint_as_float(x.w), a);
    return a;
}
// x chunk (V elements) from the fp32 residual stream: bf16(h * inv) (or fp32 h * inv), packed
// like a chunk of the act dtype.
template <typename A>
__device__ __forceinline__ uint4 norm_chunk(const float* h, int c, float inv);
template <>
__device__ __forceinline__ uint4 norm_chunk<uint16_t>(const float* h, int c, float inv) {
    const float4 a = reinterpret_cast<const float4*>(h)[2 * c], b = reinterpret_cast<const float4*>(h)[2 * c + 1];
    return make_uint4(pack_bf16x2(a.x * inv, a.y * inv), pack_bf16x2(a.z * inv, a.w * inv),
                      pack_bf16x2(b.x * inv, b.y * inv), pack_bf16x2(b.z * inv, b.w * inv));
}
template <>
__device__ __forceinline__ uint4 norm_chunk<float>(const float* h, int c, float inv) {
    const float4 a = reinterpret_cast<const float4*>(h)[c];
    return make_uint4(__float_as_uint(a.x * inv), __float_as_uint(a.y * inv), __float_as_uint(a.z * inv),
                      __float_as_uint(a.w * inv));
}

template <typename A>
__global__ void __launch_bounds__(256) dec_logits(DecLogitsArgs p) {
    constexpr int V = rvec<A>::N;  // elements per 16-byte chunk
    constexpr int NB = 8;          // chunks per lane per pass
    const int lane = lane_id(), wv = wave_id();
    const int t = blockIdx.y, d = p.d, NC = d / V;
    const float* h = reinterpret_cast<const float*>(p.x) + (int64_t)t * d;
    float inv = 1.0f;
    const int e = blockIdx.x * (blockDim.x / MOE_WAVE) + wv;
    if (p.prenorm && NC <= MOE_WAVE * NB) {
        // The wavefront's lanes hold the whole row of h between them: its chunks give the RMS
        // (one wave-wide sum) and then x, from a single round trip together with W_r's row.
        const uint4* w = reinterpret_cast<const uint4*>(reinterpret_cast<const A*>(p.wr) + (int64_t)min(e, p.E - 1) * d);
        constexpr int HF = V / 4;  // float4 of h per chunk
        float4 hv[NB][HF];
        uint4 wc[NB];
        float ss = 0.0f;
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            const int c = lane + MOE_WAVE * b;
#pragma unroll
            for (int q = 0; q < HF; ++q)
                hv[b][q] = c < NC ? reinterpret_cast<const float4*>(h)[HF * c + q] : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
            wc[b] = c < NC ? w[c] : make_uint4(0u, 0u, 0u, 0u);
        }
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int q = 0; q < HF; ++q) {
                ss = fmaf(hv[b][q].x, hv[b][q].x, ss); ss = fmaf(hv[b][q].y, hv[b][q].y, ss);
                ss = fmaf(hv[b][q].z, hv[b][q].z, ss); ss = fmaf(hv[b][q].w, hv[b][q].w, ss);
            }
        inv = 1.0f / sqrtf(wave_sum(ss) / (float)d + 1e-6f);
        float acc = 0.0f;
        uint4* xo = reinterpret_cast<uint4*>(reinterpret_cast<A*>(p.xn) + (int64_t)t * d);
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            const int c = lane + MOE_WAVE * b;
            if (c < NC) {
                uint4 xc;
                if constexpr (V == 8)
                    xc = make_uint4(pack_bf16x2(hv[b][0].x * inv, hv[b][0].y * inv), pack_bf16x2(hv[b][0].z * inv, hv[b][0].w * inv),
                                    pack_bf16x2(hv[b][HF - 1].x * inv, hv[b][HF - 1].y * inv),
                                    pack_bf16x2(hv[b][HF - 1].z * inv, hv[b][HF - 1].w * inv));
                else
                    xc = make_uint4(__float_as_uint(hv[b][0].x * inv), __float_as_uint(hv[b][0].y * inv),
                                    __float_as_uint(hv[b][0].z * inv), __float_as_uint(hv[b][0].w * inv));
                acc += dot_chunk<A>(wc[b], xc);
                if (blockIdx.x == 0 && wv == 0) xo[c] = xc;
            }
        }
        acc = wave_sum(acc);
        if (lane == 0 && e < p.E) p.logits[(int64_t)t * p.E + e] = acc + (p.b ? p.b[e] : 0.0f);
        return;
    }
    if (p.prenorm) {
        float ss = 0.0f;
        for (int c0 = 0; c0 < d / 4; c0 += MOE_WAVE * NB) {
            float4 v[NB];
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                const int c = c0 + lane + MOE_WAVE * b;
                v[b] = c < d / 4 ? reinterpret_cast<const float4*>(h)[c] : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
            }
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                ss = fmaf(v[b].x, v[b].x, ss); ss = fmaf(v[b].y, v[b].y, ss);
                ss = fmaf(v[b].z, v[b].z, ss); ss = fmaf(v[b].w, v[b].w, ss);
            }
        }
        ss = wave_sum(ss);
        inv = 1.0f / sqrtf(ss / (float)d + 1e-6f);
        if (blockIdx.x == 0)
            for (int c = threadIdx.x; c < NC; c += blockDim.x)
                reinterpret_cast<uint4*>(reinterpret_cast<A*>(p.xn) + (int64_t)t * d)[c] = norm_chunk<A>(h, c, inv);
    }
    if (e >= p.E) return;
    const uint4* w = reinterpret_cast<const uint4*>(reinterpret_cast<const A*>(p.wr) + (int64_t)e * d);
    const uint4* x = reinterpret_cast<const uint4*>(reinterpret_cast<const A*>(p.x) + (int64_t)t * d);
    float acc = 0.0f;
    for (int c0 = 0; c0 < NC; c0 += MOE_WAVE * NB) {
        uint4 wc[NB], xc[NB];
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            const int c = c0 + lane + MOE_WAVE * b;
            if (c < NC) {
                wc[b] = w[c];
                xc[b] = p.prenorm ? norm_chunk<A>(h, c, inv) : x[c];
            } else {
                wc[b] = xc[b] = make_uint4(0u, 0u, 0u, 0u);
            }
        }
#pragma unroll
        for (int b = 0; b < NB; ++b) acc += dot_chunk<A>(wc[b], xc[b]);
    }
    acc = wave_sum(acc);
    if (lane == 0) p.logits[(int64_t)t * p.E + e] = acc + (p.b ? p.b[e] : 0.0f);
}

// ------------------------------------------------------------------------------------------------
// Routing from the logits, inside one workgroup of 256 threads, in LDS.
// Slot s = (expert, first sorted position, pairs, token mask); slots ascend by expert, the
// shared expert (if any) is the last slot, expert id E, positions P..P+T-1.
// ------------------------------------------------------------------------------------------------
struct DecRoute {
    int n_slots;
    int n_routed;
    int4* slot;   // [E + 1]
    float* gate;  // [T * k], [t][j]
    int* sel;     // [T * k]
};

// The routing's LDS arrays, as pointers the caller derives from its own LDS (so the compiler
// addresses them as LDS).
struct DecRouteLds {
    int4* slot;     // [E + 1]
    float* logits;  // [T * E]
    float* gate;    // [T * k]
    int* sel;       // [T * k]
    int* cnt;       // [E]
    int* mask;      // [E]
    int* on;        // [E + 1]
};

// Dynamic LDS carve-up of the routing prologue: slots, logits, gates, experts, counts, masks.
__host__ __device__ inline size_t dec_route_lds_bytes(int T, int E, int k) {
    return (size_t)(E + 1) * 16 + (size_t)T * E * 4 + (size_t)T * k * 8 + (size_t)E * 8 + (size_t)(E + 1) * 4 + 16;
}

struct DecRouteIO {
    const float* logits;
    int32_t* topk_idx;   // workgroup 0 publishes the routing
    float* topk_w;
    int32_t* idx_out;
    int32_t* meta;       // [0] = slots
    int4* slots;
    float* pos_gate;     // [P + T]
    int T, E, k, n_shared, no_renorm;
    const uint8_t* emask;  // nullable [E + 1]: experts (and the shared one, last) left out when 0
};

template <int KPL>
__device__ __forceinline__ int dec_select(const float* l, int E, int k) {
    uint32_t key[KPL];
    const int lane = lane_id();
#pragma unroll
    for (int j = 0; j < KPL; ++j) {
        const int e = lane * KPL + j;
        key[j] = e < E ? sel_ord(l[e]) : 0u;
    }
    return wave_topk<KPL>(key, k);
}

// Slot table from the per-expert pair counts, token masks and on flags (one wavefront): lane l
// owns experts l*PER .. l*PER+PER-1, read once into registers; exclusive scans of the counts
// (first sorted position) and of the active experts (slot index).  Returns, at every lane, the
// number of active experts before its own range plus its own: lane 63 holds the total.
template <int PER>
__device__ __forceinline__ int dec_slot_scan(DecRoute& R, const int* s_cnt, const int* s_mask, const int* s_on, int E) {
    const int lane = lane_id();
    const int lo = lane * PER;
    int c[PER], m[PER];
    bool on[PER];
    int sc = 0, sa = 0;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        const bool in = lo + j < E;
        c[j] = in ? s_cnt[lo + j] : 0;
        m[j] = in ? s_mask[lo + j] : 0;
        on[j] = in && s_on[lo + j];
    }
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        sc += c[j];
        sa += c[j] > 0 && on[j];
    }
    int pc = wave_incl_scan(sc) - sc, pa = wave_incl_scan(sa) - sa;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        if (c[j] > 0 && on[j]) R.slot[pa++] = make_int4(lo + j, pc, c[j], m[j]);
        pc += c[j];
    }
    return pa;
}

// One token with the top-k renormalised gates and up to 256 experts (the decode step):
// wavefront 0 routes alone, with
// the token's logits (and on flags) loaded straight into its registers -- no LDS copy, no
// per-expert counts, masks or scan, and a single barrier.  With one token every picked expert
// holds one pair, so the slot table follows from ranking the k picks among themselves: a pick's
// first sorted position is the number of picks with a lower expert id, its slot the number of
// active picks with a lower id.  Selections, gates and table equal the general path's.
// The table, picks and gates are written through the caller's LDS pointers (pointers read back
// from the shared routing struct are generic ones: flat stores).
template <bool COH, int KPL, typename Mid>
__device__ void dec_route_one(const DecRouteIO& io, DecRoute& R, const DecRouteLds& L, Mid&& mid) {
    const int lane = lane_id(), wv = wave_id();
    const int E = io.E, k = io.k;
    float* const s_logits = L.logits;
    int* const s_on = L.on;
    float lg[KPL];
    uint32_t on = 0u;  // bit j: entry j of the lane is left in
    int shared_on = 0;
    if (wv == 0) {
#pragma unroll
        for (int j = 0; j < KPL; ++j) {
            const int e = lane * KPL + j;
            lg[j] = 0.0f;
            if (e < E) {
                lg[j] = COH ? __hip_atomic_load(io.logits + e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : io.logits[e];
                if (!io.emask || io.emask[e]) on |= 1u << j;
            }
        }
        shared_on = io.n_shared && (!io.emask || io.emask[E]);
    }
    mid();
    if (wv == 0) {
        uint32_t key[KPL];
#pragma unroll
        for (int j = 0; j < KPL; ++j) {
            const int e = lane * KPL + j;
            key[j] = e < E ? sel_ord(lg[j]) : 0u;
            if (e < E) {
                s_logits[e] = lg[j];
                s_on[e] = (on >> j) & 1u;
            }
        }
        const int my_sel = wave_topk<KPL>(key, k);
        const bool pick = lane < k;
        const float m = s_logits[__builtin_amdgcn_readlane(my_sel, 0)];
        const float term = pick ? expf(s_logits[my_sel] - m) : 0.0f;
        const float den = wave_sum(term);
        const bool act = pick && s_on[my_sel];
        int pos = 0, slot = 0;
        for (int j = 0; j < k; ++j) {
            const int sj = __builtin_amdgcn_readlane(my_sel, j);
            const int aj = __builtin_amdgcn_readlane((int)act, j);
            pos += sj < my_sel;
            slot += (aj && sj < my_sel) ? 1 : 0;
        }
        if (pick) {
            L.sel[lane] = my_sel;
            L.gate[lane] = term / den;
        }
        if (act) L.slot[slot] = make_int4(my_sel, pos, 1, 1);
        const int n_act = __popcll(__ballot(act));
        if (lane == 0) {
            R.n_routed = n_act;
            R.n_slots = n_act + shared_on;
            if (shared_on) L.slot[n_act] = make_int4(E, k, 1, 1);
        }
    }
    __syncthreads();
}

// `mid` runs once the logits are in LDS, before the top-k (the rest of the routing issues no
// global loads, so loads that `mid` leaves in flight never delay it).  COH: the logits are read
// with device-scope loads (written earlier in the same launch by other workgroups).
template <bool COH = false, typename Mid>
__device__ void dec_route_lds(const DecRouteIO& io, DecRoute& R, const DecRouteLds& L, Mid&& mid) {
    const int lane = lane_id(), wv = wave_id(), tid = threadIdx.x;
    const int NW = blockDim.x / MOE_WAVE;
    const int T = io.T, E = io.E, k = io.k;
    float* const s_logits = L.logits;
    int* const s_cnt = L.cnt;
    int* const s_mask = L.mask;
    int* const s_on = L.on;
    if (T == 1 && !io.no_renorm && E <= 256) {
        if (E <= 64) dec_route_one<COH, 1>(io, R, L, mid);
        else if (E <= 128) dec_route_one<COH, 2>(io, R, L, mid);
        else dec_route_one<COH, 4>(io, R, L, mid);
        return;
    }
    for (int i = tid; i < T * E; i += blockDim.x)
        s_logits[i] = COH ? __hip_atomic_load(io.logits + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : io.logits[i];
    for (int e = tid; e < E; e += blockDim.x) {
        s_cnt[e] = 0;
        s_mask[e] = 0;
    }
    for (int e = tid; e <= E; e += blockDim.x) s_on[e] = io.emask ? io.emask[e] : 1;
    __syncthreads();
    mid();
    // top-k + gates, a wavefront per token
    for (int t = wv; t < T; t += NW) {
        const float* l = s_logits + t * E;
        int my_sel;
        if (E <= 64) my_sel = dec_select<1>(l, E, k);
        else if (E <= 128) my_sel = dec_select<2>(l, E, k);
        else if (E <= 256) my_sel = dec_select<4>(l, E, k);
        else if (E <= 512) my_sel = dec_select<8>(l, E, k);
        else my_sel = dec_select<16>(l, E, k);
        const float m = l[__builtin_amdgcn_readlane(my_sel, 0)];
        const float term = (lane < k) ? expf(l[my_sel] - m) : 0.0f;
        float den;
        if (io.no_renorm) {
            float part = 0.0f;
            for (int e = lane; e < E; e += MOE_WAVE) part += expf(l[e] - m);
            den = wave_sum(part);
        } else {
            den = wave_sum(term);
        }
        if (lane < k) {
            const float g = term / den;
            R.sel[t * k + lane] = my_sel;
            R.gate[t * k + lane] = g;
            atomicAdd(&s_cnt[my_sel], 1);
            atomicOr(&s_mask[my_sel], 1 << t);
        }
    }
    __syncthreads();
    // slot table: exclusive scan over experts (wavefront 0)
    const int P = T * k;
    if (wv == 0) {
        int pa;
        if (E <= 64) pa = dec_slot_scan<1>(R, s_cnt, s_mask, s_on, E);
        else if (E <= 128) pa = dec_slot_scan<2>(R, s_cnt, s_mask, s_on, E);
        else if (E <= 256) pa = dec_slot_scan<4>(R, s_cnt, s_mask, s_on, E);
        else {
            const int per = (E + MOE_WAVE - 1) / MOE_WAVE;
            const int lo = min(lane * per, E), hi = min(lo + per, E);
            int sc = 0, sa = 0;
            for (int e = lo; e < hi; ++e) {
                sc += s_cnt[e];
                sa += s_cnt[e] > 0 && s_on[e];
            }
            int pc = wave_incl_scan(sc) - sc;
            pa = wave_incl_scan(sa) - sa;
            for (int e = lo; e < hi; ++e) {
                const int c = s_cnt[e];
                if (c > 0 && s_on[e]) R.slot[pa++] = make_int4(e, pc, c, s_mask[e]);
                pc += c;
            }
        }
        if (lane == MOE_WAVE - 1) {
            R.n_routed = pa;
            const int shared_on = io.n_shared && s_on[E];
            R.n_slots = pa + shared_on;
            if (shared_on) R.slot[pa] = make_int4(E, P, T, (int)(T >= 32 ? 0xFFFFFFFFu : ((1u << T) - 1u)));
        }
    }
    __syncthreads();
}

// Workgroup 0 hands the routing to the caller and the down kernel: top-k indices and gates,
// the slot table and its size, and the gate of every sorted position (a slot's positions follow
// its tokens in ascending order).  Each wavefront does its share once its own items are done,
// so publishing never delays that workgroup's weight stream.
__device__ void dec_route_publish(const DecRouteIO& io, const DecRoute& R) {
    const int lane = lane_id(), wv = wave_id();
    const int NW = blockDim.x / MOE_WAVE;
    const int T = io.T, E = io.E, k = io.k;
    for (int i = wv * MOE_WAVE + lane; i < T * k; i += NW * MOE_WAVE) {
        io.topk_idx[i] = R.sel[i];
        io.topk_w[i] = R.gate[i];
        if (io.idx_out) io.idx_out[i] = R.sel[i];
    }
    for (int s = wv; s < R.n_slots; s += NW) {
        const int4 S = R.slot[s];
        if (lane == 0) io.slots[s] = S;
        const uint32_t m = (uint32_t)S.w;
        if (lane < T && ((m >> lane) & 1u)) {
            const uint32_t below = lane == 0 ? 0u : (m & (0xFFFFFFFFu >> (32 - lane)));
            const int pos = S.y + __popc(below);
            float g = 1.0f;
            if (S.x < E)
                for (int j = 0; j < k; ++j)
                    if (R.sel[lane * k + j] == S.x) g = R.gate[lane * k + j];
            io.pos_gate[pos] = g;
        }
    }
    if (wv == 0 && lane == 0) io.meta[0] = R.n_slots;
}

// ------------------------------------------------------------------------------------------------
// dec_w13
// ------------------------------------------------------------------------------------------------
struct DecFfnArgs {
    const void* x;          // [T, d] act dtype
    DecRouteIO rt;
    const uint8_t* w13; const uint8_t* w13s;   // routed gate/up
    const uint8_t* s13; const uint8_t* s13s;   // shared gate/up
    const uint8_t* w2; const uint8_t* w2s;     // routed down
    const uint8_t* s2; const uint8_t* s2s;     // shared down
    float* a;               // [P + T, fmax] fp32, each row chunk-transposed (a_off)
    void* out;              // [T, d] (f32 or bf16)
    int T, d, f, fs, fmax, k, accumulate;
    int slot_bound;         // routed slots number at most min(T*k, E), plus the shared one
    float g13, g2, gs13, gs2;   // NVFP4 tensor scales (1 otherwise): routed / shared gate-up, down
};

// Rows of `a` are stored chunk-transposed for the down kernels: with EC elements per weight
// chunk and ncp = fmax / EC chunks per row, float4 q of chunk c sits at float (q * ncp + c) * 4,
// so the 64 lanes of a wavefront, reading chunks c0 .. c0+63, read consecutive 16-byte pieces.
template <int EC>
__device__ __forceinline__ int64_t a_off(int j, int ncp) {
    return ((int64_t)((j % EC) >> 2) * ncp + j / EC) * 4 + (j & 3);
}
template <int EC>
__device__ __forceinline__ void a_chunk(const float* row, int ncp, int c, float (&out)[EC]) {
#pragma unroll
    for (int q = 0; q < EC / 4; ++q) {
        const float4 v = reinterpret_cast<const float4*>(row)[(int64_t)q * ncp + c];
        out[4 * q] = v.x;
        out[4 * q + 1] = v.y;
        out[4 * q + 2] = v.z;
        out[4 * q + 3] = v.w;
    }
}

template <int WT> struct DecAct { using T = uint16_t; };
template <> struct DecAct<0> { using T = float; };

// One token, every picked expert taken (no expert mask, renormalised gates, E <= 256) and one
// K step per row: every wavefront runs the top-k itself on the logits in its registers, and
// issues its first item's weight loads as soon as the round that picks that item's expert is
// done -- a shared-expert item's right away, since the routing does not decide it -- instead of
// after the whole workgroup's routing and its barrier.  Where an item's output row goes (its
// sorted position: the number of picks with a lower expert id) is known once all k rounds are
// done, while those loads are in flight.  Selections, gates, the published table and every
// row's arithmetic are those of the general path (dec_route_one and the item loop).
template <int WT, int R, int U, int KPL>
__device__ void dec_w13_one(const DecFfnArgs& p, DecRoute& rs, unsigned char* dyn_lds) {
    using W = WChunk<WT>;
    constexpr int EC = W::EC;
    const int lane = lane_id(), wv = wave_id();
    const int E = p.rt.E, k = p.rt.k;
    const int ngr = (p.f + R - 1) / R, ngs = (p.fs + R - 1) / R;
    const int NC = p.d / EC;
    const int64_t rb = row_bytes(WT, p.d), sb = scale_row_bytes(WT, p.d);
    const int NWB = blockDim.x / MOE_WAVE;
    const bool shared_on = p.rt.n_shared != 0;
    const int s_items = shared_on ? ngs : 0;
    const int n_items = s_items + k * ngr;
    const int stride = gridDim.x * NWB;
    const int item0 = blockIdx.x * NWB + wv;

    // the logits first: the waits for them leave the item loads issued below in flight
    float lg[KPL];
#pragma unroll
    for (int j = 0; j < KPL; ++j) {
        const int e = lane * KPL + j;
        lg[j] = e < E ? p.rt.logits[e] : 0.0f;
    }
    W wg[R][U], wu[R][U];
    auto issue = [&](int item, int ex) {
        const bool sh = item < s_items;
        const int fc = sh ? p.fs : p.f;
        const int j0 = (sh ? item : (item - s_items) % ngr) * R;
        const uint8_t* wb = sh ? p.s13 : p.w13 + (int64_t)ex * 2 * p.f * rb;
        const uint8_t* sbp = (WT >= 2) ? (sh ? p.s13s : p.w13s + (int64_t)ex * 2 * p.f * sb) : nullptr;
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int c = lane + MOE_WAVE * u, j = j0 + r;
                if (c < NC && j < fc) {
                    wg[r][u].load(wb + (int64_t)j * rb, sbp ? sbp + (int64_t)j * sb : nullptr, c);
                    wu[r][u].load(wb + (int64_t)(fc + j) * rb, sbp ? sbp + (int64_t)(fc + j) * sb : nullptr, c);
                } else {
                    wg[r][u].zero();
                    wu[r][u].zero();
                }
            }
    };
    const bool has = item0 < n_items;
    if (has && item0 < s_items) issue(item0, E);
    const int r0 = (has && item0 >= s_items) ? (item0 - s_items) / ngr : -1;

    // top-k on order-preserving keys, k rounds of a wave-wide max (ties to the lowest expert):
    // lane r keeps pick r
    uint32_t key[KPL];
#pragma unroll
    for (int j = 0; j < KPL; ++j) key[j] = lane * KPL + j < E ? sel_ord(lg[j]) : 0u;
    int mine = 0;
    for (int r = 0; r < k; ++r) {
        uint32_t lb = 0u;
        int lj = 0;
#pragma unroll
        for (int j = 0; j < KPL; ++j)
            if (key[j] > lb) {
                lb = key[j];
                lj = j;
            }
        const uint32_t m = wave_max_u32(lb);
        const uint64_t bal = __ballot(lb == m);
        const int wl = __ffsll((unsigned long long)bal) - 1;
        const int wj = __builtin_amdgcn_readlane(lj, wl);
        if (lane == wl) {
#pragma unroll
            for (int j = 0; j < KPL; ++j)
                if (j == wj) key[j] = 0u;
        }
        const int pk = wl * KPL + wj;
        if (lane == r) mine = pk;
        if (r == r0) issue(item0, pk);
    }
    // a pick's sorted position: the number of picks with a lower expert id
    auto pos_of = [&](int ex) { return __popcll(__ballot(lane < k && mine < ex)); };

    // workgroup 0 keeps what it publishes at the end: picks, gates, the slot table (one token:
    // slot = sorted position), the shared slot last
    if (blockIdx.x == 0 && wv == 0) {
        int4* s_slot = reinterpret_cast<int4*>(dyn_lds);
        float* s_logits = reinterpret_cast<float*>(dyn_lds + (size_t)(E + 1) * 16);
        float* s_gate = s_logits + E;
        int* s_sel = reinterpret_cast<int*>(s_gate + k);
#pragma unroll
        for (int j = 0; j < KPL; ++j) {
            const int e = lane * KPL + j;
            if (e < E) s_logits[e] = lg[j];
        }
        const bool pick = lane < k;
        const float m = s_logits[__builtin_amdgcn_readlane(mine, 0)];
        const float term = pick ? expf(s_logits[mine] - m) : 0.0f;
        const float den = wave_sum(term);
        int pos = 0;
        for (int j = 0; j < k; ++j) pos += __builtin_amdgcn_readlane(mine, j) < mine;
        if (pick) {
            s_sel[lane] = mine;
            s_gate[lane] = term / den;
            s_slot[pos] = make_int4(mine, pos, 1, 1);
        }
        if (lane == 0) {
            rs.n_routed = k;
            rs.n_slots = k + (shared_on ? 1 : 0);
            if (shared_on) s_slot[k] = make_int4(E, k, 1, 1);
        }
    }

    // the items: gate/up dot products of the loaded rows, SwiGLU, the output row at its position
    const uint16_t* xr = reinterpret_cast<const uint16_t*>(p.x);
    for (int item = item0; item < n_items; item += stride) {
        const bool sh = item < s_items;
        const int ex = sh ? E : __builtin_amdgcn_readlane(mine, (item - s_items) / ngr);
        if (item != item0) issue(item, ex);
        const int fc = sh ? p.fs : p.f;
        const int j0 = (sh ? item : (item - s_items) % ngr) * R;
        const int pos = sh ? k : pos_of(ex);
        const float gsc = sh ? p.gs13 : p.g13;
        float ag[R], au[R];
#pragma unroll
        for (int r = 0; r < R; ++r) ag[r] = au[r] = 0.0f;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int c = lane + MOE_WAVE * u;
            if (c < NC) {
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    if constexpr (WT == 0) {
                        const float* xf = reinterpret_cast<const float*>(p.x);
                        ag[r] = wg[r][u].dot_f32(xf + (int64_t)c * EC, ag[r]);
                        au[r] = wu[r][u].dot_f32(xf + (int64_t)c * EC, au[r]);
                    } else {
                        ag[r] = wg[r][u].dot_bf16(xr + (int64_t)c * EC, ag[r]);
                        au[r] = wu[r][u].dot_bf16(xr + (int64_t)c * EC, au[r]);
                    }
                }
            }
        }
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const float g = wave_sum(ag[r]) * gsc, u = wave_sum(au[r]) * gsc;
            const int j = j0 + r;
            if (lane == 0 && j < fc) p.a[(int64_t)pos * p.fmax + a_off<EC>(j, p.fmax / EC)] = g / (1.0f + expf(-g)) * u;
        }
    }
    if (blockIdx.x == 0) {
        __syncthreads();
        dec_route_publish(p.rt, rs);
    }
}

template <int WT, int R, int U, int TQ>
__global__ void __launch_bounds__(512, (WT == 1 && TQ == 1) ? 8 : 1) dec_w13(DecFfnArgs p) {
    using W = WChunk<WT>;
    using A = typename DecAct<WT>::T;
    constexpr int EC = W::EC;
    extern __shared__ __attribute__((aligned(16))) unsigned char dyn_lds[];
    __shared__ DecRoute rs;
    const int lane = lane_id();
    const int ngr = (p.f + R - 1) / R, ngs = (p.fs + R - 1) / R;
    const int NC = p.d / EC;
    const int64_t rb = row_bytes(WT, p.d), sb = scale_row_bytes(WT, p.d);
    const int nsteps = (NC + MOE_WAVE * U - 1) / (MOE_WAVE * U);
    const int NWB = blockDim.x / MOE_WAVE;
    if constexpr (TQ == 1) {
        if (p.rt.T == 1 && !p.rt.emask && !p.rt.no_renorm && p.rt.E <= 256 && nsteps == 1) {
            {
                // the routing struct's table, gate and pick arrays, as dec_route_publish reads them
                unsigned char* q = dyn_lds;
                rs.slot = reinterpret_cast<int4*>(q); q += (size_t)(p.rt.E + 1) * 16;
                q += (size_t)p.rt.E * 4;
                rs.gate = reinterpret_cast<float*>(q); q += (size_t)p.rt.k * 4;
                rs.sel = reinterpret_cast<int*>(q);
            }
            if (p.rt.E <= 64) dec_w13_one<WT, R, U, 1>(p, rs, dyn_lds);
            else if (p.rt.E <= 128) dec_w13_one<WT, R, U, 2>(p, rs, dyn_lds);
            else dec_w13_one<WT, R, U, 4>(p, rs, dyn_lds);
            return;
        }
    }
    // The shared expert does not depend on the routing, so its items come first: a wavefront
    // whose first item is one touches the 64-byte pieces of that item's rows (one dword each,
    // the first NP * 4 KB of a row) while its workgroup routes -- after the logits are in LDS,
    // so the routing's own loads never wait behind these -- and its loads after the routing
    // then hit L2.  The dwords are only held until the routing ends.
    constexpr int NP = WT <= 1 ? 2 : 1;
    const bool shared_on = p.rt.n_shared && (!p.rt.emask || p.rt.emask[p.rt.E]);
    const int s_items = shared_on ? ngs : 0;
    const int item0 = blockIdx.x * NWB + wave_id();
    uint32_t warm[2][R][NP];
    auto warm_l2 = [&]() {
        const int j0 = item0 * R;
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int r = 0; r < R; ++r)
#pragma unroll
                for (int i = 0; i < NP; ++i) {
                    const int64_t o = (int64_t)(lane + i * MOE_WAVE) * 64;
                    warm[h][r][i] = 0;
                    if (item0 < s_items && j0 + r < p.fs && o < rb)
                        warm[h][r][i] = *reinterpret_cast<const uint32_t*>(p.s13 + (int64_t)(h * p.fs + j0 + r) * rb + o);
                }
    };
    {
        const int T = p.rt.T, E = p.rt.E, k = p.rt.k;
        unsigned char* q = dyn_lds;
        rs.slot = reinterpret_cast<int4*>(q); q += (size_t)(E + 1) * 16;
        float* s_logits = reinterpret_cast<float*>(q); q += (size_t)T * E * 4;
        float* rs_gate = reinterpret_cast<float*>(q); q += (size_t)T * k * 4;
        int* rs_sel = reinterpret_cast<int*>(q); q += (size_t)T * k * 4;
        rs.gate = rs_gate;
        rs.sel = rs_sel;
        int* s_cnt = reinterpret_cast<int*>(q); q += (size_t)E * 4;
        int* s_mask = reinterpret_cast<int*>(q); q += (size_t)E * 4;
        int* s_on = reinterpret_cast<int*>(q);
        const DecRouteLds L{reinterpret_cast<int4*>(dyn_lds), s_logits, rs_gate, rs_sel, s_cnt, s_mask, s_on};
        dec_route_lds(p.rt, rs, L, warm_l2);
    }
    // an empty asm that takes the warming dwords as inputs keeps their loads (the values
    // themselves are never used) and lets their registers go here
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int i = 0; i < NP; ++i) asm volatile("" ::"v"(warm[h][r][i]));

    const int n_items = s_items + rs.n_routed * ngr;
    for (int item = item0; item < n_items; item += gridDim.x * NWB) {
        const bool sh = item < s_items;
        const int s = sh ? rs.n_routed : (item - s_items) / ngr;
        const int jg = sh ? item : (item - s_items) % ngr;
        // the table sits at the start of the dynamic LDS: read it through that address (a
        // pointer kept in the shared routing struct is a generic one, read by flat loads)
        const int4 S = reinterpret_cast<const int4*>(dyn_lds)[s];
        const int fc = sh ? p.fs : p.f;
        const int j0 = jg * R;
        const uint8_t* wb = sh ? p.s13 : p.w13 + (int64_t)S.x * 2 * p.f * rb;
        const uint8_t* sbp = (WT >= 2) ? (sh ? p.s13s : p.w13s + (int64_t)S.x * 2 * p.f * sb) : nullptr;
        const float gsc = sh ? p.gs13 : p.g13;
        // the slot's tokens in ascending order, TQ at a time; one K step covers a row in the
        // configured shapes, otherwise rows are re-streamed per group of tokens (cache hits)
        uint32_t mask = (uint32_t)S.w;
        int pos = S.y;
        while (mask) {
            int tk[TQ];
            int nq = 0;
#pragma unroll
            for (int q = 0; q < TQ; ++q) {
                tk[q] = -1;
                if (mask) {
                    tk[q] = __ffs(mask) - 1;
                    mask &= mask - 1u;
                    ++nq;
                }
            }
            float ag[R][TQ], au[R][TQ];
#pragma unroll
            for (int r = 0; r < R; ++r)
#pragma unroll
                for (int q = 0; q < TQ; ++q) ag[r][q] = au[r][q] = 0.0f;
            for (int st = 0; st < nsteps; ++st) {
                const int c0 = st * MOE_WAVE * U;
                W wg[R][U], wu[R][U];
#pragma unroll
                for (int r = 0; r < R; ++r)
#pragma unroll
                    for (int u = 0; u < U; ++u) {
                        const int c = c0 + lane + MOE_WAVE * u, j = j0 + r;
                        if (c < NC && j < fc) {
                            wg[r][u].load(wb + (int64_t)j * rb, sbp ? sbp + (int64_t)j * sb : nullptr, c);
                            wu[r][u].load(wb + (int64_t)(fc + j) * rb, sbp ? sbp + (int64_t)(fc + j) * sb : nullptr, c);
                        } else {
                            wg[r][u].zero();
                            wu[r][u].zero();
                        }
                    }
#pragma unroll
                for (int q = 0; q < TQ; ++q) {
                    if (tk[q] < 0) break;
                    const A* xr = reinterpret_cast<const A*>(p.x) + (int64_t)tk[q] * p.d;
#pragma unroll
                    for (int u = 0; u < U; ++u) {
                        const int c = c0 + lane + MOE_WAVE * u;
                        if (c < NC) {
#pragma unroll
                            for (int r = 0; r < R; ++r) {
                                if constexpr (WT == 0) {
                                    ag[r][q] = wg[r][u].dot_f32(xr + (int64_t)c * EC, ag[r][q]);
                                    au[r][q] = wu[r][u].dot_f32(xr + (int64_t)c * EC, au[r][q]);
                                } else {
                                    ag[r][q] = wg[r][u].dot_bf16(xr + (int64_t)c * EC, ag[r][q]);
                                    au[r][q] = wu[r][u].dot_bf16(xr + (int64_t)c * EC, au[r][q]);
                                }
                            }
                        }
                    }
                }
            }
#pragma unroll
            for (int q = 0; q < TQ; ++q) {
                if (q >= nq) break;
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    const float g = wave_sum(ag[r][q]) * gsc, u = wave_sum(au[r][q]) * gsc;
                    const int j = j0 + r;
                    if (lane == 0 && j < fc)
                        p.a[(int64_t)(pos + q) * p.fmax + a_off<EC>(j, p.fmax / EC)] = g / (1.0f + expf(-g)) * u;
                }
            }
            pos += nq;
        }
    }
    if (blockIdx.x == 0) dec_route_publish(p.rt, rs);
}

// ------------------------------------------------------------------------------------------------
// dec_w2c: out[t, i] (+)= sum over slots of g * (W2_e[i] . a[pos]); R rows per workgroup of 8 waves
// ------------------------------------------------------------------------------------------------
template <int WT, int R, int U, bool OUT_BF16>
__global__ void __launch_bounds__(512) dec_w2c(DecFfnArgs p) {
    using W = WChunk<WT>;
    constexpr int EC = W::EC;
    constexpr int NW = 8;
    __shared__ float s_part[NW][R][DEC_MAX_T];
    __shared__ int4 s_slot[MOE_MAX_E + 1];
    __shared__ int s_n;
    const int lane = lane_id(), wv = wave_id(), tid = threadIdx.x;
    // the slot count and the slot table (up to its bound) in one round trip
    if (tid == 0) s_n = p.rt.meta[0];
    for (int s = tid; s < p.slot_bound; s += blockDim.x) s_slot[s] = p.rt.slots[s];
    __syncthreads();
    const int n_slots = s_n;
    const int T = p.T;
    const int i0 = blockIdx.x * R;
    float o[R];
#pragma unroll
    for (int r = 0; r < R; ++r) o[r] = 0.0f;
    for (int s = wv; s < n_slots; s += NW) {
        const int4 S = s_slot[s];
        const bool sh = S.x == p.rt.E;
        const int fc = sh ? p.fs : p.f;
        const int NC = fc / EC;
        const int64_t rb = row_bytes(WT, fc), sbb = scale_row_bytes(WT, fc);
        const uint8_t* base = sh ? p.s2 : p.w2 + (int64_t)S.x * p.d * rb;
        const uint8_t* sbase = (WT >= 2) ? (sh ? p.s2s : p.w2s + (int64_t)S.x * p.d * sbb) : nullptr;
        const float gsc = sh ? p.gs2 : p.g2;
        for (int c0 = 0; c0 < NC; c0 += MOE_WAVE * U) {
            W w[R][U];
#pragma unroll
            for (int r = 0; r < R; ++r)
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int i = i0 + r, c = c0 + lane + MOE_WAVE * u;
                    if (i < p.d && c < NC) w[r][u].load(base + (int64_t)i * rb, sbase ? sbase + (int64_t)i * sbb : nullptr, c);
                    else w[r][u].zero();
                }
            uint32_t mask = (uint32_t)S.w;
            for (int q = 0; q < S.z; ++q) {
                const int t = __ffs(mask) - 1;
                mask &= mask - 1u;
                const int pos = S.y + q;
                const float g = p.rt.pos_gate[pos];
                const float* ar = p.a + (int64_t)pos * p.fmax;
                float acc[R];
#pragma unroll
                for (int r = 0; r < R; ++r) acc[r] = 0.0f;
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int c = c0 + lane + MOE_WAVE * u;
                    if (c < NC) {
                        float av[EC];
                        a_chunk<EC>(ar, p.fmax / EC, c, av);
#pragma unroll
                        for (int r = 0; r < R; ++r) acc[r] = w[r][u].dot_f32(av, acc[r]);
                    }
                }
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    const float y = wave_sum(acc[r]) * gsc;
                    if (lane == t) o[r] = fmaf(g, y, o[r]);
                }
            }
        }
    }
    if (lane < DEC_MAX_T) {
#pragma unroll
        for (int r = 0; r < R; ++r) s_part[wv][r][lane] = o[r];
    }
    __syncthreads();
    if (wv == 0 && lane < T) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int i = i0 + r;
            if (i >= p.d) continue;
            float v = 0.0f;
#pragma unroll
            for (int w8 = 0; w8 < NW; ++w8) v += s_part[w8][r][lane];
            const int64_t off = (int64_t)lane * p.d + i;
            if (OUT_BF16) {
                uint16_t* out = reinterpret_cast<uint16_t*>(p.out);
                const float prev = p.accumulate ? bf16_to_f32(out[off]) : 0.0f;
                out[off] = f32_to_bf16(prev + v);
            } else {
                float* out = reinterpret_cast<float*>(p.out);
                const float prev = p.accumulate ? out[off] : 0.0f;
                out[off] = prev + v;
            }
        }
    }
}

// ------------------------------------------------------------------------------------------------
// dec_w2c1: the down kernel for a single token.  The workgroup's (slot, row) units, slot-major,
// are cut into 8 contiguous ranges, one per wavefront, so every wavefront streams about the
// same number of weight rows whatever the slot count (8 wavefronts over 9 slots would otherwise
// leave one wavefront with two slots and the others with one).  A wavefront issues the loads of
// up to MAXU units at once, then adds g * y for each unit into its LDS row partials; the 8
// partials of a row are added in wavefront order, which keeps the ascending-slot order.
// ------------------------------------------------------------------------------------------------
template <int WT, int R, int U, int MAXU, bool OUT_BF16>
__global__ void __launch_bounds__(512, 2) dec_w2c1(DecFfnArgs p) {
    using W = WChunk<WT>;
    constexpr int EC = W::EC;
    constexpr int NW = 8;
    __shared__ float s_part[NW][R];
    __shared__ int4 s_slot[MOE_MAX_K + 1];
    __shared__ float s_pg[MOE_MAX_K + 1];
    __shared__ int s_n;
    const int lane = lane_id(), wv = wave_id(), tid = threadIdx.x;
    // slot count, slot table and the per-position gates in one round trip
    if (tid == 0) s_n = p.rt.meta[0];
    for (int s = tid; s < p.slot_bound; s += blockDim.x) s_slot[s] = p.rt.slots[s];
    for (int i = tid; i <= p.k; i += blockDim.x) s_pg[i] = p.rt.pos_gate[i];
    if (tid < NW * R) (&s_part[0][0])[tid] = 0.0f;
    __syncthreads();
    const int n_slots = s_n, E = p.rt.E, ncp = p.fmax / EC;
    const int i0 = blockIdx.x * R;
    const int nu = n_slots * R;
    const int u_lo = wv * nu / NW, u_hi = (wv + 1) * nu / NW;
    for (int b0 = u_lo; b0 < u_hi; b0 += MAXU) {
        const int nb = min(MAXU, u_hi - b0);
        W w[MAXU][U];
#pragma unroll
        for (int j = 0; j < MAXU; ++j) {
            const int u = b0 + j, s = u / R, i = i0 + u % R;
            if (j < nb && i < p.d) {
                const int4 S = s_slot[s];
                const bool sh = S.x == E;
                const int fc = sh ? p.fs : p.f, NC = fc / EC;
                const int64_t rb = row_bytes(WT, fc), sbb = scale_row_bytes(WT, fc);
                const uint8_t* row = (sh ? p.s2 : p.w2 + (int64_t)S.x * p.d * rb) + (int64_t)i * rb;
                const uint8_t* srow = (WT >= 2) ? (sh ? p.s2s : p.w2s + (int64_t)S.x * p.d * sbb) + (int64_t)i * sbb : nullptr;
#pragma unroll
                for (int v = 0; v < U; ++v) {
                    const int c = lane + MOE_WAVE * v;
                    if (c < NC) w[j][v].load(row, srow, c);
                    else w[j][v].zero();
                }
            } else {
#pragma unroll
                for (int v = 0; v < U; ++v) w[j][v].zero();
            }
        }
        int cur = -1, NC = 0;
        float g = 0.0f, gsc = 1.0f;
        float av[U][EC];
#pragma unroll
        for (int j = 0; j < MAXU; ++j) {
            if (j < nb) {
                const int u = b0 + j, s = u / R, r = u % R;
                if (s != cur) {
                    const int4 S = s_slot[s];
                    const bool sh = S.x == E;
                    NC = (sh ? p.fs : p.f) / EC;
                    g = s_pg[S.y];
                    gsc = sh ? p.gs2 : p.g2;
                    const float* ar = p.a + (int64_t)S.y * p.fmax;
#pragma unroll
                    for (int v = 0; v < U; ++v) {
                        const int c = lane + MOE_WAVE * v;
                        if (c < NC) a_chunk<EC>(ar, ncp, c, av[v]);
                    }
                    cur = s;
                }
                float acc = 0.0f;
#pragma unroll
                for (int v = 0; v < U; ++v)
                    if (lane + MOE_WAVE * v < NC) acc = w[j][v].dot_f32(av[v], acc);
                const float y = wave_sum(acc) * gsc;
                if (lane == 0) s_part[wv][r] = fmaf(g, y, s_part[wv][r]);
            }
        }
    }
    __syncthreads();
    if (tid < R && i0 + tid < p.d) {
        float v = 0.0f;
#pragma unroll
        for (int w8 = 0; w8 < NW; ++w8) v += s_part[w8][tid];
        const int i = i0 + tid;
        if (OUT_BF16) {
            uint16_t* out = reinterpret_cast<uint16_t*>(p.out);
            const float prev = p.accumulate ? bf16_to_f32(out[i]) : 0.0f;
            out[i] = f32_to_bf16(prev + v);
        } else {
            float* out = reinterpret_cast<float*>(p.out);
            const float prev = p.accumulate ? out[i] : 0.0f;
            out[i] = prev + v;
        }
    }
}

// ------------------------------------------------------------------------------------------------
// dec_stack: the residual stack for one token, n_layers decode layers in ONE cooperative launch of
// resident workgroups (the 43-layer decode of the FreeToken/dothoosh page, "Architecture and the
// sparsity puzzle", without a kernel boundary between layers).  Each layer runs the three
// launches above as phases separated by grid barriers:
//   logits   wavefront wv of workgroup b computes router row e = b + G*wv exactly as dec_logits
//            does, with its row of W_r loaded before the barrier that opens the phase;
//   gate/up  every workgroup routes from the logits in LDS, issues the loads of the down
//            projection's weight rows for its own output rows (the slot table decides them), then
//            runs dec_w13's items; the down rows land while the gate/up stream runs;
//   down     dec_w2c1 on those rows; writes h for the next layer.
// The per-row arithmetic and every summation order are those of the three launches, so the
// results are equal bit for bit.
// Data that crosses workgroups goes through device-scope (sc1) stores, written through to memory.
// Readers of lines that several workgroups write (logits, a) use device-scope loads; the rest
// (x, written whole by one wavefront; h between layers, one 128-byte line per 8-row block) sit in
// regions of their own per layer that no cache can hold from before the write.  A barrier therefore
// needs the store completions (s_waitcnt vmcnt(0) at every thread) and the counters, and no cache
// write-back or invalidation.  Barrier: per-group arrival counters (group = workgroup % 32, one
// 256-byte line each), the group's last arrival bumps a top counter, the top's last arrival writes
// the release value into one flag line per group.  Every wait is bounded: a wait that runs out
// sets an error word, and every workgroup leaves at its next barrier, so the launch always ends.
// ------------------------------------------------------------------------------------------------
constexpr int STACK_GROUPS = 32, STACK_LINE = 64;  // ints per 256-byte line
constexpr int STACK_ERR = (2 * STACK_GROUPS + 1) * STACK_LINE;  // index of the error word

// Returns false when this wait, or one in another workgroup, ran out.
__device__ __forceinline__ bool stack_barrier(int* bar, int idx, int spin_limit, int* s_ok) {
    __syncthreads();
    if (threadIdx.x == 0) {
        const int G = gridDim.x, g = blockIdx.x % STACK_GROUPS;
        const int ng = G < STACK_GROUPS ? G : STACK_GROUPS;
        const int in_g = (G - g + STACK_GROUPS - 1) / STACK_GROUPS;  // workgroups of group g
        int* flags = bar + (STACK_GROUPS + 1) * STACK_LINE;
        int* err = bar + STACK_ERR;
        bool ok = __hip_atomic_load(err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0;
        if (ok) {
            const int old = __hip_atomic_fetch_add(bar + g * STACK_LINE, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (old + 1 == (idx + 1) * in_g) {
                const int t = __hip_atomic_fetch_add(bar + STACK_GROUPS * STACK_LINE, 1, __ATOMIC_RELAXED,
                                                     __HIP_MEMORY_SCOPE_AGENT);
                if (t + 1 == (idx + 1) * ng)
                    for (int r = 0; r < ng; ++r)
                        __hip_atomic_store(flags + r * STACK_LINE, idx + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
            const int* f = flags + g * STACK_LINE;
            int spins = 0;
            while (__hip_atomic_load(f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < idx + 1) {
                if (++spins > spin_limit ||
                    ((spins & 31) == 0 && __hip_atomic_load(err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0)) {
                    __hip_atomic_store(err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    ok = false;
                    break;
                }
                __builtin_amdgcn_s_sleep(1);
            }
        }
        *s_ok = ok ? 1 : 0;
    }
    __syncthreads();
    return *s_ok != 0;
}

// Every store of this thread has completed (device-scope stores: reached memory).
__device__ __forceinline__ void stores_done() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

__device__ __forceinline__ void store_dev(float* p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_dev(uint32_t* p, uint32_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
// a_chunk<32> with device-scope loads: the eight 16-byte pieces of chunk c of a row of `a`,
// issued together and waited for in the same statement.
__device__ __forceinline__ void a_chunk32_dev(const float* row, int ncp, int c, float (&out)[32]) {
    const float4* r4 = reinterpret_cast<const float4*>(row);
    u32x4_t v0, v1, v2, v3, v4, v5, v6, v7;
    asm volatile(
        "global_load_dwordx4 %0, %8, off sc1\n\t"
        "global_load_dwordx4 %1, %9, off sc1\n\t"
        "global_load_dwordx4 %2, %10, off sc1\n\t"
        "global_load_dwordx4 %3, %11, off sc1\n\t"
        "global_load_dwordx4 %4, %12, off sc1\n\t"
        "global_load_dwordx4 %5, %13, off sc1\n\t"
        "global_load_dwordx4 %6, %14, off sc1\n\t"
        "global_load_dwordx4 %7, %15, off sc1\n\t"
        "s_waitcnt vmcnt(0)"
        : "=&v"(v0), "=&v"(v1), "=&v"(v2), "=&v"(v3), "=&v"(v4), "=&v"(v5), "=&v"(v6), "=&v"(v7)
        : "v"(r4 + (int64_t)0 * ncp + c), "v"(r4 + (int64_t)1 * ncp + c), "v"(r4 + (int64_t)2 * ncp + c),
          "v"(r4 + (int64_t)3 * ncp + c), "v"(r4 + (int64_t)4 * ncp + c), "v"(r4 + (int64_t)5 * ncp + c),
          "v"(r4 + (int64_t)6 * ncp + c), "v"(r4 + (int64_t)7 * ncp + c)
        : "memory");
    const u32x4_t v[8] = {v0, v1, v2, v3, v4, v5, v6, v7};
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        out[4 * q] = __uint_as_float(v[q].x);
        out[4 * q + 1] = __uint_as_float(v[q].y);
        out[4 * q + 2] = __uint_as_float(v[q].z);
        out[4 * q + 3] = __uint_as_float(v[q].w);
    }
}

constexpr int STACK_MAX_LAYERS = STACK_LAYERS_PER_LAUNCH;
constexpr int STACK_HB = 32;  // floats per 8-row block of h between layers (one 128-byte line)

struct StackLayer {
    const uint16_t* wr;   // [E, d] bf16
    const float* br;      // [E] or NULL
    const uint8_t* w13;   // MXFP4 codes [E, 2f, d/2]
    const uint8_t* w13s;  // [E, 2f, d/32]
    const uint8_t* w2;    // [E, d, f/2]
    const uint8_t* w2s;   // [E, d, f/32]
};

struct StackArgs {
    StackLayer layer[STACK_MAX_LAYERS];
    float* h;          // [d], the caller's: the first layer's input, the last layer's output
    float* hbuf;       // n_layers - 1 regions of sh_h floats: h between layers, 8-row blocks of STACK_HB
    float* logits;     // n_layers regions of sh_lg floats
    uint16_t* xn;      // n_layers regions of sh_xn elements: x = bf16(h * inv_rms)
    float* a;          // n_layers regions of sh_a floats: k rows of f, chunk-transposed (a_off)
    int32_t* idx_out;  // nullable [n_layers, k]
    int* bar;          // barrier counters, flags and error word, zero at launch
    int64_t sh_h, sh_lg, sh_xn, sh_a;
    int n_layers, d, f, E, k, no_renorm, spin_limit;
};

template <int R13, int U13, int R2, int MAXU2>
__global__ void __launch_bounds__(512, 2) dec_stack(StackArgs p) {
    using W = WChunk<2>;
    constexpr int EC = W::EC;   // 32 elements per weight chunk
    constexpr int NW = 8;       // wavefronts per workgroup
    static_assert(R2 == 8, "h between layers is kept in 8-row blocks");
    extern __shared__ __attribute__((aligned(16))) unsigned char dyn_lds[];
    __shared__ DecRoute rs;
    __shared__ float s_part[2][NW][R2];
    __shared__ float s_pg[MOE_MAX_K + 1];
    __shared__ int s_ok;
    const int lane = lane_id(), wv = wave_id(), tid = threadIdx.x;
    const int G = gridDim.x;
    const int d = p.d, f = p.f, E = p.E, k = p.k;
    const int NCX = d / 8;                         // 16-byte chunks of a bf16 row of d
    const int NC13 = d / EC, NC2 = f / EC, ncp = f / EC;
    const int64_t rb13 = row_bytes(2, d), sb13 = scale_row_bytes(2, d);
    const int64_t rb2 = row_bytes(2, f), sb2 = scale_row_bytes(2, f);
    const int ngr = (f + R13 - 1) / R13;
    const int nsteps = (NC13 + MOE_WAVE * U13 - 1) / (MOE_WAVE * U13);
    const int n_rb = (d + R2 - 1) / R2;            // 8-row blocks of the output

    // this wavefront's router row, loaded ahead of the phase that uses it
    const int e_mine = blockIdx.x + G * wv;
    uint4 wc[8];
    auto load_router_row = [&](int l) {
        const uint4* w = reinterpret_cast<const uint4*>(p.layer[l].wr + (int64_t)(e_mine < E ? e_mine : E - 1) * d);
#pragma unroll
        for (int b = 0; b < 8; ++b) {
            const int c = lane + MOE_WAVE * b;
            wc[b] = (e_mine < E && c < NCX) ? w[c] : make_uint4(0u, 0u, 0u, 0u);
        }
    };

    // routing LDS (as dec_w13); the phases below read the table through these local pointers,
    // which the compiler keeps as LDS addresses (through rs.* it would use flat loads, whose
    // waits also drain every global load in flight)
    unsigned char* q = dyn_lds;
    int4* const s_slot = reinterpret_cast<int4*>(q); q += (size_t)(E + 1) * 16;
    float* const s_logits = reinterpret_cast<float*>(q); q += (size_t)E * 4;
    float* const s_gate = reinterpret_cast<float*>(q); q += (size_t)k * 4;
    int* const s_sel = reinterpret_cast<int*>(q); q += (size_t)k * 4;
    int* const s_cnt = reinterpret_cast<int*>(q); q += (size_t)E * 4;
    int* const s_mask = reinterpret_cast<int*>(q); q += (size_t)E * 4;
    int* const s_on = reinterpret_cast<int*>(q);
    if (tid == 0) {
        rs.slot = s_slot;
        rs.gate = s_gate;
        rs.sel = s_sel;
    }
    __syncthreads();

    load_router_row(0);
    int bi = 0;
    for (int l = 0; l < p.n_layers; ++l) {
        const StackLayer& Lw = p.layer[l];
        const bool first = l == 0, last = l == p.n_layers - 1;
        const float* hin = first ? p.h : p.hbuf + (int64_t)(l - 1) * p.sh_h;
        float* hout = last ? p.h : p.hbuf + (int64_t)l * p.sh_h;
        const int hstride = first ? 8 : STACK_HB;  // floats from one 8-element chunk of h to the next
        float* lg = p.logits + (int64_t)l * p.sh_lg;
        uint16_t* xn = p.xn + (int64_t)l * p.sh_xn;
        float* a = p.a + (int64_t)l * p.sh_a;

        // ---- logits: dec_logits' single-pass residual-stack branch
        if (e_mine < E) {
            float4 hv[8][2];
#pragma unroll
            for (int b = 0; b < 8; ++b) {
                const int c = lane + MOE_WAVE * b;
                const float4* hc = reinterpret_cast<const float4*>(hin + (int64_t)c * hstride);
#pragma unroll
                for (int q = 0; q < 2; ++q) hv[b][q] = c < NCX ? hc[q] : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
            }
            float ss = 0.0f;
#pragma unroll
            for (int b = 0; b < 8; ++b)
#pragma unroll
                for (int q = 0; q < 2; ++q) {
                    ss = fmaf(hv[b][q].x, hv[b][q].x, ss); ss = fmaf(hv[b][q].y, hv[b][q].y, ss);
                    ss = fmaf(hv[b][q].z, hv[b][q].z, ss); ss = fmaf(hv[b][q].w, hv[b][q].w, ss);
                }
            const float inv = 1.0f / sqrtf(wave_sum(ss) / (float)d + 1e-6f);
            float acc = 0.0f;
#pragma unroll
            for (int b = 0; b < 8; ++b) {
                const int c = lane + MOE_WAVE * b;
                if (c < NCX) {
                    const uint4 xc = make_uint4(pack_bf16x2(hv[b][0].x * inv, hv[b][0].y * inv),
                                                pack_bf16x2(hv[b][0].z * inv, hv[b][0].w * inv),
                                                pack_bf16x2(hv[b][1].x * inv, hv[b][1].y * inv),
                                                pack_bf16x2(hv[b][1].z * inv, hv[b][1].w * inv));
                    acc += dot_chunk<uint16_t>(wc[b], xc);
                    if (e_mine == 0) {
                        uint32_t* xo = reinterpret_cast<uint32_t*>(xn + (int64_t)c * 8);
                        store_dev(xo, xc.x); store_dev(xo + 1, xc.y); store_dev(xo + 2, xc.z); store_dev(xo + 3, xc.w);
                    }
                }
            }
            acc = wave_sum(acc);
            if (lane == 0) store_dev(lg + e_mine, acc + (Lw.br ? Lw.br[e_mine] : 0.0f));
        }
        stores_done();
        if (!stack_barrier(p.bar, bi++, p.spin_limit, &s_ok)) return;

        // ---- routing (every workgroup, in LDS), then the down rows' loads, then gate/up
        {
            const DecRouteIO io{lg, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 1, E, k, 0, p.no_renorm, nullptr};
            const DecRouteLds L{s_slot, s_logits, s_gate, s_sel, s_cnt, s_mask, s_on};
            dec_route_lds<true>(io, rs, L, [] {});
        }
        const int n_slots = rs.n_slots, n_routed = rs.n_routed;
        if (tid < n_slots) {
            // the gate of each slot's position (one token: position = slot index)
            const int4 S = s_slot[tid];
            float g = 1.0f;
            for (int j = 0; j < k; ++j)
                if (s_sel[j] == S.x) g = s_gate[j];
            s_pg[S.y] = g;
        }
        if (blockIdx.x == 0 && tid < k && p.idx_out) p.idx_out[(int64_t)l * k + tid] = s_sel[tid];
        const uint8_t* const w13p = Lw.w13;
        const uint8_t* const w13sp = Lw.w13s;
        const uint8_t* const w2p = Lw.w2;
        const uint8_t* const w2sp = Lw.w2s;
        if (tid < 2 * NW * R2) (&s_part[0][0][0])[tid] = 0.0f;

        // dec_w2c1's first batch of this workgroup's first row block, loaded now (a second
        // block's would not fit the registers beside the gate/up stream's)
        const int nu = n_slots * R2;
        const int u_lo = wv * nu / NW, u_hi = (wv + 1) * nu / NW;
        // (lanes past the row's chunks load its last chunk, which they never use: every branch
        // here is wave-uniform, so the loads go out back to back)
        const int c2 = lane < NC2 ? lane : NC2 - 1;
        auto load_down = [&](W (&dst)[MAXU2], int rb, int b0) {
            const int nb = min(MAXU2, u_hi - b0);
#pragma unroll
            for (int j = 0; j < MAXU2; ++j) {
                const int u = b0 + j, s = u / R2, i = rb * R2 + u % R2;
                if (j < nb && i < d) {
                    const int e = s_slot[s].x;
                    dst[j].load(w2p + ((int64_t)e * d + i) * rb2, w2sp + ((int64_t)e * d + i) * sb2, c2);
                } else {
                    dst[j].zero();
                }
            }
        };
        const int rb0 = blockIdx.x;
        W w2r[MAXU2];
        if (rb0 < n_rb && u_lo < u_hi) load_down(w2r, rb0, u_lo);
        __syncthreads();  // s_pg, s_part

        // gate/up items (dec_w13, one token)
        {
            const int n_items = n_routed * ngr;
            const uint16_t* xr = xn;
            for (int item = blockIdx.x * NW + wv; item < n_items; item += G * NW) {
                const int s = item / ngr, jg = item % ngr;
                const int4 S = s_slot[s];
                const int j0 = jg * R13;
                const uint8_t* wb = w13p + (int64_t)S.x * 2 * f * rb13;
                const uint8_t* sbp = w13sp + (int64_t)S.x * 2 * f * sb13;
                float ag[R13], au[R13];
#pragma unroll
                for (int r = 0; r < R13; ++r) ag[r] = au[r] = 0.0f;
                for (int st = 0; st < nsteps; ++st) {
                    const int c0 = st * MOE_WAVE * U13;
                    W wg[R13][U13], wu[R13][U13];
#pragma unroll
                    for (int r = 0; r < R13; ++r)
#pragma unroll
                        for (int u = 0; u < U13; ++u) {
                            const int c = c0 + lane + MOE_WAVE * u, j = j0 + r;
                            if (c < NC13 && j < f) {
                                wg[r][u].load(wb + (int64_t)j * rb13, sbp + (int64_t)j * sb13, c);
                                wu[r][u].load(wb + (int64_t)(f + j) * rb13, sbp + (int64_t)(f + j) * sb13, c);
                            } else {
                                wg[r][u].zero();
                                wu[r][u].zero();
                            }
                        }
#pragma unroll
                    for (int u = 0; u < U13; ++u) {
                        const int c = c0 + lane + MOE_WAVE * u;
                        if (c < NC13) {
#pragma unroll
                            for (int r = 0; r < R13; ++r) {
                                ag[r] = wg[r][u].dot_bf16(xr + (int64_t)c * EC, ag[r]);
                                au[r] = wu[r][u].dot_bf16(xr + (int64_t)c * EC, au[r]);
                            }
                        }
                    }
                }
#pragma unroll
                for (int r = 0; r < R13; ++r) {
                    const float g = wave_sum(ag[r]), u = wave_sum(au[r]);
                    const int j = j0 + r;
                    if (lane == 0 && j < f) store_dev(a + (int64_t)S.y * f + a_off<EC>(j, ncp), g / (1.0f + expf(-g)) * u);
                }
            }
        }
        stores_done();
        if (!stack_barrier(p.bar, bi++, p.spin_limit, &s_ok)) return;

        // ---- down projection + combine (dec_w2c1, one token) on this workgroup's row blocks, two
        //      at a time (blocks rb and rb + G share the slots, so one read of each slot's `a`
        //      serves both); wa holds block rb's first batch (loaded before the barrier) when pre
        auto down_pair = [&](int rbA, int rbB, W (&wa)[MAXU2], bool pre) {
            for (int b0 = u_lo; b0 < u_hi; b0 += MAXU2) {
                if (!pre || b0 != u_lo) load_down(wa, rbA, b0);
                W wb[MAXU2];
                if (rbB >= 0) load_down(wb, rbB, b0);
                const int nb = min(MAXU2, u_hi - b0);
                int cur = -1;
                float g = 0.0f;
                float av[EC];
#pragma unroll
                for (int j = 0; j < MAXU2; ++j) {
                    if (j < nb) {
                        const int u = b0 + j, s = u / R2, r = u % R2;
                        if (s != cur) {
                            const int4 S = s_slot[s];
                            g = s_pg[S.y];
                            if (lane < NC2) a_chunk32_dev(a + (int64_t)S.y * f, ncp, lane, av);
                            cur = s;
                        }
                        float acc = 0.0f;
                        if (lane < NC2) acc = wa[j].dot_f32(av, acc);
                        const float y = wave_sum(acc);
                        if (lane == 0) s_part[0][wv][r] = fmaf(g, y, s_part[0][wv][r]);
                        if (rbB >= 0) {
                            float acc2 = 0.0f;
                            if (lane < NC2) acc2 = wb[j].dot_f32(av, acc2);
                            const float y2 = wave_sum(acc2);
                            if (lane == 0) s_part[1][wv][r] = fmaf(g, y2, s_part[1][wv][r]);
                        }
                    }
                }
            }
            __syncthreads();
            const int hb = tid / R2, rt = tid % R2, rb = hb == 0 ? rbA : rbB;
            if (tid < 2 * R2 && rb >= 0 && rb * R2 + rt < d) {
                float v = 0.0f;
#pragma unroll
                for (int w8 = 0; w8 < NW; ++w8) v += s_part[hb][w8][rt];
                const int i = rb * R2 + rt;
                const float* hp = first ? hin + i : hin + (int64_t)rb * STACK_HB + rt;
                const float prev = __hip_atomic_load(hp, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                store_dev(last ? hout + i : hout + (int64_t)rb * STACK_HB + rt, prev + v);
            }
            __syncthreads();
            if (tid < 2 * NW * R2) (&s_part[0][0][0])[tid] = 0.0f;
        };
        for (int rb = rb0; rb < n_rb; rb += 2 * G) down_pair(rb, rb + G < n_rb ? rb + G : -1, w2r, rb == rb0);
        stores_done();
        if (!last) load_router_row(l + 1);
        if (!stack_barrier(p.bar, bi++, p.spin_limit, &s_ok)) return;
    }
}

__global__ void stack_clear(int* bar, int n) {
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) bar[i] = 0;
}

// ------------------------------------------------------------------------------------------------
// Host side
// ------------------------------------------------------------------------------------------------
bool dec_supported(int T, int E, int k) {
    return T >= 1 && T <= DEC_MAX_T && T * E <= DEC_MAX_TE && k <= MOE_MAX_K && dec_route_lds_bytes(T, E, k) <= 60 * 1024;
}

hipError_t launch_dec_logits(int act_dtype, const void* x, const void* wr, const float* b, float* logits, void* xn,
                             int T, int d, int E, bool prenorm, hipStream_t st) {
    DecLogitsArgs p{x, wr, b, logits, xn, T, d, E, prenorm ? 1 : 0};
    // one wavefront per workgroup: the router rows spread over up to E compute units instead of
    // E / 4 (each wavefront's loads all go out at once; fewer per CU means less queueing)
    const dim3 grid(E, T), block(MOE_WAVE);
    if (act_dtype == 0) hipLaunchKernelGGL((dec_logits<float>), grid, block, 0, st, p);
    else hipLaunchKernelGGL((dec_logits<uint16_t>), grid, block, 0, st, p);
    return hipGetLastError();
}

// Workgroups of `kernel` that are resident on the current device at once: its occupancy per CU
// (registers, LDS) times the CU count, cached per (kernel, device, LDS bytes).
static int resident_blocks(const void* kernel, int threads, size_t lds) {
    static std::mutex mu;
    static std::map<std::tuple<const void*, int, size_t>, int> cache;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) dev = -1;
    std::lock_guard<std::mutex> lock(mu);
    const auto key = std::make_tuple(kernel, dev, lds);
    const auto it = cache.find(key);
    if (it != cache.end()) return it->second;
    int cus = 0, per_cu = 0;
    if (dev < 0 || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
        cus = 256;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, lds) != hipSuccess || per_cu < 1)
        per_cu = 1;
    return cache[key] = per_cu * cus;
}

// The gate/up grid fills the device exactly once (every workgroup redoes the routing, so a
// second round of workgroups would pay it again), capped by the items there can be.
static unsigned dec_grid(int64_t max_items, int resident) {
    int64_t blocks = (max_items + 7) / 8;
    if (blocks > resident) blocks = resident;
    return (unsigned)(blocks < 1 ? 1 : blocks);
}

hipError_t launch_dec_ffn(int wt, bool out_bf16, const void* x, const float* logits, int32_t* topk_idx,
                          float* topk_w, int32_t* idx_out, int32_t* meta, int4* slots, float* pos_gate,
                          bool no_renorm, const void* w13, const uint8_t* w13s, const void* s13, const uint8_t* s13s,
                          const void* w2, const uint8_t* w2s, const void* s2, const uint8_t* s2s, float* a, void* out,
                          int T, int d, int f, int fs, int k, int E, int n_shared, bool accumulate,
                          const uint8_t* mask, const float* gsc, hipStream_t st) {
    const int fmax = (n_shared && fs > f) ? fs : f;
    DecRouteIO rt{logits, topk_idx, topk_w, idx_out, meta, slots, pos_gate, T, E, k, n_shared, no_renorm ? 1 : 0, mask};
    const int64_t max_slots = (int64_t)(T * k < E ? T * k : E);
    DecFfnArgs p{x, rt, (const uint8_t*)w13, w13s, (const uint8_t*)s13, s13s, (const uint8_t*)w2, w2s,
                 (const uint8_t*)s2, s2s, a, out, T, d, f, n_shared ? fs : 0, fmax, k, accumulate ? 1 : 0,
                 (int)max_slots + n_shared, gsc[0], gsc[1], gsc[2], gsc[3]};
    const size_t lds = dec_route_lds_bytes(T, E, k);
#define MOE_DW13Q(WTV, RV, UV, TQV)                                                                              \
    do {                                                                                                         \
        const int64_t items = max_slots * ((f + RV - 1) / RV) + (n_shared ? (fs + RV - 1) / RV : 0);             \
        const int res = resident_blocks((const void*)dec_w13<WTV, RV, UV, TQV>, 512, lds);                      \
        MOE_LAUNCH(PROF_FFN_UP, (dec_w13<WTV, RV, UV, TQV>), dim3(dec_grid(items, res)), dim3(512), lds, st, p); \
    } while (0)
    // one token needs a single accumulator per row (fewer registers, more resident wavefronts)
#define MOE_DW13(WTV, RV, UV)                 \
    do {                                      \
        if (T == 1) MOE_DW13Q(WTV, RV, UV, 1); \
        else MOE_DW13Q(WTV, RV, UV, 4);       \
    } while (0)
    // about 8 16-byte loads per lane in flight per item (HBM streams best at 4-8 per lane)
    if (wt == 0) MOE_DW13(0, 2, 1);
    else if (wt == 1) MOE_DW13(1, 1, 4);
    else if (wt == 2) MOE_DW13(2, 2, 2);
    else MOE_DW13(3, 1, 2);
#undef MOE_DW13
#undef MOE_DW13Q
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
#define MOE_DW2(WTV, RV, UV)                                                                                     \
    do {                                                                                                         \
        const dim3 grid((d + RV - 1) / RV);                                                                      \
        if (out_bf16) MOE_LAUNCH(PROF_FFN_DOWN, (dec_w2c<WTV, RV, UV, true>), grid, dim3(512), 0, st, p);         \
        else MOE_LAUNCH(PROF_FFN_DOWN, (dec_w2c<WTV, RV, UV, false>), grid, dim3(512), 0, st, p);                 \
    } while (0)
#define MOE_DW21(WTV, RV, UV, MU)                                                                               \
    do {                                                                                                         \
        const dim3 grid((d + RV - 1) / RV);                                                                      \
        if (out_bf16) MOE_LAUNCH(PROF_FFN_DOWN, (dec_w2c1<WTV, RV, UV, MU, true>), grid, dim3(512), 0, st, p);    \
        else MOE_LAUNCH(PROF_FFN_DOWN, (dec_w2c1<WTV, RV, UV, MU, false>), grid, dim3(512), 0, st, p);            \
    } while (0)
    // one token: (slot, row) units split evenly over the wavefronts, when a row is one step
    const int ec = wt == 0 ? 4 : (wt == 1 ? 8 : 32);
    const int u1 = wt == 1 ? 2 : 1;
    if (T == 1 && fmax / ec <= MOE_WAVE * u1) {
        if (wt == 0) MOE_DW21(0, 4, 1, 8);
        else if (wt == 1) MOE_DW21(1, 4, 2, 6);
        else if (wt == 2) MOE_DW21(2, 8, 1, 6);
        else MOE_DW21(3, 8, 1, 6);
    } else {
        if (wt == 0) MOE_DW2(0, 4, 1);
        else if (wt == 1) MOE_DW2(1, 4, 2);
        else if (wt == 2) MOE_DW2(2, 16, 1);
        else MOE_DW2(3, 16, 1);
    }
#undef MOE_DW21
#undef MOE_DW2
    return hipGetLastError();
}


int dec_stack_bar_ints() { return STACK_ERR + STACK_LINE; }
int dec_stack_err_index() { return STACK_ERR; }

bool dec_stack_supported(int d, int f, int E, int k) {
    // x chunks of one row in one pass per lane (d <= 4096), one weight chunk per lane and row of
    // the down projection (f <= 2048): the shapes whose three-launch path is dec_logits'
    // single-pass branch and dec_w2c1
    return d % 32 == 0 && d / 8 <= MOE_WAVE * 8 && f % 32 == 0 && f / 32 <= MOE_WAVE && dec_supported(1, E, k);
}

hipError_t launch_dec_stack(const StackLayerPtrs* layers, int n_layers, float* h, float* hbuf, float* logits,
                            uint16_t* xn, float* a, int32_t* idx_out, int* bar, int64_t sh_h, int64_t sh_lg,
                            int64_t sh_xn, int64_t sh_a, int d, int f, int E, int k, bool no_renorm, int spin_limit,
                            bool clear_err, hipStream_t st) {
    if (n_layers < 1 || n_layers > STACK_MAX_LAYERS) return hipErrorInvalidValue;
    StackArgs p{};
    for (int l = 0; l < n_layers; ++l)
        p.layer[l] = StackLayer{(const uint16_t*)layers[l].wr, layers[l].br, (const uint8_t*)layers[l].w13,
                                layers[l].w13s, (const uint8_t*)layers[l].w2, layers[l].w2s};
    p.h = h; p.hbuf = hbuf; p.logits = logits; p.xn = xn; p.a = a; p.idx_out = idx_out; p.bar = bar;
    p.sh_h = sh_h; p.sh_lg = sh_lg; p.sh_xn = sh_xn; p.sh_a = sh_a;
    p.n_layers = n_layers; p.d = d; p.f = f; p.E = E; p.k = k; p.no_renorm = no_renorm ? 1 : 0;
    p.spin_limit = spin_limit;
    // the three-launch path's tiles: dec_w13<2, 2, 2, 1> and dec_w2c1<2, 8, 1, 6>
    constexpr int R13 = 2, U13 = 2, R2 = 8, MAXU2 = 6;
    const void* kern = reinterpret_cast<const void*>(&dec_stack<R13, U13, R2, MAXU2>);
    const size_t lds = dec_route_lds_bytes(1, E, k);
    const int resident = resident_blocks(kern, 512, lds);
    const int n_rb = (d + R2 - 1) / R2;
    const int G = resident < n_rb ? resident : n_rb;
    if (G * 8 < E) return hipErrorInvalidConfiguration;  // a wavefront per router row
    // counters and flags start at zero; the error word is cleared by the first launch of a call only,
    // so that a timeout in an earlier launch of the same call stays visible
    hipLaunchKernelGGL(stack_clear, dim3(1), dim3(256), 0, st, bar, clear_err ? dec_stack_bar_ints() : STACK_ERR);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    void* args[] = {&p};
    return hipLaunchCooperativeKernel(kern, dim3(G), dim3(512), args, (unsigned)lds, st);
}

}  // namespace moe
