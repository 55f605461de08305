// Decode path of the whole layer (T <= 32 tokens) in three launches.
//
// At decode a token touches only its k experts (FreeToken/dothoosh, "Architecture and the
// sparsity puzzle": 13B of 284B parameters per token), so the layer is a stream of a few
// experts' weight rows from HBM.  Everything that is not that stream is latency, so the three
// kernels are arranged to start the weight stream as early as possible and keep many 16-byte
// loads in flight per lane:
//
//   dec_route   one wavefront per router row computes the logits of every token; the last
//               workgroup to finish (ticket counter) selects the top-k, forms the gates, sorts
//               the pairs by expert and writes a compact slot table:
//                 slot s = (expert, first sorted position, pairs) for the experts that got
//                 tokens, ascending, then the shared expert; pos_tok / pos_gate per position.
//               With RMS-norm input (the residual stack) every workgroup normalises h itself.
//   dec_w13     gate/up rows of each slot's expert -> a = silu(g) * u (fp32), one wavefront
//               per (slot, R columns).
//   dec_w2c     down projection fused with the combine: a wavefront owns R output rows of
//               every token, issues the loads of a batch of SB experts' rows at once, and adds
//               the experts in ascending order (shared last) -- deterministic, no atomics.
#include "common.h"
#include "kernels.h"
#include "wchunk.h"

namespace moe {

__device__ __forceinline__ uint64_t dec_select_key(float v, int e) {
    uint32_t ord;
    if (v != v) {
        ord = 0u;
    } else {
        uint32_t u = (v == 0.0f) ? 0u : __float_as_uint(v);
        ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    }
    return ((uint64_t)ord << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)e);
}

// ------------------------------------------------------------------------------------------------
// dec_route
// ------------------------------------------------------------------------------------------------
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

struct DecRouteArgs {
    const void* x;         // [T, d] act dtype, or (prenorm) the fp32 residual stream h [T, d]
    const void* wr;        // [E, d] act dtype
    const float* b;        // [E] or NULL
    float* logits;         // [T, E]
    int32_t* topk_idx;     // [T, k]
    float* topk_w;         // [T, k]
    int32_t* idx_out;      // optional copy of topk_idx
    int32_t* counts;       // [E]
    int32_t* offsets;      // [E+1]
    int32_t* perm;         // [P]
    int32_t* inv;          // [P]
    int32_t* meta;         // meta[0] = slots (incl. shared)
    int4* slots;           // [E+1] (expert, pos0, npos, shared)
    int32_t* pos_tok;      // [P + T]
    float* pos_gate;       // [P + T]
    void* xn;              // prenorm: normalised x written here (act dtype) by the last workgroup
    unsigned* ticket;      // zero on entry; left zero on exit
    int T, d, E, k, n_shared, no_renorm, prenorm;
};

// Row of token t of the layer input, as fp32 values, for chunk i (V elements).
template <typename A>
__device__ __forceinline__ void load_x(const DecRouteArgs& p, int t, int i, float inv, float* v) {
    constexpr int V = rvec<A>::N;
    if (p.prenorm) {
        const float* h = reinterpret_cast<const float*>(p.x) + (int64_t)t * p.d + i;
#pragma unroll
        for (int q = 0; q < V; ++q) v[q] = bf16_to_f32(f32_to_bf16(h[q] * inv));  // the bf16 value K2 will see
        if (sizeof(A) == 4) {
#pragma unroll
            for (int q = 0; q < V; ++q) v[q] = h[q] * inv;
        }
    } else {
        rvec<A>::load(reinterpret_cast<const A*>(p.x) + (int64_t)t * p.d + i, v);
    }
}

template <typename A>
__global__ void __launch_bounds__(512) dec_route(DecRouteArgs p) {
    constexpr int V = rvec<A>::N;
    constexpr int NW = 8;  // wavefronts per workgroup
    __shared__ float s_inv[32];
    __shared__ int s_cnt[MOE_MAX_E];
    __shared__ int s_cur[MOE_MAX_E];
    __shared__ int s_last;
    const int lane = lane_id(), wv = wave_id();
    const int T = p.T, E = p.E, k = p.k, d = p.d;

    // RMS normalisation factors of the residual stream (stack input), one per token.
    if (p.prenorm) {
        for (int t = wv; t < T; t += NW) {
            const float* h = reinterpret_cast<const float*>(p.x) + (int64_t)t * d;
            float ss = 0.0f;
            for (int i = lane; i < d; i += MOE_WAVE) ss = fmaf(h[i], h[i], ss);
            ss = wave_sum(ss);
            if (lane == 0) s_inv[t] = 1.0f / sqrtf(ss / (float)d + 1e-6f);
        }
        __syncthreads();
    }

    // Logits: wavefront per router row.
    const int e = blockIdx.x * NW + wv;
    if (e < E) {
        const A* w = reinterpret_cast<const A*>(p.wr) + (int64_t)e * d;
        const float bias = p.b ? p.b[e] : 0.0f;
        for (int t0 = 0; t0 < T; t0 += 8) {
            float acc[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) acc[q] = 0.0f;
            for (int i = lane * V; i < d; i += MOE_WAVE * V) {
                float wvv[V];
                rvec<A>::load(w + i, wvv);
#pragma unroll
                for (int q = 0; q < 8; ++q) {
                    if (t0 + q < T) {
                        float xv[V];
                        load_x<A>(p, t0 + q, i, p.prenorm ? s_inv[t0 + q] : 1.0f, xv);
#pragma unroll
                        for (int v = 0; v < V; ++v) acc[q] = fmaf(wvv[v], xv[v], acc[q]);
                    }
                }
            }
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const float s = wave_sum(acc[q]);
                if (lane == 0 && t0 + q < T) p.logits[(int64_t)(t0 + q) * E + e] = s + bias;
            }
        }
    }

    // Ticket: the last workgroup continues with selection and grouping.
    __threadfence();
    __syncthreads();
    if (threadIdx.x == 0) {
        const unsigned t = atomicAdd(p.ticket, 1u);
        s_last = (t == gridDim.x - 1) ? 1 : 0;
    }
    __syncthreads();
    if (!s_last) return;
    __threadfence();

    // Normalised input for the FFN kernels (stack).
    if (p.prenorm) {
        for (int t = 0; t < T; ++t)
            for (int i = threadIdx.x; i < d; i += blockDim.x) {
                const float v = reinterpret_cast<const float*>(p.x)[(int64_t)t * d + i] * s_inv[t];
                io<A>::st(reinterpret_cast<A*>(p.xn), (int64_t)t * d + i, v);
            }
    }

    // Top-k + gates: wavefront per token.
    for (int t = wv; t < T; t += NW) {
        const volatile float* l = p.logits + (int64_t)t * E;
        uint64_t key[MOE_MAX_E / MOE_WAVE];
        const int epl = (E + MOE_WAVE - 1) / MOE_WAVE;
#pragma unroll
        for (int j = 0; j < MOE_MAX_E / MOE_WAVE; ++j) {
            const int ee = lane + MOE_WAVE * j;
            key[j] = (j < epl && ee < E) ? dec_select_key(l[ee], ee) : 0ull;
        }
        int my_sel = 0;
        for (int r = 0; r < k; ++r) {
            uint64_t best = 0ull;
#pragma unroll
            for (int j = 0; j < MOE_MAX_E / MOE_WAVE; ++j) best = key[j] > best ? key[j] : best;
            best = wave_max_u64(best);
            const int ee = (int)(0xFFFFFFFFu - (uint32_t)best);
#pragma unroll
            for (int j = 0; j < MOE_MAX_E / MOE_WAVE; ++j)
                if (lane + MOE_WAVE * j == ee) key[j] = 0ull;
            if (lane == r) my_sel = ee;
        }
        const float m = l[__shfl(my_sel, 0, MOE_WAVE)];
        const float term = (lane < k) ? expf(l[my_sel] - m) : 0.0f;
        float den;
        if (p.no_renorm) {
            float part = 0.0f;
            for (int ee = lane; ee < E; ee += MOE_WAVE) part += expf(l[ee] - m);
            den = wave_sum(part);
        } else {
            den = wave_sum(term);
        }
        if (lane < k) {
            p.topk_idx[(int64_t)t * k + lane] = my_sel;
            p.topk_w[(int64_t)t * k + lane] = term / den;
            if (p.idx_out) p.idx_out[(int64_t)t * k + lane] = my_sel;
        }
    }
    __syncthreads();

    // Counting sort of the T*k pairs (wave 0 scatters stably), slot table.
    const int P = T * k;
    for (int ee = threadIdx.x; ee < E; ee += blockDim.x) s_cnt[ee] = 0;
    __syncthreads();
    for (int q = threadIdx.x; q < P; q += blockDim.x) atomicAdd(&s_cnt[p.topk_idx[q]], 1);
    __syncthreads();
    if (wv == 0) {
        // exclusive scan over experts, active list
        const int per = (E + MOE_WAVE - 1) / MOE_WAVE;
        const int lo = min(lane * per, E), hi = min(lo + per, E);
        int sc = 0, sa = 0;
        for (int ee = lo; ee < hi; ++ee) {
            sc += s_cnt[ee];
            sa += s_cnt[ee] > 0;
        }
        int ic = sc, ia = sa;
#pragma unroll
        for (int o = 1; o < MOE_WAVE; o <<= 1) {
            const int u = __shfl_up(ic, o, MOE_WAVE), w = __shfl_up(ia, o, MOE_WAVE);
            if (lane >= o) { ic += u; ia += w; }
        }
        int pc = ic - sc, pa = ia - sa;
        for (int ee = lo; ee < hi; ++ee) {
            const int c = s_cnt[ee];
            p.counts[ee] = c;
            p.offsets[ee] = pc;
            s_cur[ee] = pc;
            if (c > 0) p.slots[pa++] = make_int4(ee, pc, c, 0);
            pc += c;
        }
        if (lane == MOE_WAVE - 1) {
            p.offsets[E] = pc;
            if (p.n_shared) p.slots[pa] = make_int4(E, P, T, 1);
            p.meta[0] = pa + p.n_shared;
        }
        // stable scatter (ballot per expert-id bit)
        int nbits = 0;
        while ((1 << nbits) < E) ++nbits;
        const uint64_t lt = lanemask_lt();
        for (int c0 = 0; c0 < P; c0 += MOE_WAVE) {
            const int q = c0 + lane;
            const bool valid = q < P;
            const int ee = valid ? p.topk_idx[q] : 0;
            uint64_t msk = __ballot(valid);
            for (int bb = 0; bb < nbits; ++bb) {
                const bool bit = (ee >> bb) & 1;
                const uint64_t bl = __ballot(valid && bit);
                msk &= bit ? bl : ~bl;
            }
            if (valid) {
                const int base = s_cur[ee];
                const int pos = base + __popcll(msk & lt);
                p.perm[pos] = q;
                p.inv[q] = pos;
                p.pos_tok[pos] = q / k;
                p.pos_gate[pos] = p.topk_w[q];
                if ((msk >> lane) == 1ull) s_cur[ee] = base + __popcll(msk);
            }
        }
        if (p.n_shared)
            for (int t = lane; t < T; t += MOE_WAVE) {
                p.pos_tok[P + t] = t;
                p.pos_gate[P + t] = 1.0f;
            }
    }
    if (threadIdx.x == 0) *p.ticket = 0u;  // ready for the next call
}

// ------------------------------------------------------------------------------------------------
// dec_w13: a[pos, j] = silu(Wg[j] . x) * (Wu[j] . x) for every position of every slot
// ------------------------------------------------------------------------------------------------
struct DecFfnArgs {
    const void* x;          // [T, d] act dtype
    const int32_t* meta;
    const int4* slots;
    const int32_t* pos_tok;
    const float* pos_gate;
    const uint8_t* w13; const uint8_t* w13s;   // routed gate/up
    const uint8_t* s13; const uint8_t* s13s;   // shared gate/up
    const uint8_t* w2; const uint8_t* w2s;     // routed down
    const uint8_t* s2; const uint8_t* s2s;     // shared down
    float* a;               // [P + T, fmax]
    void* out;              // [T, d] (f32 or bf16)
    int T, d, f, fs, fmax, k, accumulate;
};

template <int WT> struct DecAct { using T = uint16_t; };
template <> struct DecAct<0> { using T = float; };

template <int WT, int R, int U>
__global__ void __launch_bounds__(256) dec_w13(DecFfnArgs p) {
    using W = WChunk<WT>;
    using A = typename DecAct<WT>::T;
    constexpr int EC = W::EC;
    const int lane = lane_id();
    const int n_slots = p.meta[0];
    const int T = p.T;
    const int ngr = (p.f + R - 1) / R, ngs = (p.fs + R - 1) / R;
    const int wave_global = blockIdx.x * 4 + wave_id();
    const int n_waves = gridDim.x * 4;
    // items: routed slots first (ngr each), the shared slot last (ngs)
    const int4 last = n_slots > 0 ? p.slots[n_slots - 1] : make_int4(0, 0, 0, 0);
    const int n_routed = (n_slots > 0 && last.w) ? n_slots - 1 : n_slots;
    const int r_items = n_routed * ngr;
    const int n_items = r_items + (n_slots > n_routed ? ngs : 0);
    const int NC = p.d / EC;
    const int64_t rb = row_bytes(WT, p.d), sb = p.d / 32;
    for (int item = wave_global; item < n_items; item += n_waves) {
        // routed slots first (ngr items each), then the shared slot (ngs items)
        const int s = item < r_items ? item / ngr : n_routed;
        const int jg = item < r_items ? item % ngr : item - r_items;
        const int4 S = p.slots[s];
        const bool sh = S.w != 0;
        const int fc = sh ? p.fs : p.f;
        const int j0 = jg * R;
        const uint8_t* wb = sh ? p.s13 : p.w13 + (int64_t)S.x * 2 * p.f * rb;
        const uint8_t* sbp = (WT == 2) ? (sh ? p.s13s : p.w13s + (int64_t)S.x * 2 * p.f * sb) : nullptr;
        // One K step covers the row when NC <= 64*U (the configured shapes); otherwise every
        // pair re-streams the rows step by step (L1/L2 hits after the first pair).
        const int nsteps = (NC + MOE_WAVE * U - 1) / (MOE_WAVE * U);
        const int npass = nsteps == 1 ? 1 : S.z;
        for (int ps = 0; ps < npass; ++ps) {
            const int q_lo = nsteps == 1 ? 0 : ps, q_hi = nsteps == 1 ? S.z : ps + 1;
            float ag[R][4], au[R][4];  // up to 4 pairs accumulated across K steps (slow path: 1)
#pragma unroll
            for (int r = 0; r < R; ++r)
#pragma unroll
                for (int q = 0; q < 4; ++q) ag[r][q] = au[r][q] = 0.0f;
            for (int qb = q_lo; qb < q_hi; qb += 4) {
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
                    for (int q = 0; q < 4; ++q) {
                        if (qb + q >= q_hi) break;
                        const int t = p.pos_tok[S.y + qb + q];
                        const A* xr = reinterpret_cast<const A*>(p.x) + (int64_t)t * p.d;
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
                for (int q = 0; q < 4; ++q) {
                    if (qb + q >= q_hi) break;
                    const int pos = S.y + qb + q;
#pragma unroll
                    for (int r = 0; r < R; ++r) {
                        const float g = wave_sum(ag[r][q]), u = wave_sum(au[r][q]);
                        ag[r][q] = au[r][q] = 0.0f;
                        const int j = j0 + r;
                        if (lane == 0 && j < fc) p.a[(int64_t)pos * p.fmax + j] = g / (1.0f + expf(-g)) * u;
                    }
                }
            }
        }
    }
}

// ------------------------------------------------------------------------------------------------
// dec_w2c: out[t, i] = sum_slots g * (W2_e[i] . a[pos]) (+ out), slots in ascending expert order
// ------------------------------------------------------------------------------------------------
template <int WT, int R, int U, int SB, bool OUT_BF16>
__global__ void __launch_bounds__(256) dec_w2c(DecFfnArgs p) {
    using W = WChunk<WT>;
    constexpr int EC = W::EC;
    const int lane = lane_id();
    const int n_slots = p.meta[0];
    const int n_items = (p.d + R - 1) / R;
    const int wave_global = blockIdx.x * 4 + wave_id();
    const int n_waves = gridDim.x * 4;
    for (int item = wave_global; item < n_items; item += n_waves) {
        const int i0 = item * R;
        float o[R];
#pragma unroll
        for (int r = 0; r < R; ++r) o[r] = 0.0f;
        const int NCmax = (p.fs > p.f ? p.fs : p.f) / EC;
        for (int s0 = 0; s0 < n_slots; s0 += SB) {
            int4 S[SB];
#pragma unroll
            for (int sb = 0; sb < SB; ++sb) S[sb] = (s0 + sb < n_slots) ? p.slots[s0 + sb] : make_int4(0, 0, 0, -1);
            // K steps (one for the configured shapes); each adds g * partial dot to o
            for (int c0 = 0; c0 < NCmax; c0 += MOE_WAVE * U) {
                // every row of the batch: issue all loads first
                W w[SB][R][U];
#pragma unroll
                for (int sb = 0; sb < SB; ++sb) {
                    const bool live = S[sb].w >= 0;
                    const bool sh = S[sb].w == 1;
                    const int fc = sh ? p.fs : p.f;
                    const int NC = fc / EC;
                    const int64_t rb = row_bytes(WT, fc), sbb = fc / 32;
                    const uint8_t* base = sh ? p.s2 : p.w2 + (int64_t)S[sb].x * p.d * rb;
                    const uint8_t* sbase = (WT == 2) ? (sh ? p.s2s : p.w2s + (int64_t)S[sb].x * p.d * sbb) : nullptr;
#pragma unroll
                    for (int r = 0; r < R; ++r)
#pragma unroll
                        for (int u = 0; u < U; ++u) {
                            const int i = i0 + r, c = c0 + lane + MOE_WAVE * u;
                            if (live && i < p.d && c < NC)
                                w[sb][r][u].load(base + (int64_t)i * rb, sbase ? sbase + (int64_t)i * sbb : nullptr, c);
                            else
                                w[sb][r][u].zero();
                        }
                }
#pragma unroll
                for (int sb = 0; sb < SB; ++sb) {
                    if (S[sb].w < 0) continue;
                    const bool sh = S[sb].w == 1;
                    const int fc = sh ? p.fs : p.f;
                    const int NC = fc / EC;
                    for (int q = 0; q < S[sb].z; ++q) {
                        const int pos = S[sb].y + q;
                        const int t = p.pos_tok[pos];
                        const float g = p.pos_gate[pos];
                        const float* ar = p.a + (int64_t)pos * p.fmax;
                        float acc[R];
#pragma unroll
                        for (int r = 0; r < R; ++r) acc[r] = 0.0f;
#pragma unroll
                        for (int u = 0; u < U; ++u) {
                            const int c = c0 + lane + MOE_WAVE * u;
                            if (c < NC) {
#pragma unroll
                                for (int r = 0; r < R; ++r) acc[r] = w[sb][r][u].dot_f32(ar + (int64_t)c * EC, acc[r]);
                            }
                        }
#pragma unroll
                        for (int r = 0; r < R; ++r) {
                            const float y = wave_sum(acc[r]);
                            if (lane == t) o[r] = fmaf(g, y, o[r]);
                        }
                    }
                }
            }
        }
        if (lane < p.T) {
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const int i = i0 + r;
                if (i >= p.d) continue;
                const int64_t off = (int64_t)lane * p.d + i;
                if (OUT_BF16) {
                    uint16_t* out = reinterpret_cast<uint16_t*>(p.out);
                    const float prev = p.accumulate ? bf16_to_f32(out[off]) : 0.0f;
                    out[off] = f32_to_bf16(prev + o[r]);
                } else {
                    float* out = reinterpret_cast<float*>(p.out);
                    const float prev = p.accumulate ? out[off] : 0.0f;
                    out[off] = prev + o[r];
                }
            }
        }
    }
}

// ------------------------------------------------------------------------------------------------
// Host side
// ------------------------------------------------------------------------------------------------
hipError_t launch_dec_route(int act_dtype, const void* x, const void* wr, const float* b, float* logits,
                            int32_t* topk_idx, float* topk_w, int32_t* idx_out, int32_t* counts, int32_t* offsets,
                            int32_t* perm, int32_t* inv, int32_t* meta, int4* slots, int32_t* pos_tok,
                            float* pos_gate, void* xn, unsigned* ticket, int T, int d, int E, int k, int n_shared,
                            bool no_renorm, bool prenorm, hipStream_t st) {
    DecRouteArgs p{x, wr, b, logits, topk_idx, topk_w, idx_out, counts, offsets, perm, inv, meta, slots, pos_tok,
                   pos_gate, xn, ticket, T, d, E, k, n_shared, no_renorm ? 1 : 0, prenorm ? 1 : 0};
    const dim3 grid((E + 7) / 8), block(512);
    if (act_dtype == 0) hipLaunchKernelGGL((dec_route<float>), grid, block, 0, st, p);
    else hipLaunchKernelGGL((dec_route<uint16_t>), grid, block, 0, st, p);
    return hipGetLastError();
}

static unsigned dec_grid(int64_t max_items) {
    int64_t waves = max_items < 256 * 16 ? max_items : 256 * 16;
    int64_t blocks = (waves + 3) / 4;
    return (unsigned)(blocks < 1 ? 1 : blocks);
}

hipError_t launch_dec_ffn(int wt, bool out_bf16, const void* x, const int32_t* meta, const int4* slots,
                          const int32_t* pos_tok, const float* pos_gate, const void* w13, const uint8_t* w13s,
                          const void* s13, const uint8_t* s13s, const void* w2, const uint8_t* w2s, const void* s2,
                          const uint8_t* s2s, float* a, void* out, int T, int d, int f, int fs, int k, int E,
                          int n_shared, bool accumulate, hipStream_t st, hipEvent_t ev_up_done,
                          hipEvent_t ev_down_start) {
    const int fmax = (n_shared && fs > f) ? fs : f;
    DecFfnArgs p{x, meta, slots, pos_tok, pos_gate, (const uint8_t*)w13, w13s, (const uint8_t*)s13, s13s,
                 (const uint8_t*)w2, w2s, (const uint8_t*)s2, s2s, a, out, T, d, f, n_shared ? fs : 0, fmax, k,
                 accumulate ? 1 : 0};
    const int64_t max_slots = (int64_t)(T * k < E ? T * k : E);
    // gate/up
    if (wt == 0) {
        constexpr int R = 2;
        const int64_t items = max_slots * ((f + R - 1) / R) + (n_shared ? (fs + R - 1) / R : 0);
        hipLaunchKernelGGL((dec_w13<0, R, 1>), dim3(dec_grid(items)), dim3(256), 0, st, p);
    } else if (wt == 1) {
        constexpr int R = 2;
        const int64_t items = max_slots * ((f + R - 1) / R) + (n_shared ? (fs + R - 1) / R : 0);
        hipLaunchKernelGGL((dec_w13<1, R, 4>), dim3(dec_grid(items)), dim3(256), 0, st, p);
    } else {
        constexpr int R = 4;
        const int64_t items = max_slots * ((f + R - 1) / R) + (n_shared ? (fs + R - 1) / R : 0);
        hipLaunchKernelGGL((dec_w13<2, R, 2>), dim3(dec_grid(items)), dim3(256), 0, st, p);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (ev_up_done && (e = hipEventRecord(ev_up_done, st)) != hipSuccess) return e;
    if (ev_down_start && (e = hipEventRecord(ev_down_start, st)) != hipSuccess) return e;
    // down + combine
#define MOE_DW2(WTV, RV, UV, SBV)                                                                                    \
    do {                                                                                                             \
        const int64_t items = (d + RV - 1) / RV;                                                                     \
        if (out_bf16) hipLaunchKernelGGL((dec_w2c<WTV, RV, UV, SBV, true>), dim3(dec_grid(items)), dim3(256), 0, st, p); \
        else hipLaunchKernelGGL((dec_w2c<WTV, RV, UV, SBV, false>), dim3(dec_grid(items)), dim3(256), 0, st, p);       \
    } while (0)
    if (wt == 0) MOE_DW2(0, 1, 1, 8);
    else if (wt == 1) MOE_DW2(1, 1, 2, 8);
    else MOE_DW2(2, 2, 1, 8);
#undef MOE_DW2
    return hipGetLastError();
}

}  // namespace moe
