// Decode path of the expert FFNs at small T (gate/up, down, combine): grouped GEMV that streams only the
// active experts' weight rows from HBM.
//
// At decode a token needs only its k experts (plus the shared one); the pages' whole point is
// that these few experts' bytes are what must move (dothoosh.com FreeToken article,
// "FreeToken architecture and the sparsity puzzle": 13B of 284B parameters per token; host vs
// GPU memory bandwidth in the same section).  The work is HBM-bound: every kernel here reads a
// weight row with 16-byte loads per lane, keeps it in registers, and reuses it for every token
// routed to that expert.
//
//   gemv_w13          a[pos, j]  = silu(Wg_e[j] . x_t) * (Wu_e[j] . x_t)        (fp32 a)
//   gemv_w2_combine   out[t, i]  = sum_e g_{t,e} (W2_e[i] . a[pos(t,e)]) + shared  (fused combine)
//   gemv_w2_sorted    y[pos, i]  = W2_e[i] . a[pos]                              (moe_grouped_ffn)
//
// The routed experts' pairs come from the permute: act_list lists the experts that received
// tokens in ascending order (meta[0] of them) and offsets[e]..offsets[e+1] are their sorted
// slots; the shared expert is an extra slot that sees every token.
#include "common.h"
#include "kernels.h"
#include "wchunk.h"

namespace moe {

struct GemvW13Args {
    const void* x;              // [T, d] act dtype
    const int32_t* perm;
    const int32_t* offsets;
    const int32_t* act_list;
    const int32_t* meta;        // meta[0] = number of active routed experts
    const uint8_t* w13;         // routed [E, 2f, d]
    const uint8_t* w13s;        // scales (MXFP4)
    const uint8_t* s13;         // shared [2fs, d] or NULL
    const uint8_t* s13s;
    float* a;                   // routed [P, f] then shared [T, fs]
    int T, d, f, fs, k, n_shared;
    float g_r, g_s;             // NVFP4 tensor scales of the routed / shared gate-up weights (1 otherwise)
};

template <int WT> struct ActOf { using T = uint16_t; };
template <> struct ActOf<0> { using T = float; };

template <int WT>
__device__ __forceinline__ float chunk_dot_act(const WChunk<WT>& w, const typename ActOf<WT>::T* x, float acc) {
    if constexpr (WT == 0) return w.dot_f32(x, acc);
    else return w.dot_bf16(x, acc);
}

// R output columns (gate row j and up row f+j each) per wavefront item, U chunks per lane per
// K step, PG tokens per pass over the rows.
template <int WT, int R, int U, int PG>
__global__ void __launch_bounds__(256) gemv_w13(GemvW13Args p) {
    using W = WChunk<WT>;
    using A = typename ActOf<WT>::T;
    constexpr int EC = W::EC;
    const int lane = lane_id();
    const int n_act = p.meta[0];
    const int ngr = (p.f + R - 1) / R;
    const int ngs = p.n_shared ? (p.fs + R - 1) / R : 0;
    const int n_items = n_act * ngr + ngs;
    const int NC = p.d / EC;  // chunks per row
    const int64_t rb = row_bytes(WT, p.d), sb = scale_row_bytes(WT, p.d);
    const int P = p.T * p.k;
    const int wave_global = blockIdx.x * (blockDim.x / MOE_WAVE) + wave_id();
    const int n_waves = gridDim.x * (blockDim.x / MOE_WAVE);

    for (int item = wave_global; item < n_items; item += n_waves) {
        const uint8_t* wbase;
        const uint8_t* sbase;
        int fcur, j0, pos0, npos;
        float* abase;
        bool routed = item < n_act * ngr;
        const float gsc = routed ? p.g_r : p.g_s;
        if (routed) {
            const int e = p.act_list[item / ngr];
            j0 = (item % ngr) * R;
            fcur = p.f;
            wbase = p.w13 + (int64_t)e * 2 * p.f * rb;
            sbase = p.w13s ? p.w13s + (int64_t)e * 2 * p.f * sb : nullptr;
            pos0 = p.offsets[e];
            npos = p.offsets[e + 1] - pos0;
            abase = p.a;
        } else {
            j0 = (item - n_act * ngr) * R;
            fcur = p.fs;
            wbase = p.s13;
            sbase = p.s13s;
            pos0 = 0;
            npos = p.T;
            abase = p.a + (int64_t)P * p.f;
        }
        for (int q0 = 0; q0 < npos; q0 += PG) {
            float ag[R][PG], au[R][PG];
            int tok[PG];
#pragma unroll
            for (int q = 0; q < PG; ++q) {
                const int pos = pos0 + q0 + q;
                tok[q] = (q0 + q < npos) ? (routed ? p.perm[pos] / p.k : pos) : -1;
#pragma unroll
                for (int r = 0; r < R; ++r) ag[r][q] = au[r][q] = 0.0f;
            }
            for (int c0 = 0; c0 < NC; c0 += MOE_WAVE * U) {
                W wg[R][U], wu[R][U];
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    const int j = j0 + r;
#pragma unroll
                    for (int u = 0; u < U; ++u) {
                        const int c = c0 + lane + MOE_WAVE * u;
                        if (j < fcur && c < NC) {
                            wg[r][u].load(wbase + (int64_t)j * rb, sbase ? sbase + (int64_t)j * sb : nullptr, c);
                            wu[r][u].load(wbase + (int64_t)(fcur + j) * rb, sbase ? sbase + (int64_t)(fcur + j) * sb : nullptr, c);
                        } else {
                            wg[r][u].zero();
                            wu[r][u].zero();
                        }
                    }
                }
#pragma unroll
                for (int q = 0; q < PG; ++q) {
                    if (tok[q] < 0) continue;
                    const A* xr = reinterpret_cast<const A*>(p.x) + (int64_t)tok[q] * p.d;
#pragma unroll
                    for (int u = 0; u < U; ++u) {
                        const int c = c0 + lane + MOE_WAVE * u;
                        if (c < NC) {
#pragma unroll
                            for (int r = 0; r < R; ++r) {
                                ag[r][q] = chunk_dot_act<WT>(wg[r][u], xr + (int64_t)c * EC, ag[r][q]);
                                au[r][q] = chunk_dot_act<WT>(wu[r][u], xr + (int64_t)c * EC, au[r][q]);
                            }
                        }
                    }
                }
            }
#pragma unroll
            for (int q = 0; q < PG; ++q) {
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    const float g = wave_sum(ag[r][q]) * gsc;
                    const float u = wave_sum(au[r][q]) * gsc;
                    const int j = j0 + r;
                    if (lane == 0 && tok[q] >= 0 && j < fcur) {
                        const int pos = pos0 + q0 + q;
                        abase[(int64_t)pos * fcur + j] = g / (1.0f + expf(-g)) * u;
                    }
                }
            }
        }
    }
}

struct GemvW2Args {
    const float* a;             // routed [P, f] then shared [T, fs]
    const int32_t* perm;
    const int32_t* offsets;
    const int32_t* act_list;
    const int32_t* meta;
    const float* topk_w;        // [T, k] gates (combine variant)
    const uint8_t* w2;          // routed [E, d, f]
    const uint8_t* w2s;
    const uint8_t* s2;          // shared [d, fs]
    const uint8_t* s2s;
    void* out;                  // combine: [T, d] (f32 or bf16); sorted: y [P, d] act dtype
    void* y_shared;             // sorted variant: [T, d] act dtype, or NULL
    int T, d, f, fs, k, n_shared;
    int accumulate;             // combine: out += result
    float g_r, g_s;             // NVFP4 tensor scales of the routed / shared down weights (1 otherwise)
};

template <int WT>
__device__ __forceinline__ void load_rows_w2(WChunk<WT>* w, int R, const uint8_t* base, const uint8_t* sbase,
                                             int64_t rb, int64_t sb, int i0, int d, int NC, int lane) {
    for (int r = 0; r < R; ++r) {
        const int i = i0 + r;
        const int c = lane;
        if (i < d && c < NC) w[r].load(base + (int64_t)i * rb, sbase ? sbase + (int64_t)i * sb : nullptr, c);
        else w[r].zero();
    }
}

// One wavefront item = R output rows of d for every token; loops over the active experts in
// ascending order, then the shared expert, so each out[t, i] is summed in the reference order.
// Requires T <= 64 (lane t holds token t's running sums).  OUT_BF16 selects the output type.
template <int WT, int R, int U, bool OUT_BF16>
__global__ void __launch_bounds__(256) gemv_w2_combine(GemvW2Args p) {
    using W = WChunk<WT>;
    constexpr int EC = W::EC;
    const int lane = lane_id();
    const int n_act = p.meta[0];
    const int n_items = (p.d + R - 1) / R;
    const int P = p.T * p.k;
    const int wave_global = blockIdx.x * (blockDim.x / MOE_WAVE) + wave_id();
    const int n_waves = gridDim.x * (blockDim.x / MOE_WAVE);
    const int n_slots = n_act + (p.n_shared ? 1 : 0);

    for (int item = wave_global; item < n_items; item += n_waves) {
        const int i0 = item * R;
        float o[R];
#pragma unroll
        for (int r = 0; r < R; ++r) o[r] = 0.0f;
        for (int sl = 0; sl < n_slots; ++sl) {
            const bool routed = sl < n_act;
            const int fcur = routed ? p.f : p.fs;
            const int NC = fcur / EC;
            const int64_t rb = row_bytes(WT, fcur), sb = scale_row_bytes(WT, fcur);
            const float gsc = routed ? p.g_r : p.g_s;
            const uint8_t* base;
            const uint8_t* sbase;
            int pos0, npos;
            const float* abase;
            if (routed) {
                const int e = p.act_list[sl];
                base = p.w2 + (int64_t)e * p.d * rb;
                sbase = p.w2s ? p.w2s + (int64_t)e * p.d * sb : nullptr;
                pos0 = p.offsets[e];
                npos = p.offsets[e + 1] - pos0;
                abase = p.a;
            } else {
                base = p.s2;
                sbase = p.s2s;
                pos0 = 0;
                npos = p.T;
                abase = p.a + (int64_t)P * p.f;
            }
            for (int c0 = 0; c0 < NC; c0 += MOE_WAVE * U) {
                W w[R][U];
#pragma unroll
                for (int r = 0; r < R; ++r)
#pragma unroll
                    for (int u = 0; u < U; ++u) {
                        const int i = i0 + r, c = c0 + lane + MOE_WAVE * u;
                        if (i < p.d && c < NC) w[r][u].load(base + (int64_t)i * rb, sbase ? sbase + (int64_t)i * sb : nullptr, c);
                        else w[r][u].zero();
                    }
                // Partial dot products of this K step, one per (row, pair); pairs handled one by one.
                for (int q = 0; q < npos; ++q) {
                    const int pos = pos0 + q;
                    const float* ar = abase + (int64_t)pos * fcur;
                    float acc[R];
#pragma unroll
                    for (int r = 0; r < R; ++r) acc[r] = 0.0f;
#pragma unroll
                    for (int u = 0; u < U; ++u) {
                        const int c = c0 + lane + MOE_WAVE * u;
                        if (c < NC) {
#pragma unroll
                            for (int r = 0; r < R; ++r) acc[r] = w[r][u].dot_f32(ar + (int64_t)c * EC, acc[r]);
                        }
                    }
                    const int pr = routed ? p.perm[pos] : pos;
                    const int t = routed ? pr / p.k : pos;
                    const float g = routed ? p.topk_w[pr] : 1.0f;
#pragma unroll
                    for (int r = 0; r < R; ++r) {
                        const float y = wave_sum(acc[r]) * gsc;
                        // Multi-step K (f > 64*U*EC) accumulates g*partial; exact order differs
                        // only in fp32 rounding.
                        if (lane == t) o[r] = fmaf(g, y, o[r]);
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

// y[pos, i] = W2_e[i] . a[pos] for every sorted slot; one item = (slot, R rows).
template <int WT, int R, int U, bool Y_BF16>
__global__ void __launch_bounds__(256) gemv_w2_sorted(GemvW2Args p) {
    using W = WChunk<WT>;
    constexpr int EC = W::EC;
    const int lane = lane_id();
    const int n_act = p.meta[0];
    const int ngr = (p.d + R - 1) / R;
    const int n_slots = n_act + (p.n_shared ? 1 : 0);
    const int n_items = n_slots * ngr;
    const int P = p.T * p.k;
    const int wave_global = blockIdx.x * (blockDim.x / MOE_WAVE) + wave_id();
    const int n_waves = gridDim.x * (blockDim.x / MOE_WAVE);

    for (int item = wave_global; item < n_items; item += n_waves) {
        const int sl = item / ngr;
        const int i0 = (item % ngr) * R;
        const bool routed = sl < n_act;
        const int fcur = routed ? p.f : p.fs;
        const int NC = fcur / EC;
        const int64_t rb = row_bytes(WT, fcur), sb = scale_row_bytes(WT, fcur);
        const float gsc = routed ? p.g_r : p.g_s;
        const uint8_t* base;
        const uint8_t* sbase;
        int pos0, npos;
        const float* abase;
        void* ybase;
        if (routed) {
            const int e = p.act_list[sl];
            base = p.w2 + (int64_t)e * p.d * rb;
            sbase = p.w2s ? p.w2s + (int64_t)e * p.d * sb : nullptr;
            pos0 = p.offsets[e];
            npos = p.offsets[e + 1] - pos0;
            abase = p.a;
            ybase = p.out;
        } else {
            base = p.s2;
            sbase = p.s2s;
            pos0 = 0;
            npos = p.T;
            abase = p.a + (int64_t)P * p.f;
            ybase = p.y_shared;
        }
        for (int q = 0; q < npos; ++q) {
            const int pos = pos0 + q;
            const float* ar = abase + (int64_t)pos * fcur;
            float acc[R];
#pragma unroll
            for (int r = 0; r < R; ++r) acc[r] = 0.0f;
            for (int c0 = 0; c0 < NC; c0 += MOE_WAVE * U) {
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int c = c0 + lane + MOE_WAVE * u;
                    if (c >= NC) continue;
#pragma unroll
                    for (int r = 0; r < R; ++r) {
                        const int i = i0 + r;
                        if (i >= p.d) continue;
                        W w;
                        w.load(base + (int64_t)i * rb, sbase ? sbase + (int64_t)i * sb : nullptr, c);
                        acc[r] = w.dot_f32(ar + (int64_t)c * EC, acc[r]);
                    }
                }
            }
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const float y = wave_sum(acc[r]) * gsc;
                const int i = i0 + r;
                if (lane == 0 && i < p.d && ybase) {
                    const int64_t off = (int64_t)pos * p.d + i;
                    if (Y_BF16) reinterpret_cast<uint16_t*>(ybase)[off] = f32_to_bf16(y);
                    else reinterpret_cast<float*>(ybase)[off] = y;
                }
            }
        }
    }
}

// ------------------------------------------------------------------------------------------------
// Host launchers
// ------------------------------------------------------------------------------------------------
static int gemv_grid(int64_t max_items, int waves_per_block) {
    // Enough wavefronts to cover every CU several times over; items beyond loop.
    int64_t waves = max_items < 256 * 16 ? max_items : 256 * 16;
    int64_t blocks = (waves + waves_per_block - 1) / waves_per_block;
    return (int)(blocks < 1 ? 1 : blocks);
}

hipError_t launch_gemv_w13(int wt, const void* x, const int32_t* perm, const int32_t* offsets,
                           const int32_t* act_list, const int32_t* meta, const void* w13, const uint8_t* w13s,
                           const void* s13, const uint8_t* s13s, float* a, int T, int d, int f, int fs, int k,
                           int E, int n_shared, float g_r, float g_s, hipStream_t st) {
    GemvW13Args p{x, perm, offsets, act_list, meta, (const uint8_t*)w13, w13s, (const uint8_t*)s13, s13s,
                  a, T, d, f, fs, k, n_shared, g_r, g_s};
    const int64_t max_act = (int64_t)(T * k < E ? T * k : E);
    if (wt == 0) {
        constexpr int R = 1;
        int64_t items = max_act * ((f + R - 1) / R) + (n_shared ? (fs + R - 1) / R : 0);
        MOE_LAUNCH(PROF_FFN_UP, (gemv_w13<0, R, 4, 4>), dim3(gemv_grid(items, 4)), dim3(256), 0, st, p);
    } else if (wt == 1) {
        constexpr int R = 1;
        int64_t items = max_act * ((f + R - 1) / R) + (n_shared ? (fs + R - 1) / R : 0);
        MOE_LAUNCH(PROF_FFN_UP, (gemv_w13<1, R, 4, 4>), dim3(gemv_grid(items, 4)), dim3(256), 0, st, p);
    } else if (wt == 2) {
        constexpr int R = 2;
        int64_t items = max_act * ((f + R - 1) / R) + (n_shared ? (fs + R - 1) / R : 0);
        MOE_LAUNCH(PROF_FFN_UP, (gemv_w13<2, R, 2, 4>), dim3(gemv_grid(items, 4)), dim3(256), 0, st, p);
    } else {
        constexpr int R = 2;
        int64_t items = max_act * ((f + R - 1) / R) + (n_shared ? (fs + R - 1) / R : 0);
        MOE_LAUNCH(PROF_FFN_UP, (gemv_w13<3, R, 2, 4>), dim3(gemv_grid(items, 4)), dim3(256), 0, st, p);
    }
    return hipGetLastError();
}

hipError_t launch_gemv_w2_combine(int wt, bool out_bf16, const float* a, const int32_t* perm, const int32_t* offsets,
                                  const int32_t* act_list, const int32_t* meta, const float* topk_w, const void* w2,
                                  const uint8_t* w2s, const void* s2, const uint8_t* s2s, void* out, int T, int d,
                                  int f, int fs, int k, int n_shared, bool accumulate, float g_r, float g_s,
                                  hipStream_t st) {
    GemvW2Args p{a, perm, offsets, act_list, meta, topk_w, (const uint8_t*)w2, w2s, (const uint8_t*)s2, s2s,
                 out, nullptr, T, d, f, fs, k, n_shared, accumulate ? 1 : 0, g_r, g_s};
#define MOE_W2C(WTV, RV, UV)                                                                              \
    do {                                                                                                  \
        int64_t items = (d + RV - 1) / RV;                                                                \
        if (out_bf16)                                                                                     \
            MOE_LAUNCH(PROF_FFN_DOWN, (gemv_w2_combine<WTV, RV, UV, true>), dim3(gemv_grid(items, 4)), dim3(256), 0, st, p); \
        else                                                                                              \
            MOE_LAUNCH(PROF_FFN_DOWN, (gemv_w2_combine<WTV, RV, UV, false>), dim3(gemv_grid(items, 4)), dim3(256), 0, st, p); \
    } while (0)
    if (wt == 0) MOE_W2C(0, 1, 2);
    else if (wt == 1) MOE_W2C(1, 2, 2);
    else if (wt == 2) MOE_W2C(2, 4, 1);
    else MOE_W2C(3, 4, 1);
#undef MOE_W2C
    return hipGetLastError();
}

hipError_t launch_gemv_w2_sorted(int wt, bool y_bf16, const float* a, const int32_t* perm, const int32_t* offsets,
                                 const int32_t* act_list, const int32_t* meta, const void* w2, const uint8_t* w2s,
                                 const void* s2, const uint8_t* s2s, void* y, void* y_shared, int T, int d, int f,
                                 int fs, int k, int E, int n_shared, float g_r, float g_s, hipStream_t st) {
    GemvW2Args p{a, perm, offsets, act_list, meta, nullptr, (const uint8_t*)w2, w2s, (const uint8_t*)s2, s2s,
                 y, y_shared, T, d, f, fs, k, n_shared, 0, g_r, g_s};
    const int64_t max_act = (int64_t)(T * k < E ? T * k : E) + (n_shared ? 1 : 0);
#define MOE_W2S(WTV, RV, UV)                                                                              \
    do {                                                                                                  \
        int64_t items = max_act * ((d + RV - 1) / RV);                                                    \
        if (y_bf16)                                                                                       \
            MOE_LAUNCH(PROF_FFN_DOWN, (gemv_w2_sorted<WTV, RV, UV, true>), dim3(gemv_grid(items, 4)), dim3(256), 0, st, p); \
        else                                                                                              \
            MOE_LAUNCH(PROF_FFN_DOWN, (gemv_w2_sorted<WTV, RV, UV, false>), dim3(gemv_grid(items, 4)), dim3(256), 0, st, p); \
    } while (0)
    if (wt == 0) MOE_W2S(0, 1, 2);
    else if (wt == 1) MOE_W2S(1, 2, 2);
    else if (wt == 2) MOE_W2S(2, 4, 1);
    else MOE_W2S(3, 4, 1);
#undef MOE_W2S
    return hipGetLastError();
}

}  // namespace moe
