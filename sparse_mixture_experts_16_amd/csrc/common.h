// Device helpers shared by the gfx950 kernels of the MoE layer.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#define MOE_WAVE 64

namespace moe {

// ----------------------------------------------------------------------------------------------
// Number formats
// ----------------------------------------------------------------------------------------------
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// fp32 -> bf16, round to nearest even; NaN stays a quiet NaN (its top payload bits kept).  One
// v_cvt_pk_bf16_f32 on gfx950, checked on the GPU against the bit-level rounding over all 2^32
// inputs (identical, NaN payloads included); the branchy bit-level form cost the GEMM epilogues
// an exec-mask round trip per element.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

// silu(g) = g / (1 + e^-g) on the hardware exp2 and reciprocal (about 2 ulp; infinities and
// NaN propagate as in the exact form).
__device__ __forceinline__ float silu_hw(float g) {
    return g * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-g * 1.4426950408889634f));
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return (uint32_t)f32_to_bf16(lo) | ((uint32_t)f32_to_bf16(hi) << 16);
}

template <typename T> struct io;
template <> struct io<float> {
    __device__ __forceinline__ static float ld(const float* p, int64_t i) { return p[i]; }
    __device__ __forceinline__ static void st(float* p, int64_t i, float v) { p[i] = v; }
};
template <> struct io<uint16_t> {
    __device__ __forceinline__ static float ld(const uint16_t* p, int64_t i) { return bf16_to_f32(p[i]); }
    __device__ __forceinline__ static void st(uint16_t* p, int64_t i, float v) { p[i] = f32_to_bf16(v); }
};

// ----------------------------------------------------------------------------------------------
// Wave-level reductions (64 lanes)
// ----------------------------------------------------------------------------------------------
// Cross-lane steps on the DPP path (no LDS crossbar).  A lane whose row is masked off, or
// whose source lane lies outside its row, takes `old`.
//   0xB1 quad_perm [1,0,3,2]   0x4E quad_perm [2,3,0,1]   0x141 row_half_mirror
//   0x140 row_mirror           0x111.. row_shr:n          0x142 row_bcast:15   0x143 row_bcast:31
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ uint32_t dpp(uint32_t old, uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp((int)old, (int)v, CTRL, ROW_MASK, 0xF, false);
}
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ float dppf(float v) {  // 0.0 where masked off
    return __uint_as_float(dpp<CTRL, ROW_MASK>(0u, __float_as_uint(v)));
}
__device__ __forceinline__ float readlane_f(float v, int l) {
    return __uint_as_float((uint32_t)__builtin_amdgcn_readlane((int)__float_as_uint(v), l));
}

// Sum over the 64 lanes, returned to every lane: quads, halves of rows and rows by DPP
// permutes, then rows 0..3 folded into lane 63 by the two row broadcasts.
__device__ __forceinline__ float wave_sum(float v) {
    v += dppf<0xB1>(v);
    v += dppf<0x4E>(v);
    v += dppf<0x141>(v);
    v += dppf<0x140>(v);
    v += dppf<0x142, 0xA>(v);
    v += dppf<0x143, 0xC>(v);
    return readlane_f(v, 63);
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    uint32_t w;
    w = dpp<0xB1>(0u, v); v = w > v ? w : v;
    w = dpp<0x4E>(0u, v); v = w > v ? w : v;
    w = dpp<0x141>(0u, v); v = w > v ? w : v;
    w = dpp<0x140>(0u, v); v = w > v ? w : v;
    w = dpp<0x142, 0xA>(0u, v); v = w > v ? w : v;
    w = dpp<0x143, 0xC>(0u, v); v = w > v ? w : v;
    return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}
// Inclusive prefix sum over the 64 lanes: shifts within each row of 16, then each row adds the
// totals of the rows before it through the row broadcasts.
__device__ __forceinline__ int wave_incl_scan(int v) {
    uint32_t u = (uint32_t)v;
    u += dpp<0x111>(0u, u);
    u += dpp<0x112>(0u, u);
    u += dpp<0x114>(0u, u);
    u += dpp<0x118>(0u, u);
    u += dpp<0x142, 0xA>(0u, u);
    u += dpp<0x143, 0xC>(0u, u);
    return (int)u;
}
// Exclusive prefix of per-group tile counts into s_pref[0..G] (s_pref[G] = the total), by one
// wavefront: lane l takes groups l*per .. l*per+per-1 (per <= TPL), issues all of their count
// loads at once, and a single wave scan joins the lanes.
template <int TPL, typename F>
__device__ __forceinline__ void wave_tile_prefix(int G, int* s_pref, F&& tiles_of) {
    const int lane = threadIdx.x & 63;
    const int per = (G + 63) / 64;
    const int lo = min(lane * per, G), hi = min(lo + per, G);
    int t[TPL];
    int sum = 0;
#pragma unroll
    for (int j = 0; j < TPL; ++j) {
        t[j] = (j < per && lo + j < hi) ? tiles_of(lo + j) : 0;
        sum += t[j];
    }
    const int incl = wave_incl_scan(sum);
    int run = incl - sum;
#pragma unroll
    for (int j = 0; j < TPL; ++j)
        if (j < per && lo + j < hi) {
            s_pref[lo + j] = run;
            run += t[j];
        }
    if (lane == 63) s_pref[G] = incl;
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        uint64_t w = __shfl_xor(v, o, MOE_WAVE);
        v = w > v ? w : v;
    }
    return v;
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & (MOE_WAVE - 1); }
// The wavefront's index in its workgroup, as a wave-uniform (scalar) value, so that loops and
// addresses derived from it stay on the scalar unit.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x / MOE_WAVE); }

// Lanes below this one in the wave.
__device__ __forceinline__ uint64_t lanemask_lt() {
    int l = lane_id();
    return l == 0 ? 0ull : (~0ull >> (64 - l));
}

// ----------------------------------------------------------------------------------------------
// Top-k selection inside one wavefront
// ----------------------------------------------------------------------------------------------
// Order-preserving 32-bit key of a logit: a larger logit gives a larger key, -0 and +0 are equal,
// NaN ranks below every number (key 1) and 0 marks an entry already taken or absent.
__device__ __forceinline__ uint32_t sel_ord(float v) {
    if (v != v) return 1u;
    const uint32_t u = (v == 0.0f) ? 0u : __float_as_uint(v);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// k rounds of arg-max over the wave's keys, lane l holding entries l*KPL .. l*KPL+KPL-1 (so a lower
// lane means a lower index).  Each round takes the largest key; among equal keys the lowest
// index, found as the lowest lane of a ballot and the first such entry inside that lane.  Lane
// r < k returns the index picked in round r (the others return 0).  Needs k <= the number of
// present entries.
template <int KPL>
__device__ __forceinline__ int wave_topk(uint32_t (&key)[KPL], int k) {
    const int lane = lane_id();
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
        if (lane == r) mine = wl * KPL + wj;
    }
    return mine;
}

}  // namespace moe
