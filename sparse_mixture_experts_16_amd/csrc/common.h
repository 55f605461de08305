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

// fp32 -> bf16, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x0040u);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
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
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, MOE_WAVE);
    return v;
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
__device__ __forceinline__ int wave_id() { return threadIdx.x / MOE_WAVE; }

// Lanes below this one in the wave.
__device__ __forceinline__ uint64_t lanemask_lt() {
    int l = lane_id();
    return l == 0 ? 0ull : (~0ull >> (64 - l));
}

}  // namespace moe
