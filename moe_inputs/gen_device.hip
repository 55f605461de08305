// Seeded synthetic-input generator, device side (HIP, gfx950).
//
// Same definition as gen_host.c (counter-based SplitMix64 words; Irwin-Hall
// normals made of exact integer work and one IEEE fp32 multiply; bf16 by
// round-to-nearest-even), so that tensors too large to build on the host
// (tens to hundreds of GB of expert weights) are generated in HBM with the
// bytes the host would produce.  No arithmetic of the layer lives here.
#include <hip/hip_runtime.h>
#include <stdint.h>

#define MG_GAMMA 0x9E3779B97F4A7C15ULL

__device__ __host__ static inline uint64_t mgd_mix(uint64_t z) {
    z ^= z >> 30; z *= 0xBF58476D1CE4E5B9ULL;
    z ^= z >> 27; z *= 0x94D049BB133111EBULL;
    z ^= z >> 31;
    return z;
}
__device__ __host__ static inline uint64_t mgd_derive(uint64_t key, uint64_t x) {
    return mgd_mix(key ^ mgd_mix(x + MG_GAMMA));
}
__device__ static inline uint64_t mgd_word(uint64_t key, uint64_t i) { return mgd_mix(key + (i + 1) * MG_GAMMA); }

__device__ static inline float mgd_normal(uint64_t r, float c) {
    int32_t s = (int32_t)(r & 0xFFFF) + (int32_t)((r >> 16) & 0xFFFF) +
                (int32_t)((r >> 32) & 0xFFFF) + (int32_t)((r >> 48) & 0xFFFF) - 131070;
    return __fmul_rn((float)s, c);
}
__device__ static inline uint16_t mgd_bf16(float v) {
    uint32_t u = __float_as_uint(v);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// One launch covers n_experts sub-streams of n_per_expert elements each; for a
// single tensor pass n_experts = 1 and use_derive = 0 (key used as is).
__global__ void mgd_normal_bf16_kernel(uint16_t* out, int64_t n_per, int64_t e0, int64_t n_exp,
                                       uint64_t key, float c, int use_derive) {
    int64_t total = n_per * n_exp;
    for (int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; g < total;
         g += (int64_t)gridDim.x * blockDim.x) {
        int64_t e = g / n_per, i = g - e * n_per;
        uint64_t k = use_derive ? mgd_derive(key, (uint64_t)(e0 + e)) : key;
        out[g] = mgd_bf16(mgd_normal(mgd_word(k, (uint64_t)i), c));
    }
}
__global__ void mgd_normal_f32_kernel(float* out, int64_t n_per, int64_t e0, int64_t n_exp,
                                      uint64_t key, float c, int use_derive) {
    int64_t total = n_per * n_exp;
    for (int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; g < total;
         g += (int64_t)gridDim.x * blockDim.x) {
        int64_t e = g / n_per, i = g - e * n_per;
        uint64_t k = use_derive ? mgd_derive(key, (uint64_t)(e0 + e)) : key;
        out[g] = mgd_normal(mgd_word(k, (uint64_t)i), c);
    }
}
// Bytes: each thread writes 8 bytes (one word) when the 8 bytes lie in one expert.
__global__ void mgd_bytes_kernel(uint8_t* out, int64_t n_per, int64_t e0, int64_t n_exp,
                                 uint64_t key, int use_derive) {
    int64_t total = n_per * n_exp;
    for (int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; g < total;
         g += (int64_t)gridDim.x * blockDim.x) {
        int64_t e = g / n_per, i = g - e * n_per;
        uint64_t k = use_derive ? mgd_derive(key, (uint64_t)(e0 + e)) : key;
        out[g] = (uint8_t)(mgd_word(k, (uint64_t)i >> 3) >> (8 * (i & 7)));
    }
}
__global__ void mgd_scale_bytes_kernel(uint8_t* out, int64_t n_per, int64_t e0, int64_t n_exp,
                                       uint64_t key, int lo, int hi, int use_derive) {
    int64_t total = n_per * n_exp;
    uint64_t span = (uint64_t)(hi - lo + 1);
    for (int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; g < total;
         g += (int64_t)gridDim.x * blockDim.x) {
        int64_t e = g / n_per, i = g - e * n_per;
        uint64_t k = use_derive ? mgd_derive(key, (uint64_t)(e0 + e)) : key;
        out[g] = (uint8_t)(lo + (int)(((mgd_word(k, (uint64_t)i) >> 32) * span) >> 32));
    }
}

static int mgd_grid(int64_t total) {
    int64_t b = (total + 255) / 256;
    if (b > 65536) b = 65536;
    if (b < 1) b = 1;
    return (int)b;
}

extern "C" {
// All return 0 on success, a HIP error code otherwise. `out` is a device
// pointer with room for n_per * n_exp elements; `stream` is a hipStream_t.
int mgd_fill_normal_bf16(void* out, int64_t n_per, int64_t e0, int64_t n_exp, uint64_t key, float c,
                         int use_derive, void* stream) {
    if (n_per * n_exp == 0) return 0;
    hipLaunchKernelGGL(mgd_normal_bf16_kernel, dim3(mgd_grid(n_per * n_exp)), dim3(256), 0,
                       (hipStream_t)stream, (uint16_t*)out, n_per, e0, n_exp, key, c, use_derive);
    return (int)hipGetLastError();
}
int mgd_fill_normal_f32(void* out, int64_t n_per, int64_t e0, int64_t n_exp, uint64_t key, float c,
                        int use_derive, void* stream) {
    if (n_per * n_exp == 0) return 0;
    hipLaunchKernelGGL(mgd_normal_f32_kernel, dim3(mgd_grid(n_per * n_exp)), dim3(256), 0,
                       (hipStream_t)stream, (float*)out, n_per, e0, n_exp, key, c, use_derive);
    return (int)hipGetLastError();
}
int mgd_fill_bytes(void* out, int64_t n_per, int64_t e0, int64_t n_exp, uint64_t key, int use_derive,
                   void* stream) {
    if (n_per * n_exp == 0) return 0;
    hipLaunchKernelGGL(mgd_bytes_kernel, dim3(mgd_grid(n_per * n_exp)), dim3(256), 0,
                       (hipStream_t)stream, (uint8_t*)out, n_per, e0, n_exp, key, use_derive);
    return (int)hipGetLastError();
}
int mgd_fill_scale_bytes(void* out, int64_t n_per, int64_t e0, int64_t n_exp, uint64_t key, int lo,
                         int hi, int use_derive, void* stream) {
    if (n_per * n_exp == 0) return 0;
    hipLaunchKernelGGL(mgd_scale_bytes_kernel, dim3(mgd_grid(n_per * n_exp)), dim3(256), 0,
                       (hipStream_t)stream, (uint8_t*)out, n_per, e0, n_exp, key, lo, hi, use_derive);
    return (int)hipGetLastError();
}
}
