// Gather combine (prefill path), standalone MXFP4 / NVFP4 dequantisation and the
// residual-stack RMS normalisation.
#include "common.h"
#include "kernels.h"
#include "wchunk.h"

namespace moe {

// ------------------------------------------------------------------------------------------------
// out[t] = sum over the token's k pairs in ascending sorted position (= ascending expert id) of
// g * y_sorted[pos] (+ y_shared[t]) (+ out[t] when accumulating); fp32 sums.  The exact merge of
// partial expert sums is the pages' own claim (dothoosh.com FreeToken article, "FreeToken
// architecture and the sparsity puzzle", mechanism 1).  One workgroup per token, 8 columns per
// thread with 16-byte loads.
// ------------------------------------------------------------------------------------------------
// 8 consecutive values as 16-byte loads/stores (bf16: one, f32: two)
template <typename T> struct vec8;
template <> struct vec8<uint16_t> {
    __device__ __forceinline__ static void load(const uint16_t* p, float* v) {
        const uint4 q = *reinterpret_cast<const uint4*>(p);
        v[0] = bf16_lo(q.x); v[1] = bf16_hi(q.x); v[2] = bf16_lo(q.y); v[3] = bf16_hi(q.y);
        v[4] = bf16_lo(q.z); v[5] = bf16_hi(q.z); v[6] = bf16_lo(q.w); v[7] = bf16_hi(q.w);
    }
    __device__ __forceinline__ static void store(uint16_t* p, const float* v) {
        *reinterpret_cast<uint4*>(p) = make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]),
                                                  pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7]));
    }
};
template <> struct vec8<float> {
    __device__ __forceinline__ static void load(const float* p, float* v) {
        const float4 a = reinterpret_cast<const float4*>(p)[0], b = reinterpret_cast<const float4*>(p)[1];
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    }
    __device__ __forceinline__ static void store(float* p, const float* v) {
        reinterpret_cast<float4*>(p)[0] = make_float4(v[0], v[1], v[2], v[3]);
        reinterpret_cast<float4*>(p)[1] = make_float4(v[4], v[5], v[6], v[7]);
    }
};

template <typename Y, typename O>
__global__ void __launch_bounds__(256) combine_gather(const Y* __restrict__ y, const int32_t* __restrict__ inv,
                                                      const float* __restrict__ topk_w, const Y* __restrict__ ysh,
                                                      O* __restrict__ out, int d, int k, int accumulate,
                                                      const int32_t* __restrict__ idx, const uint8_t* __restrict__ mask,
                                                      int E) {
    __shared__ int s_raw[MOE_MAX_K];
    __shared__ int s_pos[MOE_MAX_K];
    __shared__ float s_g[MOE_MAX_K];
    const int t = blockIdx.x;
    // the token's pairs in ascending sorted position (= ascending expert): thread j < k loads pair j
    // and places it at its rank (positions are distinct; pairs outside a partial layer get -1 and
    // rank first, in pair order)
    int pos = -1;
    float g = 0.0f;
    if (threadIdx.x < k) {
        const int j = threadIdx.x;
        pos = inv[(int64_t)t * k + j];
        g = topk_w[(int64_t)t * k + j];
        if (mask) {
            const int e = idx[(int64_t)t * k + j];
            if (e < 0 || e >= E || !mask[e]) pos = -1;  // expert outside this partial layer
        }
        s_raw[j] = pos;
    }
    __syncthreads();
    if (threadIdx.x < k) {
        const int j = threadIdx.x;
        int r = 0;
        for (int i = 0; i < k; ++i) {
            const int pi = s_raw[i];
            r += pi < pos || (pi == pos && i < j);
        }
        s_pos[r] = pos;
        s_g[r] = g;
    }
    __syncthreads();
    for (int i0 = threadIdx.x * 8; i0 < d; i0 += blockDim.x * 8) {
        const int nv = min(8, d - i0);  // d is a multiple of 4 (f32) or 8 (bf16)
        if (nv == 8) {
            // 8 columns as whole 16-byte loads, 8 pairs' rows in flight at a time
            float acc[8];
#pragma unroll
            for (int v = 0; v < 8; ++v) acc[v] = 0.0f;
            for (int q0 = 0; q0 < k; q0 += 8) {
                float rv[8][8];
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const int pos = q0 + j < k ? s_pos[q0 + j] : -1;
                    if (pos >= 0) vec8<Y>::load(y + (int64_t)pos * d + i0, rv[j]);
                }
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const int pos = q0 + j < k ? s_pos[q0 + j] : -1;
                    if (pos < 0) continue;
                    const float g = s_g[q0 + j];
#pragma unroll
                    for (int v = 0; v < 8; ++v) acc[v] = fmaf(g, rv[j][v], acc[v]);
                }
            }
            if (ysh && (!mask || mask[E])) {
                float sv[8];
                vec8<Y>::load(ysh + (int64_t)t * d + i0, sv);
#pragma unroll
                for (int v = 0; v < 8; ++v) acc[v] += sv[v];
            }
            O* orow = out + (int64_t)t * d + i0;
            if (accumulate) {
                float pv[8];
                vec8<O>::load(orow, pv);
#pragma unroll
                for (int v = 0; v < 8; ++v) acc[v] += pv[v];
            }
            vec8<O>::store(orow, acc);
            continue;
        }
        float acc[8];
#pragma unroll
        for (int v = 0; v < 8; ++v) acc[v] = 0.0f;
        for (int q = 0; q < k; ++q) {
            const int pos = s_pos[q];
            if (pos < 0) continue;  // pair dropped by the permute (expert id out of range)
            const float g = s_g[q];
            const Y* yr = y + (int64_t)pos * d + i0;
#pragma unroll
            for (int v = 0; v < 8; ++v)
                if (v < nv) acc[v] = fmaf(g, io<Y>::ld(yr, v), acc[v]);
        }
        if (ysh && (!mask || mask[E])) {
            const Y* sr = ysh + (int64_t)t * d + i0;
#pragma unroll
            for (int v = 0; v < 8; ++v)
                if (v < nv) acc[v] += io<Y>::ld(sr, v);
        }
        O* orow = out + (int64_t)t * d + i0;
#pragma unroll
        for (int v = 0; v < 8; ++v) {
            if (v >= nv) continue;
            const float prev = accumulate ? io<O>::ld(orow, v) : 0.0f;
            io<O>::st(orow, v, prev + acc[v]);
        }
    }
}

hipError_t launch_combine(int y_dtype, int out_dtype, const void* y, const int32_t* inv, const float* topk_w,
                          const void* ysh, void* out, int T, int d, int k, bool accumulate, const int32_t* idx,
                          const uint8_t* mask, int E, hipStream_t st) {
    const int acc = accumulate ? 1 : 0;
    if (y_dtype == 0 && out_dtype == 0)
        hipLaunchKernelGGL((combine_gather<float, float>), dim3(T), dim3(256), 0, st, (const float*)y, inv, topk_w,
                           (const float*)ysh, (float*)out, d, k, acc, idx, mask, E);
    else if (y_dtype == 1 && out_dtype == 1)
        hipLaunchKernelGGL((combine_gather<uint16_t, uint16_t>), dim3(T), dim3(256), 0, st, (const uint16_t*)y, inv,
                           topk_w, (const uint16_t*)ysh, (uint16_t*)out, d, k, acc, idx, mask, E);
    else if (y_dtype == 1 && out_dtype == 0)
        hipLaunchKernelGGL((combine_gather<uint16_t, float>), dim3(T), dim3(256), 0, st, (const uint16_t*)y, inv,
                           topk_w, (const uint16_t*)ysh, (float*)out, d, k, acc, idx, mask, E);
    else
        hipLaunchKernelGGL((combine_gather<float, uint16_t>), dim3(T), dim3(256), 0, st, (const float*)y, inv,
                           topk_w, (const float*)ysh, (uint16_t*)out, d, k, acc, idx, mask, E);
    return hipGetLastError();
}

// ------------------------------------------------------------------------------------------------
// MXFP4 -> f32, one 16-byte code chunk (32 elements) per thread, through the same scaled
// converts the FFN kernels use.
// ------------------------------------------------------------------------------------------------
__global__ void __launch_bounds__(256) mxfp4_dequant_kernel(const uint8_t* __restrict__ codes,
                                                            const uint8_t* __restrict__ scales,
                                                            float* __restrict__ out, int64_t n_chunks) {
    for (int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; c < n_chunks;
         c += (int64_t)gridDim.x * blockDim.x) {
        const uint4 v = reinterpret_cast<const uint4*>(codes)[c];
        const uint32_t s = scales[c];
        const float sc = e8m0_to_f32(s);
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
        float4* o = reinterpret_cast<float4*>(out + c * 32);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            f32x2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[q], sc, 0);
            f32x2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[q], sc, 1);
            f32x2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[q], sc, 2);
            f32x2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[q], sc, 3);
            float4 a = make_float4(p0.x, p0.y, p1.x, p1.y);
            float4 b = make_float4(p2.x, p2.y, p3.x, p3.y);
            if (s == 255u) {
                const float nan = __uint_as_float(0x7FC00000u);
                a = make_float4(nan, nan, nan, nan);
                b = a;
            }
            o[2 * q] = a;
            o[2 * q + 1] = b;
        }
    }
}

hipError_t launch_mxfp4_dequant(const uint8_t* codes, const uint8_t* scales, float* out, int64_t rows, int64_t K,
                                hipStream_t st) {
    const int64_t n_chunks = rows * (K / 32);
    if (n_chunks == 0) return hipSuccess;
    int64_t blocks = (n_chunks + 255) / 256;
    if (blocks > 16384) blocks = 16384;
    hipLaunchKernelGGL(mxfp4_dequant_kernel, dim3((unsigned)blocks), dim3(256), 0, st, codes, scales, out, n_chunks);
    return hipGetLastError();
}

// NVFP4 -> f32: per 32-element chunk, the unit-scale converts give the exact E2M1 values, each
// 16-element block's E4M3 scale multiplies them exactly, and the tensor scale rounds once.
__global__ void __launch_bounds__(256) nvfp4_dequant_kernel(const uint8_t* __restrict__ codes,
                                                            const uint8_t* __restrict__ scales, float gscale,
                                                            float* __restrict__ out, int64_t n_chunks) {
    for (int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; c < n_chunks;
         c += (int64_t)gridDim.x * blockDim.x) {
        const uint4 v = reinterpret_cast<const uint4*>(codes)[c];
        const uint32_t s2 = reinterpret_cast<const uint16_t*>(scales)[c];
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
        float4* o = reinterpret_cast<float4*>(out + c * 32);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const float sb = e4m3_to_f32(q < 2 ? (s2 & 0xFFu) : (s2 >> 8));
            f32x2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[q], 1.0f, 0);
            f32x2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[q], 1.0f, 1);
            f32x2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[q], 1.0f, 2);
            f32x2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[q], 1.0f, 3);
            o[2 * q] = make_float4((p0.x * sb) * gscale, (p0.y * sb) * gscale, (p1.x * sb) * gscale, (p1.y * sb) * gscale);
            o[2 * q + 1] = make_float4((p2.x * sb) * gscale, (p2.y * sb) * gscale, (p3.x * sb) * gscale, (p3.y * sb) * gscale);
        }
    }
}

hipError_t launch_nvfp4_dequant(const uint8_t* codes, const uint8_t* scales, float gscale, float* out, int64_t rows,
                                int64_t K, hipStream_t st) {
    const int64_t n_chunks = rows * (K / 32);
    if (n_chunks == 0) return hipSuccess;
    int64_t blocks = (n_chunks + 255) / 256;
    if (blocks > 16384) blocks = 16384;
    hipLaunchKernelGGL(nvfp4_dequant_kernel, dim3((unsigned)blocks), dim3(256), 0, st, codes, scales, gscale, out,
                       n_chunks);
    return hipGetLastError();
}

// ------------------------------------------------------------------------------------------------
// Residual stack glue: x = h / sqrt(mean(h^2) + eps), rounded to the activation dtype.
// One workgroup per token.
// ------------------------------------------------------------------------------------------------
template <typename X>
__global__ void __launch_bounds__(256) rmsnorm_kernel(const float* __restrict__ h, X* __restrict__ x, int d, float eps) {
    __shared__ float s_part[4];
    const int t = blockIdx.x;
    const float* hr = h + (int64_t)t * d;
    float ss = 0.0f;
    for (int i = threadIdx.x; i < d; i += blockDim.x) ss = fmaf(hr[i], hr[i], ss);
    ss = wave_sum(ss);
    if (lane_id() == 0) s_part[wave_id()] = ss;
    __syncthreads();
    const float tot = s_part[0] + s_part[1] + s_part[2] + s_part[3];
    const float inv = 1.0f / sqrtf(tot / (float)d + eps);
    X* xr = x + (int64_t)t * d;
    for (int i = threadIdx.x; i < d; i += blockDim.x) io<X>::st(xr, i, hr[i] * inv);
}

hipError_t launch_rmsnorm(int x_dtype, const float* h, void* x, int T, int d, float eps, hipStream_t st) {
    if (x_dtype == 0)
        hipLaunchKernelGGL((rmsnorm_kernel<float>), dim3(T), dim3(256), 0, st, h, (float*)x, d, eps);
    else
        hipLaunchKernelGGL((rmsnorm_kernel<uint16_t>), dim3(T), dim3(256), 0, st, h, (uint16_t*)x, d, eps);
    return hipGetLastError();
}

}  // namespace moe
