// 16-byte weight chunks and their dot products with activation segments.
//
// A lane always loads 16 contiguous bytes of a weight row (one global_load_dwordx4):
//   f32   -> 4 elements
//   bf16  -> 8 elements
//   MXFP4 -> 32 elements (E2M1 codes, element 2i in the low nibble of byte i) plus the one
//            E8M0 scale byte shared by those 32 elements.
// MXFP4 codes are expanded in registers with the gfx950 scaled converts
// (v_cvt_scalef32_pk_{bf16,f32}_fp4), which multiply by a power-of-two fp32 scale; a scale
// byte of 0xFF (NaN in E8M0) is applied afterwards by forcing the chunk's result to NaN.
#pragma once
#include "common.h"

namespace moe {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ bf16x2_t as_bf16x2(uint32_t u) { return __builtin_bit_cast(bf16x2_t, u); }
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(a), as_bf16x2(b), c, false);
}

// 2^(s-127) as an fp32 number (s = 0 gives the subnormal 2^-127; s = 255 is handled by callers).
__device__ __forceinline__ float e8m0_to_f32(uint32_t s) {
    return s == 0 ? __uint_as_float(0x00400000u) : __uint_as_float(s << 23);
}

template <int WT> struct WChunk;

// ---------------------------------------------------------------- f32 weights
template <> struct WChunk<0> {
    static constexpr int EC = 4;
    uint4 v;
    __device__ __forceinline__ void load(const uint8_t* row, const uint8_t*, int c) {
        v = reinterpret_cast<const uint4*>(row)[c];
    }
    __device__ __forceinline__ void zero() { v = make_uint4(0, 0, 0, 0); }
    // activation segment of EC f32 values
    __device__ __forceinline__ float dot_f32(const float* a, float acc) const {
        float4 x = *reinterpret_cast<const float4*>(a);
        acc = fmaf(__uint_as_float(v.x), x.x, acc);
        acc = fmaf(__uint_as_float(v.y), x.y, acc);
        acc = fmaf(__uint_as_float(v.z), x.z, acc);
        acc = fmaf(__uint_as_float(v.w), x.w, acc);
        return acc;
    }
};

// ---------------------------------------------------------------- bf16 weights
template <> struct WChunk<1> {
    static constexpr int EC = 8;
    uint4 v;
    __device__ __forceinline__ void load(const uint8_t* row, const uint8_t*, int c) {
        v = reinterpret_cast<const uint4*>(row)[c];
    }
    __device__ __forceinline__ void zero() { v = make_uint4(0, 0, 0, 0); }
    // activation segment of EC bf16 values (16 bytes): exact products, fp32 sums
    __device__ __forceinline__ float dot_bf16(const uint16_t* a, float acc) const {
        uint4 x = *reinterpret_cast<const uint4*>(a);
        acc = dot2_bf16(v.x, x.x, acc);
        acc = dot2_bf16(v.y, x.y, acc);
        acc = dot2_bf16(v.z, x.z, acc);
        acc = dot2_bf16(v.w, x.w, acc);
        return acc;
    }
    __device__ __forceinline__ float dot_f32(const float* a, float acc) const {
        float4 x0 = reinterpret_cast<const float4*>(a)[0];
        float4 x1 = reinterpret_cast<const float4*>(a)[1];
        acc = fmaf(bf16_lo(v.x), x0.x, acc);
        acc = fmaf(bf16_hi(v.x), x0.y, acc);
        acc = fmaf(bf16_lo(v.y), x0.z, acc);
        acc = fmaf(bf16_hi(v.y), x0.w, acc);
        acc = fmaf(bf16_lo(v.z), x1.x, acc);
        acc = fmaf(bf16_hi(v.z), x1.y, acc);
        acc = fmaf(bf16_lo(v.w), x1.z, acc);
        acc = fmaf(bf16_hi(v.w), x1.w, acc);
        return acc;
    }
};

// ---------------------------------------------------------------- MXFP4 weights
template <> struct WChunk<2> {
    static constexpr int EC = 32;
    uint4 v;
    uint32_t s;  // scale byte
    __device__ __forceinline__ void load(const uint8_t* row, const uint8_t* srow, int c) {
        v = reinterpret_cast<const uint4*>(row)[c];
        s = srow[c];
    }
    __device__ __forceinline__ void zero() {
        v = make_uint4(0, 0, 0, 0);
        s = 127;
    }
    // 8 codes of one 32-bit word against 8 bf16 activations (uint4 = 4 pairs)
    __device__ __forceinline__ static float word_bf16(uint32_t w, float sc, uint4 x, float acc) {
        acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 0), as_bf16x2(x.x), acc, false);
        acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 1), as_bf16x2(x.y), acc, false);
        acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 2), as_bf16x2(x.z), acc, false);
        acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 3), as_bf16x2(x.w), acc, false);
        return acc;
    }
    __device__ __forceinline__ float dot_bf16(const uint16_t* a, float acc) const {
        const uint4* x = reinterpret_cast<const uint4*>(a);
        const float sc = e8m0_to_f32(s);
        float part = 0.0f;
        part = word_bf16(v.x, sc, x[0], part);
        part = word_bf16(v.y, sc, x[1], part);
        part = word_bf16(v.z, sc, x[2], part);
        part = word_bf16(v.w, sc, x[3], part);
        return s == 255u ? __uint_as_float(0x7FC00000u) : acc + part;
    }
    __device__ __forceinline__ static float word_f32(uint32_t w, float sc, const float* a, float acc) {
        const float4 a0 = reinterpret_cast<const float4*>(a)[0];
        const float4 a1 = reinterpret_cast<const float4*>(a)[1];
        const f32x2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, sc, 0);
        const f32x2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, sc, 1);
        const f32x2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, sc, 2);
        const f32x2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, sc, 3);
        acc = fmaf(p0.x, a0.x, acc);
        acc = fmaf(p0.y, a0.y, acc);
        acc = fmaf(p1.x, a0.z, acc);
        acc = fmaf(p1.y, a0.w, acc);
        acc = fmaf(p2.x, a1.x, acc);
        acc = fmaf(p2.y, a1.y, acc);
        acc = fmaf(p3.x, a1.z, acc);
        acc = fmaf(p3.y, a1.w, acc);
        return acc;
    }
    __device__ __forceinline__ float dot_f32(const float* a, float acc) const {
        const float sc = e8m0_to_f32(s);
        float part = 0.0f;
        part = word_f32(v.x, sc, a, part);
        part = word_f32(v.y, sc, a + 8, part);
        part = word_f32(v.z, sc, a + 16, part);
        part = word_f32(v.w, sc, a + 24, part);
        return s == 255u ? __uint_as_float(0x7FC00000u) : acc + part;
    }
};

// ---------------------------------------------------------------- NVFP4 weights
// OCP FP8 E4M3 (no infinities) -> fp32 from its bit fields: (1 + m/8) * 2^(e-7), subnormal
// m/8 * 2^-6, NaN for e = 15 and m = 7.
__device__ __forceinline__ float e4m3_to_f32(uint32_t b) {
    const uint32_t e = (b >> 3) & 15u, m = b & 7u;
    float v = e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : (float)m * 0x1p-9f;
    if (e == 15u && m == 7u) v = __uint_as_float(0x7FC00000u);
    return (b & 0x80u) ? -v : v;
}

// 32 E2M1 codes (16 bytes) and their two E4M3 block scales (one per 16 elements); the codes
// expand exactly with the unit-scale converts and each block's partial sum takes its scale.
// The tensor's fp32 scale is applied by the kernels to the finished row sums.
template <> struct WChunk<3> {
    static constexpr int EC = 32;
    uint4 v;
    uint32_t s;  // two scale bytes: block 0 in bits 0..7, block 1 in bits 8..15
    __device__ __forceinline__ void load(const uint8_t* row, const uint8_t* srow, int c) {
        v = reinterpret_cast<const uint4*>(row)[c];
        s = reinterpret_cast<const uint16_t*>(srow)[c];
    }
    __device__ __forceinline__ void zero() {
        v = make_uint4(0, 0, 0, 0);
        s = 0x3838u;  // 1.0, 1.0
    }
    __device__ __forceinline__ float dot_bf16(const uint16_t* a, float acc) const {
        const uint4* x = reinterpret_cast<const uint4*>(a);
        float p0 = 0.0f, p1 = 0.0f;
        p0 = WChunk<2>::word_bf16(v.x, 1.0f, x[0], p0);
        p0 = WChunk<2>::word_bf16(v.y, 1.0f, x[1], p0);
        p1 = WChunk<2>::word_bf16(v.z, 1.0f, x[2], p1);
        p1 = WChunk<2>::word_bf16(v.w, 1.0f, x[3], p1);
        return acc + p0 * e4m3_to_f32(s & 0xFFu) + p1 * e4m3_to_f32(s >> 8);
    }
    __device__ __forceinline__ float dot_f32(const float* a, float acc) const {
        float p0 = 0.0f, p1 = 0.0f;
        p0 = WChunk<2>::word_f32(v.x, 1.0f, a, p0);
        p0 = WChunk<2>::word_f32(v.y, 1.0f, a + 8, p0);
        p1 = WChunk<2>::word_f32(v.z, 1.0f, a + 16, p1);
        p1 = WChunk<2>::word_f32(v.w, 1.0f, a + 24, p1);
        return acc + p0 * e4m3_to_f32(s & 0xFFu) + p1 * e4m3_to_f32(s >> 8);
    }
};

__host__ __device__ __forceinline__ int64_t row_bytes(int wt, int64_t K) {
    return wt == 0 ? K * 4 : (wt == 1 ? K * 2 : K / 2);
}
// Scale bytes per weight row: MXFP4 one E8M0 per 32 elements, NVFP4 one E4M3 per 16.
__host__ __device__ __forceinline__ int64_t scale_row_bytes(int wt, int64_t K) {
    return wt == 2 ? K / 32 : (wt == 3 ? K / 16 : 0);
}

}  // namespace moe
