// MXFP8 (OCP Microscaling Formats v1.0: E4M3 elements, one E8M0 scale per 32) quantisation of
// one 32-element block on gfx950's scaled converts; used by the activation quantiser and the MX
// gate/up epilogue (mxgemm.hip) and by the bf16 path's down-projection correction plane (gemm.hip).
#pragma once
#include "common.h"

namespace moe {

typedef short v2i16_t __attribute__((ext_vector_type(2)));

// E4M3 codes of four finite values, rounded to nearest even, magnitudes above 448 (E4M3's
// largest normal) clamped to it; code k in byte k.  v_cvt_scalef32_pk_fp8_f32 (scale 1) rounds to
// nearest even but does not saturate, so its inputs are clamped first: checked on the GPU against
// the rounding done on the fp32 bits, identical for every finite fp32 input (subnormal steps of
// 2^-9 and signed zeros included).
__device__ __forceinline__ float clamp448(float q) { return fminf(fmaxf(q, -448.0f), 448.0f); }
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d) {
    v2i16_t r = {0, 0};
    r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(r, clamp448(a), clamp448(b), 1.0f, false);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(r, clamp448(c), clamp448(d), 1.0f, true);
    return __builtin_bit_cast(uint32_t, r);
}

// Shared scale of a block from the bit pattern of its largest magnitude: E8M0 byte
// floor(log2 amax) - 8 + 127 = (biased fp32 exponent) - 8, at least 0; 0xFF (NaN) when the
// block holds an infinity or a NaN.  Codes are packed 4 to a word, element i in byte i % 4.
__device__ __forceinline__ uint32_t mx_block(const float (&v)[32], uint32_t (&code)[8]) {
    uint32_t am = 0u;
#pragma unroll
    for (int i = 0; i < 32; ++i) am = max(am, __float_as_uint(v[i]) & 0x7FFFFFFFu);
    const uint32_t ex = am >> 23;
    if (ex == 0xFFu) {
#pragma unroll
        for (int w = 0; w < 8; ++w) code[w] = 0x7F7F7F7Fu;
        return 0xFFu;
    }
    const uint32_t sb = ex > 8u ? ex - 8u : 0u;
    const float mul = __uint_as_float((254u - sb) << 23);  // 2^(127 - sb): exact scaling
#pragma unroll
    for (int w = 0; w < 8; ++w) code[w] = e4m3x4(v[4 * w] * mul, v[4 * w + 1] * mul, v[4 * w + 2] * mul, v[4 * w + 3] * mul);
    return sb;
}

}  // namespace moe
