/*
 * Seeded synthetic-input generator, host side (plain C).
 *
 * This file holds no arithmetic of the mixture-of-experts layer: it only
 * turns (seed, tensor tag, index) into bytes.  The device twin in
 * gen_device.hip implements the same definition; a test checks that both
 * produce identical bytes.
 *
 * Definition (counter-based, after SplitMix64 -- G. Steele, D. Lea,
 * C. Flood, "Fast splittable pseudorandom number generators", OOPSLA 2014,
 * with the output mix constants of S. Vigna's public splitmix64.c):
 *   GAMMA       = 0x9E3779B97F4A7C15
 *   mix(z)      : z ^= z>>30; z *= 0xBF58476D1CE4E5B9;
 *                 z ^= z>>27; z *= 0x94D049BB133111EB; z ^= z>>31
 *   derive(k,x) = mix(k ^ mix(x + GAMMA))           (sub-stream keys)
 *   word(k,i)   = mix(k + (i+1)*GAMMA)              (i-th 64-bit word)
 *   normal      : s = sum of the four 16-bit fields of word(k,i) - 131070,
 *                 value = (float)s * c  with c = (float)(sigma/sqrt((2^32-1)/3))
 *                 (Irwin-Hall sum of four uniforms: mean 0, std sigma,
 *                 bounded by +-3.46 sigma; exact integer work and one IEEE
 *                 fp32 multiply, so host and device agree bit for bit)
 *   bf16        : round-to-nearest-even of the fp32 value
 *   bytes       : byte i = bits 8*(i%8).. of word(k, i/8)
 *   scale bytes : byte i = lo + (((word(k,i) >> 32) * (hi-lo+1)) >> 32)
 */
#include <stdint.h>
#include <stddef.h>

#define MG_GAMMA 0x9E3779B97F4A7C15ULL

static inline uint64_t mg_mix(uint64_t z) {
    z ^= z >> 30; z *= 0xBF58476D1CE4E5B9ULL;
    z ^= z >> 27; z *= 0x94D049BB133111EBULL;
    z ^= z >> 31;
    return z;
}

uint64_t mg_derive(uint64_t key, uint64_t x) { return mg_mix(key ^ mg_mix(x + MG_GAMMA)); }

uint64_t mg_word(uint64_t key, uint64_t i) { return mg_mix(key + (i + 1) * MG_GAMMA); }

static inline int32_t mg_irwin_hall(uint64_t r) {
    int32_t s = (int32_t)(r & 0xFFFF) + (int32_t)((r >> 16) & 0xFFFF) +
                (int32_t)((r >> 32) & 0xFFFF) + (int32_t)((r >> 48) & 0xFFFF);
    return s - 131070;
}

static inline uint16_t mg_f32_to_bf16_rne(float v) {
    union { float f; uint32_t u; } b; b.f = v;
    uint32_t u = b.u;
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

/* out[i] = normal value i of the stream, as fp32, for i in [start, start+n) */
void mg_fill_normal_f32(float* out, int64_t n, uint64_t key, float c, int64_t start) {
    for (int64_t i = 0; i < n; ++i)
        out[i] = (float)mg_irwin_hall(mg_word(key, (uint64_t)(start + i))) * c;
}

void mg_fill_normal_bf16(uint16_t* out, int64_t n, uint64_t key, float c, int64_t start) {
    for (int64_t i = 0; i < n; ++i)
        out[i] = mg_f32_to_bf16_rne((float)mg_irwin_hall(mg_word(key, (uint64_t)(start + i))) * c);
}

void mg_fill_bytes(uint8_t* out, int64_t n, uint64_t key, int64_t start) {
    for (int64_t i = 0; i < n; ++i) {
        uint64_t j = (uint64_t)(start + i);
        out[i] = (uint8_t)(mg_word(key, j >> 3) >> (8 * (j & 7)));
    }
}

void mg_fill_scale_bytes(uint8_t* out, int64_t n, uint64_t key, int lo, int hi, int64_t start) {
    uint64_t span = (uint64_t)(hi - lo + 1);
    for (int64_t i = 0; i < n; ++i)
        out[i] = (uint8_t)(lo + (int)(((mg_word(key, (uint64_t)(start + i)) >> 32) * span) >> 32));
}

/* Per-expert tensors: expert e of n_experts uses key derive(key, e) and
   indices 0..n_per_expert-1; the output is [n_experts, n_per_expert]. */
void mg_fill_normal_bf16_experts(uint16_t* out, int64_t n_per_expert, int64_t e0, int64_t n_experts,
                                 uint64_t key, float c) {
    for (int64_t e = 0; e < n_experts; ++e)
        mg_fill_normal_bf16(out + e * n_per_expert, n_per_expert, mg_derive(key, (uint64_t)(e0 + e)), c, 0);
}

void mg_fill_normal_f32_experts(float* out, int64_t n_per_expert, int64_t e0, int64_t n_experts,
                                uint64_t key, float c) {
    for (int64_t e = 0; e < n_experts; ++e)
        mg_fill_normal_f32(out + e * n_per_expert, n_per_expert, mg_derive(key, (uint64_t)(e0 + e)), c, 0);
}

void mg_fill_bytes_experts(uint8_t* out, int64_t n_per_expert, int64_t e0, int64_t n_experts, uint64_t key) {
    for (int64_t e = 0; e < n_experts; ++e)
        mg_fill_bytes(out + e * n_per_expert, n_per_expert, mg_derive(key, (uint64_t)(e0 + e)), 0);
}

void mg_fill_scale_bytes_experts(uint8_t* out, int64_t n_per_expert, int64_t e0, int64_t n_experts,
                                 uint64_t key, int lo, int hi) {
    for (int64_t e = 0; e < n_experts; ++e)
        mg_fill_scale_bytes(out + e * n_per_expert, n_per_expert, mg_derive(key, (uint64_t)(e0 + e)), lo, hi, 0);
}
