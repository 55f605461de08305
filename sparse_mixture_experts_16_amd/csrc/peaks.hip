// Peak probes of the machine the layer runs on, for the benchmark's roofline figures: what the
// HBM read stream and the matrix cores deliver on this device when nothing else limits them.
// Built into its own library (libmoe_peaks.so); the layer library does not use it.
//
//   peak_hbm_read    every lane streams 16-byte chunks of a buffer (grid-stride, all loads of a
//                    pass issued before any use) and folds them into one word per thread
//   peak_mfma_bf16   v_mfma_f32_32x32x16_bf16 on register operands, 8 independent accumulators
//                    per wavefront (the dependent-issue latency is covered)
//   peak_mfma_f8f4   v_mfma_scale_f32_32x32x64_f8f6f4 with fp8 (E4M3) x fp4 (E2M1) operands, the
//                    instruction of the MX prefill path, likewise
//   rows64_read      the prefill GEMM's tile-row pattern, for the read counters' calibration: rows
//                    of 4096 bytes, a wavefront reads 64-byte pieces of 16 rows per instruction and
//                    the next pieces of the same rows one instruction later; through registers or
//                    through LDS (global_load_lds_dwordx4, as the GEMMs fill their rings)
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef int i32x8_t __attribute__((ext_vector_type(8)));

namespace {

constexpr int READ_UNROLL = 8;

__global__ void __launch_bounds__(256) hbm_read(const uint4* __restrict__ src, size_t n_chunks, uint32_t* out) {
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    uint32_t acc = 0;
    for (; i + (READ_UNROLL - 1) * stride < n_chunks; i += READ_UNROLL * stride) {
        uint4 v[READ_UNROLL];
#pragma unroll
        for (int u = 0; u < READ_UNROLL; ++u) v[u] = src[i + u * stride];
#pragma unroll
        for (int u = 0; u < READ_UNROLL; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    for (; i < n_chunks; i += stride) {
        const uint4 v = src[i];
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = acc;
}

constexpr int ROW_BYTES = 4096, ROWS_PER_WAVE = 16;

__global__ void __launch_bounds__(256) rows64_read(const uint8_t* __restrict__ src, int rows, uint32_t* out) {
    const int lane = threadIdx.x & 63, wave = (int)((blockIdx.x * blockDim.x + threadIdx.x) >> 6);
    const int r = wave * ROWS_PER_WAVE + (lane >> 2);
    uint32_t acc = 0;
    if (r < rows) {
        const uint8_t* p = src + (size_t)r * ROW_BYTES + (lane & 3) * 16;
        for (int k = 0; k < ROW_BYTES / 64; ++k) {
            const uint4 v = *reinterpret_cast<const uint4*>(p + k * 64);
            acc ^= v.x ^ v.y ^ v.z ^ v.w;
        }
    }
    out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = acc;
}

__global__ void __launch_bounds__(256) rows64_dma(const uint8_t* __restrict__ src, int rows, uint32_t* out) {
    __shared__ __attribute__((aligned(16))) uint8_t lds[4][4][1024];  // wavefront x ring slot x 64 lanes * 16 B
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int wave = (int)((blockIdx.x * blockDim.x + threadIdx.x) >> 6);
    const int r = wave * ROWS_PER_WAVE + (lane >> 2);
    const uint8_t* p = src + (size_t)(r < rows ? r : 0) * ROW_BYTES + (lane & 3) * 16;
    uint32_t acc = 0;
    for (int k = 0; k < ROW_BYTES / 64; ++k) {
        __builtin_amdgcn_global_load_lds(p + k * 64, &lds[wv][k & 3][0], 16, 0, 0);
        if ((k & 3) == 3) {
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            for (int q = 0; q < 4; ++q) acc ^= *reinterpret_cast<volatile uint32_t*>(&lds[wv][q][lane * 16]);
        }
    }
    out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = acc;
}

constexpr int NACC = 8;

__global__ void __launch_bounds__(256) mfma_bf16(int iters, float* out) {
    const int lane = threadIdx.x & 63;
    bf16x8_t a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a[i] = (__bf16)(0.001f * (float)(lane + i));
        b[i] = (__bf16)(0.002f * (float)(lane - i));
    }
    f32x16_t acc[NACC];
#pragma unroll
    for (int j = 0; j < NACC; ++j) acc[j] = f32x16_t{};
    for (int it = 0; it < iters; ++it)
#pragma unroll
        for (int j = 0; j < NACC; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[j], 0, 0, 0);
    float s = 0.0f;
#pragma unroll
    for (int j = 0; j < NACC; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) s += acc[j][e];
    out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

__global__ void __launch_bounds__(256) mfma_f8f4(int iters, float* out) {
    const int lane = threadIdx.x & 63;
    i32x8_t a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a[i] = 0x38383838 ^ (lane << (i & 3));  // E4M3 bytes around 1.0
        b[i] = i < 4 ? (0x22222222 ^ (lane & 0x11)) : 0;  // E2M1 nibbles around 1.0
    }
    f32x16_t acc[NACC];
#pragma unroll
    for (int j = 0; j < NACC; ++j) acc[j] = f32x16_t{};
    for (int it = 0; it < iters; ++it)
#pragma unroll
        for (int j = 0; j < NACC; ++j)
            acc[j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc[j], 0, 4, 0, 127, 0, 127);
    float s = 0.0f;
#pragma unroll
    for (int j = 0; j < NACC; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) s += acc[j][e];
    out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

}  // namespace

extern "C" {

// Reads `bytes` (a multiple of 16) of device memory at src; out receives blocks * 256 words.
int peak_hbm_read(const void* src, size_t bytes, int blocks, void* out, void* stream) {
    if (!src || !out || bytes % 16 || blocks < 1) return -1;
    hipLaunchKernelGGL(hbm_read, dim3(blocks), dim3(256), 0, (hipStream_t)stream, (const uint4*)src, bytes / 16,
                       (uint32_t*)out);
    return hipGetLastError() == hipSuccess ? 0 : -4;
}

// blocks workgroups of 4 wavefronts, each wavefront iters x NACC matrix instructions;
// out receives blocks * 256 floats.  Flops: blocks * 4 * iters * NACC * (2 * 32 * 32 * K),
// K = 16 (bf16) or 64 (fp8 x fp4).
int peak_mfma(int kind, int blocks, int iters, void* out, void* stream) {
    if (!out || blocks < 1 || iters < 1) return -1;
    if (kind == 0) hipLaunchKernelGGL(mfma_bf16, dim3(blocks), dim3(256), 0, (hipStream_t)stream, iters, (float*)out);
    else hipLaunchKernelGGL(mfma_f8f4, dim3(blocks), dim3(256), 0, (hipStream_t)stream, iters, (float*)out);
    return hipGetLastError() == hipSuccess ? 0 : -4;
}

int peak_mfma_per_wave(void) { return NACC; }

// Reads `bytes` (a multiple of 64 rows of 4096 bytes) in the tile-row pattern, through registers
// (dma = 0) or through LDS (dma = 1); out receives bytes / 256 words.
int peak_rows64_read(const void* src, size_t bytes, int dma, void* out, void* stream) {
    if (!src || !out || bytes % ((size_t)ROW_BYTES * ROWS_PER_WAVE * 4)) return -1;
    const int rows = (int)(bytes / ROW_BYTES);
    const dim3 grid(rows / (ROWS_PER_WAVE * 4)), block(256);
    if (dma) hipLaunchKernelGGL(rows64_dma, grid, block, 0, (hipStream_t)stream, (const uint8_t*)src, rows, (uint32_t*)out);
    else hipLaunchKernelGGL(rows64_read, grid, block, 0, (hipStream_t)stream, (const uint8_t*)src, rows, (uint32_t*)out);
    return hipGetLastError() == hipSuccess ? 0 : -4;
}

}  // extern "C"
