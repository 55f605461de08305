// LDS staging helpers shared by the MFMA kernels: direct global -> LDS loads and the explicit
// wait that keeps the next pipeline stage in flight.
#pragma once
#include <hip/hip_runtime.h>

namespace moe {

typedef float f32x16_t __attribute__((ext_vector_type(16)));

// s_waitcnt immediate: vmcnt(n) (n < 16), expcnt untouched, lgkmcnt(0).
#define VM_WAIT(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (7 << 4))

// global_load_lds: lane i's 4 or 16 bytes land at the wavefront's LDS base + (4 or 16) * i.
// (Plain functions: the builtin inside a lambda of a kernel template loses the host stub.)
__device__ __forceinline__ void dma16(const void* g, void* lds) { __builtin_amdgcn_global_load_lds(g, lds, 16, 0, 0); }
__device__ __forceinline__ void dma4(const void* g, void* lds) { __builtin_amdgcn_global_load_lds(g, lds, 4, 0, 0); }

// 16-byte chunk c of tile row r sits at physical chunk c ^ chunk_swz(r): every 8 (and 16)
// consecutive rows' reads of one chunk fall on distinct banks (64-byte rows).
__device__ __forceinline__ int chunk_swz(int r) { return ((r >> 1) ^ (r >> 2)) & 3; }

}  // namespace moe
