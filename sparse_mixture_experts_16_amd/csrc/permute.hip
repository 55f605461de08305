// Grouping tokens by expert: a stable counting sort of the flat (token, slot) pairs
// p = t*k + j by expert id, with an LDS histogram, a prefix scan and a stable scatter.
//
// At prefill thousands of tokens reach nearly every expert (dothoosh.com FreeToken article,
// "FreeToken architecture and the sparsity puzzle", first failure mode), so the sort must
// scale; at decode only T*k <= a few hundred pairs exist and one workgroup does everything.
//
// Stability without atomics deciding order: within a wavefront, the lanes holding the same
// expert are found with one ballot per bit of the expert id; a lane's rank among them is the
// popcount of that mask below it, and the group's last lane advances the expert's cursor.
// Chunks are visited in pair order, so the output order is ascending p within each expert.
#include "common.h"
#include "kernels.h"

namespace moe {

// Wave 0 of the block: from LDS counts s_cnt[0..E), write counts/offsets, the ascending list of
// experts with tokens, the per-expert tile offsets (ceil(count/bm) tiles each) and meta
// (meta[0] = active experts, meta[1] = tiles); leaves s_cur[e] = offsets[e].
__device__ void scan_counts_wave0(const int* s_cnt, int* s_cur, int E, int bm, int32_t* counts, int32_t* offsets,
                                  int32_t* act_list, int32_t* tile_off, int32_t* meta) {
    const int lane = lane_id();
    const int per = (E + MOE_WAVE - 1) / MOE_WAVE;
    const int lo = min(lane * per, E), hi = min(lo + per, E);
    int sc = 0, sa = 0, st = 0;
    for (int e = lo; e < hi; ++e) {
        int c = s_cnt[e];
        sc += c;
        sa += (c > 0);
        st += (c + bm - 1) / bm;
    }
    int pc = wave_incl_scan(sc) - sc, pa = wave_incl_scan(sa) - sa, pt = wave_incl_scan(st) - st;
    for (int e = lo; e < hi; ++e) {
        int c = s_cnt[e];
        if (counts) counts[e] = c;
        if (offsets) offsets[e] = pc;
        if (s_cur) s_cur[e] = pc;
        tile_off[e] = pt;
        if (c > 0) act_list[pa++] = e;
        pc += c;
        pt += (c + bm - 1) / bm;
    }
    if (lane == MOE_WAVE - 1) {
        if (offsets) offsets[E] = pc;
        tile_off[E] = pt;
        meta[0] = pa;
        meta[1] = pt;
    }
}

// Stable scatter of pairs [p0, p1) by wave 0, cursors in LDS.
__device__ void stable_scatter_wave(const int32_t* __restrict__ idx, int p0, int p1, int nbits, int e_lim, int* s_cur,
                                    int32_t* __restrict__ perm, int32_t* __restrict__ inv) {
    const int lane = lane_id();
    const uint64_t lt = lanemask_lt();
    for (int c = p0; c < p1; c += MOE_WAVE) {
        const int p = c + lane;
        int e = p < p1 ? idx[p] : 0;
        const bool valid = p < p1 && (unsigned)e < (unsigned)e_lim;
        if (p < p1 && !valid) inv[p] = -1;  // expert id outside [0, E): dropped
        if (!valid) e = 0;
        uint64_t m = __ballot(valid);
        for (int b = 0; b < nbits; ++b) {
            const bool bit = (e >> b) & 1;
            const uint64_t bb = __ballot(valid && bit);
            m &= bit ? bb : ~bb;
        }
        if (valid) {
            const int base = s_cur[e];
            const int pos = base + __popcll(m & lt);
            perm[pos] = p;
            inv[p] = pos;
            if ((m >> lane) == 1ull) s_cur[e] = base + __popcll(m);
        }
    }
}

__device__ __forceinline__ int bits_for(int E) {
    int b = 0;
    while ((1 << b) < E) ++b;
    return b;
}

// Single workgroup: histogram, scan and scatter for small P (decode).
__global__ void __launch_bounds__(256) permute_small(const int32_t* __restrict__ idx, int P, int E, int bm,
                                                     int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* inv,
                                                     int32_t* act_list, int32_t* tile_off, int32_t* meta) {
    __shared__ int s_cnt[MOE_MAX_E];
    __shared__ int s_cur[MOE_MAX_E];
    for (int e = threadIdx.x; e < E; e += blockDim.x) s_cnt[e] = 0;
    __syncthreads();
    for (int p = threadIdx.x; p < P; p += blockDim.x) {
        const int e = idx[p];
        if ((unsigned)e < (unsigned)E) atomicAdd(&s_cnt[e], 1);
    }
    __syncthreads();
    if (wave_id() == 0) {
        scan_counts_wave0(s_cnt, s_cur, E, bm, counts, offsets, act_list, tile_off, meta);
        stable_scatter_wave(idx, 0, P, bits_for(E), E, s_cur, perm, inv);
    }
}

// Large P, pass 1: per-chunk histograms blk[b][e].
__global__ void __launch_bounds__(256) permute_hist(const int32_t* __restrict__ idx, int P, int E, int chunk,
                                                    int32_t* __restrict__ blk) {
    __shared__ int s_cnt[MOE_MAX_E];
    for (int e = threadIdx.x; e < E; e += blockDim.x) s_cnt[e] = 0;
    __syncthreads();
    const int p0 = blockIdx.x * chunk, p1 = min(p0 + chunk, P);
    for (int p = p0 + threadIdx.x; p < p1; p += blockDim.x) {
        const int e = idx[p];
        if ((unsigned)e < (unsigned)E) atomicAdd(&s_cnt[e], 1);
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += blockDim.x) blk[(int64_t)blockIdx.x * E + e] = s_cnt[e];
}

// Large P, pass 2 (one workgroup): totals, offsets, lists, and each chunk's starting cursor
// blk[b][e] = offsets[e] + (pairs of expert e in chunks before b).  The nblk x E counts are
// staged in LDS with coalesced loads; each expert's chunks are split into segments, one thread
// per (expert, segment) sums its segment, the segment sums are scanned per expert, and each
// thread writes its chunks' running sums.
__global__ void __launch_bounds__(1024) permute_scan(int32_t* __restrict__ blk, int nblk, int E, int bm,
                                                     int32_t* counts, int32_t* offsets, int32_t* act_list,
                                                     int32_t* tile_off, int32_t* meta) {
    __shared__ int s_blk[PERMUTE_SCAN_LDS];
    __shared__ int s_seg[1024];
    __shared__ int s_cnt[MOE_MAX_E];
    __shared__ int s_cur[MOE_MAX_E];
    const int n = nblk * E;
    for (int i0 = threadIdx.x; i0 < n; i0 += 8 * blockDim.x) {  // 8 loads in flight per thread
        int v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int i = i0 + j * blockDim.x;
            v[j] = i < n ? blk[i] : 0;
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int i = i0 + j * blockDim.x;
            if (i < n) s_blk[i] = v[j];
        }
    }
    const int nseg = E >= (int)blockDim.x ? 1 : (int)blockDim.x / E;
    const int seg_len = (nblk + nseg - 1) / nseg;
    __syncthreads();
    for (int t = threadIdx.x; t < E * nseg; t += blockDim.x) {
        const int e = t % E, sg = t / E;
        const int b0 = sg * seg_len, b1 = min(b0 + seg_len, nblk);
        int sum = 0;
        for (int b = b0; b < b1; ++b) sum += s_blk[b * E + e];
        s_seg[t] = sum;
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += blockDim.x) {
        int run = 0;
        for (int sg = 0; sg < nseg; ++sg) {
            const int c = s_seg[sg * E + e];
            s_seg[sg * E + e] = run;
            run += c;
        }
        s_cnt[e] = run;
    }
    __syncthreads();
    for (int t = threadIdx.x; t < E * nseg; t += blockDim.x) {
        const int e = t % E, sg = t / E;
        const int b0 = sg * seg_len, b1 = min(b0 + seg_len, nblk);
        int run = s_seg[t];
        for (int b = b0; b < b1; ++b) {
            const int c = s_blk[b * E + e];
            s_blk[b * E + e] = run;
            run += c;
        }
    }
    if (wave_id() == 0) scan_counts_wave0(s_cnt, s_cur, E, bm, counts, offsets, act_list, tile_off, meta);
    __syncthreads();
    for (int i = threadIdx.x; i < n; i += blockDim.x) blk[i] = s_blk[i] + s_cur[i % E];
}

// Large P, pass 3: one wavefront per chunk scatters its pairs stably from its cursors.
__global__ void __launch_bounds__(64) permute_scatter(const int32_t* __restrict__ idx, int P, int E, int chunk,
                                                      const int32_t* __restrict__ blk, int32_t* __restrict__ perm,
                                                      int32_t* __restrict__ inv) {
    __shared__ int s_cur[MOE_MAX_E];
    for (int e = threadIdx.x; e < E; e += blockDim.x) s_cur[e] = blk[(int64_t)blockIdx.x * E + e];
    __syncthreads();
    const int p0 = blockIdx.x * chunk, p1 = min(p0 + chunk, P);
    stable_scatter_wave(idx, p0, p1, bits_for(E), E, s_cur, perm, inv);
}

// From caller-provided offsets (moe_grouped_ffn): the active-expert list, tile offsets, meta.
__global__ void __launch_bounds__(256) active_from_offsets(const int32_t* __restrict__ offsets, int E, int bm,
                                                           int32_t* act_list, int32_t* tile_off, int32_t* meta) {
    __shared__ int s_cnt[MOE_MAX_E];
    for (int e = threadIdx.x; e < E; e += blockDim.x) {
        const int c = offsets[e + 1] - offsets[e];
        s_cnt[e] = c > 0 ? c : 0;
    }
    __syncthreads();
    if (wave_id() == 0) scan_counts_wave0(s_cnt, nullptr, E, bm, nullptr, nullptr, act_list, tile_off, meta);
}

hipError_t launch_active_from_offsets(const int32_t* offsets, int E, int bm, int32_t* act_list, int32_t* tile_off,
                                      int32_t* meta, hipStream_t st) {
    hipLaunchKernelGGL(active_from_offsets, dim3(1), dim3(256), 0, st, offsets, E, bm, act_list, tile_off, meta);
    return hipGetLastError();
}

hipError_t launch_permute(const int32_t* idx, int P, int E, int bm, int32_t* counts, int32_t* offsets,
                          int32_t* perm, int32_t* inv, int32_t* act_list, int32_t* tile_off, int32_t* meta,
                          int32_t* blk, hipStream_t st) {
    if (P <= PERMUTE_SMALL_MAX) {
        hipLaunchKernelGGL(permute_small, dim3(1), dim3(256), 0, st, idx, P, E, bm, counts, offsets, perm, inv,
                           act_list, tile_off, meta);
        return hipGetLastError();
    }
    const int chunk = permute_chunk(P, E);
    const int nblk = (P + chunk - 1) / chunk;
    hipLaunchKernelGGL(permute_hist, dim3(nblk), dim3(256), 0, st, idx, P, E, chunk, blk);
    hipLaunchKernelGGL(permute_scan, dim3(1), dim3(1024), 0, st, blk, nblk, E, bm, counts, offsets, act_list,
                       tile_off, meta);
    hipLaunchKernelGGL(permute_scatter, dim3(nblk), dim3(64), 0, st, idx, P, E, chunk, blk, perm, inv);
    return hipGetLastError();
}

}  // namespace moe
