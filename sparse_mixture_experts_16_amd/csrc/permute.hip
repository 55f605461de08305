// Grouping tokens by expert: a stable counting sort of the flat (token, slot) pairs
// p = t*k + j by expert id, with an LDS histogram, a prefix scan and a stable scatter
// (large batches: per-chunk histograms, then one kernel that scans and scatters).
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
// (meta[0] = active experts, meta[1] = tiles); leaves s_cur[e] = offsets[e].  Lane l handles
// experts l*per .. l*per+per-1 (per = ceil(E/64)).  Null outputs are skipped.
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
        if (tile_off) tile_off[e] = pt;
        if (c > 0 && act_list) act_list[pa] = e;
        pa += (c > 0);
        pc += c;
        pt += (c + bm - 1) / bm;
    }
    if (lane == MOE_WAVE - 1) {
        if (offsets) offsets[E] = pc;
        if (tile_off) tile_off[E] = pt;
        if (meta) {
            meta[0] = pa;
            meta[1] = pt;
        }
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

// Large P, pass 2: one workgroup per chunk.  Every workgroup reads all nblk x E chunk counts
// (consecutive threads take consecutive experts, so the reads are coalesced) and forms each
// expert's total and the part of it in the chunks before its own; wave 0 scans the totals into
// the expert offsets and adds its chunk's prefix.  The chunk is cut into one contiguous piece
// per wavefront; each wavefront counts its piece's pairs per expert, the counts are turned into
// per-piece cursors (the pieces in order), and every wavefront scatters its piece stably from
// its own cursors.  Workgroup 0 also writes counts, offsets, the active-expert list, tile
// offsets and meta.  (Integer sums: the LDS atomics that gather them cannot change them.)
constexpr int PERMUTE_SCATTER_THREADS = 512;
constexpr int PERMUTE_WAVES = PERMUTE_SCATTER_THREADS / MOE_WAVE;
constexpr int PERMUTE_BATCH = 32;  // chunk counts per thread in flight at once
__global__ void __launch_bounds__(PERMUTE_SCATTER_THREADS) permute_scatter(
    const int32_t* __restrict__ idx, int P, int E, int chunk, int nblk, int bm, const int32_t* __restrict__ blk,
    int32_t* counts, int32_t* offsets, int32_t* act_list, int32_t* tile_off, int32_t* meta,
    int32_t* __restrict__ perm, int32_t* __restrict__ inv) {
    __shared__ int s_tot[MOE_MAX_E];
    __shared__ int s_pre[MOE_MAX_E];
    __shared__ int s_cur[MOE_MAX_E];
    __shared__ int s_wcur[PERMUTE_WAVES][MOE_MAX_E];  // per-piece counts, then cursors
    const int tid = threadIdx.x, b = blockIdx.x, wv = wave_id(), lane = lane_id();
    for (int e = tid; e < E; e += blockDim.x) {
        s_tot[e] = 0;
        s_pre[e] = 0;
    }
    for (int i = tid; i < PERMUTE_WAVES * E; i += blockDim.x) s_wcur[i / E][i % E] = 0;
    __syncthreads();
    // (expert, part) items: each part covers a contiguous run of L chunks of one expert
    const int np = E >= (int)blockDim.x ? 1 : (int)blockDim.x / E;
    const int L = (nblk + np - 1) / np;
    for (int s = tid; s < E * np; s += blockDim.x) {
        const int e = s % E, q0 = (s / E) * L, q1 = min(q0 + L, nblk);
        int tot = 0, pre = 0;
        for (int qb = q0; qb < q1; qb += PERMUTE_BATCH) {
            int c[PERMUTE_BATCH];
#pragma unroll
            for (int j = 0; j < PERMUTE_BATCH; ++j) {
                const int q = qb + j;
                c[j] = q < q1 ? blk[(int64_t)q * E + e] : 0;
            }
#pragma unroll
            for (int j = 0; j < PERMUTE_BATCH; ++j) {
                tot += c[j];
                pre += (qb + j < b) ? c[j] : 0;
            }
        }
        if (np == 1) {
            s_tot[e] = tot;
            s_pre[e] = pre;
        } else {
            atomicAdd(&s_tot[e], tot);
            atomicAdd(&s_pre[e], pre);
        }
    }
    // this wavefront's piece of the chunk, and its pairs per expert
    const int p0 = b * chunk, p1 = min(p0 + chunk, P);
    const int piece = (chunk / PERMUTE_WAVES + MOE_WAVE - 1) / MOE_WAVE * MOE_WAVE;
    const int w0 = min(p0 + wv * piece, p1), w1 = min(w0 + piece, p1);
    for (int p = w0 + lane; p < w1; p += MOE_WAVE) {
        const int e = idx[p];
        if ((unsigned)e < (unsigned)E) atomicAdd(&s_wcur[wv][e], 1);
    }
    __syncthreads();
    if (wv == 0) {
        const bool first = b == 0;
        scan_counts_wave0(s_tot, s_cur, E, bm, first ? counts : nullptr, first ? offsets : nullptr,
                          first ? act_list : nullptr, first ? tile_off : nullptr, first ? meta : nullptr);
        // the lane that wrote s_cur[e] (experts lane*per ..) adds this chunk's prefix
        const int per = (E + MOE_WAVE - 1) / MOE_WAVE, lo = min(lane * per, E), hi = min(lo + per, E);
        for (int e = lo; e < hi; ++e) s_cur[e] += s_pre[e];
    }
    __syncthreads();
    // per-piece cursors: the chunk's cursor plus the pairs of the pieces before
    for (int e = tid; e < E; e += blockDim.x) {
        int run = s_cur[e];
#pragma unroll
        for (int w = 0; w < PERMUTE_WAVES; ++w) {
            const int c = s_wcur[w][e];
            s_wcur[w][e] = run;
            run += c;
        }
    }
    __syncthreads();
    stable_scatter_wave(idx, w0, w1, bits_for(E), E, s_wcur[wv], perm, inv);
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
    hipLaunchKernelGGL(permute_scatter, dim3(nblk), dim3(PERMUTE_SCATTER_THREADS), 0, st, idx, P, E, chunk, nblk, bm,
                       blk, counts, offsets, act_list, tile_off, meta, perm, inv);
    return hipGetLastError();
}

}  // namespace moe
