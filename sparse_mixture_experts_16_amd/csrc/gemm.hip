// Prefill path (router logits and the expert FFNs at large T): grouped GEMM on the gfx950 matrix cores.
//
// At prefill thousands of tokens reach nearly every expert (dothoosh.com FreeToken article,
// "FreeToken architecture and the sparsity puzzle", first failure mode), so each expert's
// weights are read once and reused across all of its tokens: this is a dense contraction per
// expert and belongs on MFMA.  One kernel template covers three products:
//
//   MODE_W13     a[pos, j] = silu(x_t . Wg_e[j]) * (x_t . Wu_e[j])   A rows gathered via perm
//   MODE_W2      y[pos, n] = a[pos] . W2_e[n]                          A rows contiguous
//   MODE_ROUTER  l[t, e]   = x_t . W_r[e] + b[e]                       one group, fp32 out
//
// The tile shape, operand layouts and K pipeline are described above the kernel template below.
// For MODE_W13 the LDS B tile interleaves gate rows and the matching up rows per wavefront
// column, so the SwiGLU pairs meet in the same lane and the activation is fused into the
// epilogue.
//
// Tile order: a flat list over (group, m-tile, n-tile), n fastest, built per workgroup from
// the expert offsets; workgroup b (on XCD b % 8) takes entry b / 8 of the (b % 8)-th eighth of
// the list, so that each of the 8 XCDs walks an equal contiguous stretch and an expert's weight
// tiles are shared in that XCD's L2.
#include "common.h"
#include "kernels.h"
#include "lds_dma.h"
#include "wchunk.h"

namespace moe {

constexpr int TBM = 128;
enum { MODE_W13 = 0, MODE_W2 = 1, MODE_ROUTER = 2 };

struct GemmArgs {
    const uint16_t* A;        // W13/ROUTER: x [T, d]; W2: a hi plane (routed [P, f], shared at +P*f as [T, fs])
    const int32_t* perm;      // W13: sorted slot -> pair
    const int32_t* offsets;   // [E+1] (W13/W2)
    const uint8_t* w;         // routed weights (ROUTER: W_r [E, d] bf16)
    const uint8_t* wsc;       // routed MXFP4 scales
    const uint8_t* sw;        // shared expert weights
    const uint8_t* swsc;
    const float* bias;        // ROUTER: b [E] or NULL
    void* out;                // W13: a hi plane (bf16); W2: y (bf16) [P, d]; ROUTER: logits (f32) [T, E]
    uint16_t* out_sh;         // W2: y_shared [T, d]
    int64_t lo_off;           // elements from the a hi plane to the a lo plane
    int T, d, f, fs, k, E, n_shared;
    const uint8_t* mask;      // nullable [E + 1]: groups whose byte is 0 get no tiles
    int ksplit;               // ROUTER: K split over this many workgroups (fp32 partials, no bias) when > 1
};

__device__ __forceinline__ uint32_t cvt2(uint32_t w, float sc, int sel) {
    bf16x2_t v;
    switch (sel) {
        case 0: v = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 0); break;
        case 1: v = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 1); break;
        case 2: v = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 2); break;
        default: v = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 3); break;
    }
    return __builtin_bit_cast(uint32_t, v);
}

// 8 E2M1 codes (one 32-bit word) -> 8 bf16 (uint4); a 0xFF scale gives NaN.
__device__ __forceinline__ uint4 fp4x8_to_bf16(uint32_t w, uint32_t s) {
    const float sc = e8m0_to_f32(s);
    uint4 r;
    r.x = cvt2(w, sc, 0);
    r.y = cvt2(w, sc, 1);
    r.z = cvt2(w, sc, 2);
    r.w = cvt2(w, sc, 3);
    if (s == 255u) r = make_uint4(0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u);
    return r;
}

// Tile: BM = 128 token rows x BN weight rows, K in steps of BK = 32, 256 threads as 2 x 2
// wavefronts each owning 64 x BN/2 with v_mfma_f32_32x32x16_bf16 (A lane l: row l%32,
// k = 8*(l/32)..+7; B lane l: column l%32, same k; accumulator j of lane l: row
// 8*(j/4) + 4*(l/32) + j%4, column l%32).
//
// K pipeline: a ring of NS LDS stages filled straight from HBM by global_load_lds_dwordx4
// (each lane's 16 bytes land at the wave's LDS base + 16 * lane; no register staging).  With
// three stages, while stage kt is consumed, stages kt+1 and kt+2 are in flight; the wait for
// stage kt is a vmcnt(n) that still lets the next stage's loads be outstanding, followed by a
// bare s_barrier, so the compiler's full vmcnt(0) of __syncthreads never drains the pipe.  With
// two stages (the down projection's 256-column tiles, whose two A planes and 256 B rows would
// not fit three deep at two workgroups per CU), stage kt+1 loads while stage kt is consumed.
// Tile rows are 64 bytes (32 bf16) unpadded; 16-byte chunk c of row r sits at physical chunk
// c ^ (((r >> 1) ^ (r >> 2)) & 3), which spreads every 8 (and 16) consecutive rows' fragment
// reads over distinct banks.
// MXFP4 weights: the 16 code bytes of a row's 32-element block go to LDS as they are, one
// chunk per row; each B fragment (8 codes, one dword) is expanded at read time with the
// scaled bf16 converts (exact: E2M1 x 2^k fits bf16).  The E8M0 scales travel as one dword
// (4 consecutive blocks) per row every fourth stage into a double-buffered LDS row list.
// SPLIT: the A operand comes as two bf16 planes a = hi + lo (lo = a - hi rounded to bf16), and
// every B fragment is applied to both, so the fp32 SwiGLU output keeps ~16 significant bits
// through the bf16 matrix cores.
typedef __bf16 bf16x8v __attribute__((ext_vector_type(8)));

template <int MODE, int WT, int BN, bool SPLIT, int NWN, int NS = 3>
__global__ void __launch_bounds__(128 * NWN, NWN == 4 ? 1 : 2) ggemm(GemmArgs p) {  // 2 waves per SIMD: <= 256 registers
    constexpr int BM = TBM, BK = 32;
    static_assert(NS == 2 || NS == 3, "ring depth");
    constexpr int THREADS = 128 * NWN;              // 2 wavefronts along M x NWN along N
    constexpr int NPL = SPLIT ? 2 : 1;              // A planes
    constexpr int WN = BN / NWN;                    // wave tile columns
    constexpr int NT32 = WN / 32;                   // 32-wide MFMA column tiles per wave (2 or 4)
    constexpr int ROWE = BK;                        // bf16 elements per LDS tile row (64 B)
    constexpr int BROW = (WT == 1) ? 32 : 8;        // uint16 per LDS B row (bf16: 64 B, MXFP4 codes: 16 B)
    constexpr int NA = BM * 4 / THREADS;            // A chunks per thread per plane
    constexpr int NB = (WT == 1) ? BN * 4 / THREADS : (BN + THREADS - 1) / THREADS;  // B chunks per thread (max)
    static_assert(NA >= 1 && (WT != 1 || NB >= 1), "tile / thread count");
    // vector-memory ops one stage adds per thread, counted for the wave that issues the fewest
    constexpr int OPS = NPL * NA + ((WT == 1) ? NB : (BN >= THREADS ? 1 : 0));
    static_assert(OPS < 16, "vmcnt immediate");
    // One LDS object carved by offsets.  Fragment reads are loads of plain (vector) types: the
    // compiler's wait insertion drains every LDS-DMA load in flight before an LDS read that carries
    // no type-based alias information; LDS-DMA completion is left to the explicit vmcnt waits below.
    constexpr int SZ_A = NS * NPL * BM * ROWE * 2, SZ_B = NS * BN * BROW * 2, SZ_S = (WT == 2 ? 2 * BN * 4 : 0);
    // output staging after the K loop (reuses the ring): bf16 rows of NCOL columns, pitch OP
    constexpr int NCOL = (MODE == MODE_W13) ? BN / 2 : BN, OP = NCOL + 8;
    constexpr int SZ_O = (MODE == MODE_ROUTER) ? 0 : BM * OP * 2;  // one bf16 plane at a time
    constexpr int SZ_RING = (SZ_A + SZ_B + SZ_S) > SZ_O ? (SZ_A + SZ_B + SZ_S) : SZ_O;
    __shared__ __attribute__((aligned(16))) uint8_t smem[SZ_RING + (MOE_MAX_E + 2) * 4];
    auto sA = reinterpret_cast<uint16_t(*)[NPL][BM * ROWE]>(smem);
    auto sB = reinterpret_cast<uint16_t(*)[BN * BROW]>(smem + SZ_A);
    auto sS = reinterpret_cast<uint32_t(*)[BN]>(smem + SZ_A + SZ_B);
    int* s_pref = reinterpret_cast<int*>(smem + SZ_RING);

    const int tid = threadIdx.x, lane = tid & 63, wv = wave_id(), wm = wv / NWN, wn = wv % NWN;
    const int G = (MODE == MODE_ROUTER) ? 1 : p.E + p.n_shared;
    const int P = p.T * p.k;

    // ---- flat tile list: tiles of group g = ceil(rows_g / BM) * ntiles_g
    auto tiles_of = [&](int g) -> int {
        int rows, nt;
        if (MODE == MODE_ROUTER) {
            rows = p.T;
            nt = (p.E + BN - 1) / BN * p.ksplit;
        } else {
            const bool sh = g == p.E;
            rows = (p.mask && !p.mask[g]) ? 0 : (sh ? p.T : p.offsets[g + 1] - p.offsets[g]);
            nt = (MODE == MODE_W13) ? ((sh ? p.fs : p.f) + BN / 2 - 1) / (BN / 2) : (p.d + BN - 1) / BN;
        }
        return ((rows + BM - 1) / BM) * nt;
    };
    if (wv == 0) {
        const int per = (G + 63) / 64;
        const int lo = min(lane * per, G), hi = min(lo + per, G);
        int sum = 0;
        for (int g = lo; g < hi; ++g) sum += tiles_of(g);
        int incl = sum;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            int u = __shfl_up(incl, o, 64);
            if (lane >= o) incl += u;
        }
        int run = incl - sum;
        for (int g = lo; g < hi; ++g) {
            s_pref[g] = run;
            run += tiles_of(g);
        }
        if (lane == 63) s_pref[G] = incl;
    }
    __syncthreads();

    // workgroup b runs on XCD b % 8; XCD x takes the x-th eighth of the actual list (the grid is
    // only a bound on its length), so all eight share the work and each walks a contiguous stretch
    const int total = s_pref[G];
    const int xcd = blockIdx.x & 7, j = blockIdx.x >> 3;  // gridDim.x / 8 >= ceil(total / 8)
    const int t_lo = (int)(((int64_t)total * xcd) >> 3), t_hi = (int)(((int64_t)total * (xcd + 1)) >> 3);
    if (t_lo + j >= t_hi) return;
    const int L = t_lo + j;
    int g = 0;
    {
        int lo = 0, hi = G;
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (s_pref[mid] <= L) lo = mid;
            else hi = mid;
        }
        g = lo;
    }
    const bool shared = (MODE != MODE_ROUTER) && g == p.E;
    const int fg = shared ? p.fs : p.f;
    int rows_g, base, ntiles, K, N;
    const uint8_t* W;
    const uint8_t* WS;
    if (MODE == MODE_ROUTER) {
        rows_g = p.T; base = 0; K = p.d; N = p.E; ntiles = (p.E + BN - 1) / BN;
        W = p.w; WS = nullptr;
    } else {
        rows_g = shared ? p.T : p.offsets[g + 1] - p.offsets[g];
        base = shared ? 0 : p.offsets[g];
        if (MODE == MODE_W13) { K = p.d; N = 2 * fg; ntiles = (fg + BN / 2 - 1) / (BN / 2); }
        else { K = fg; N = p.d; ntiles = (p.d + BN - 1) / BN; }
        const int64_t rb = row_bytes(WT, K), sb = K / 32;
        W = shared ? p.sw : p.w + (int64_t)g * N * rb;
        WS = (WT == 2) ? (shared ? p.swsc : p.wsc + (int64_t)g * N * sb) : nullptr;
    }
    int local = L - s_pref[g];
    int ks = 0;
    if (MODE == MODE_ROUTER && p.ksplit > 1) {
        ks = local % p.ksplit;
        local /= p.ksplit;
        K /= p.ksplit;
    }
    const int mt = local / ntiles, nt = local % ntiles;
    const int m0 = mt * BM;
    const int mrows = min(BM, rows_g - m0);
    const int64_t wrb = row_bytes(WT, K * (MODE == MODE_ROUTER ? p.ksplit : 1)), wsb = K / 32;

    // ---- this thread's global sources.  A chunk slot s = i*256 + tid holds row s/4 at physical
    // chunk s%4; rows past the group's end re-read the tile's first row (their results are
    // never stored).
    const int pc = tid & 3;
    const uint16_t* asrc[NA];
#pragma unroll
    for (int i = 0; i < NA; ++i) {
        int r = i * (THREADS / 4) + (tid >> 2);
        const int c = pc ^ chunk_swz(r);
        if (r >= mrows) r = 0;
        int64_t src;
        if (MODE == MODE_W13) src = shared ? (int64_t)(m0 + r) * p.d : (int64_t)(p.perm[base + m0 + r] / p.k) * p.d;
        else if (MODE == MODE_W2) src = shared ? (int64_t)P * p.f + (int64_t)(m0 + r) * p.fs : (int64_t)(base + m0 + r) * p.f;
        else src = (int64_t)(m0 + r) * p.d;
        asrc[i] = p.A + src + (int64_t)ks * K + c * 8;
    }
    // LDS B row n -> weight row.  Gate/up: each wavefront column holds BN/4 gate rows and the
    // matching BN/4 up rows, so SwiGLU pairs meet in the same lane.  Rows past the end map to
    // weight row 0 (their columns are never stored).
    auto wrow_of = [&](int n) -> int {
        if (MODE == MODE_W13) {
            constexpr int H = BN / (2 * NWN);
            const int j0 = nt * (BN / 2), h = n / (2 * H), w = n % (2 * H);
            const int j = j0 + h * H + (w < H ? w : w - H);
            if (j >= fg) return 0;
            return w < H ? j : fg + j;
        }
        const int r = nt * BN + n;
        return r < N ? r : 0;
    };
    const uint8_t* bsrc[NB];
    const uint8_t* ssrc = nullptr;
    bool b_on = true, s_on = false;
    if (WT == 1) {
#pragma unroll
        for (int i = 0; i < NB; ++i) {
            const int n = i * (THREADS / 4) + (tid >> 2);
            bsrc[i] = W + (int64_t)wrow_of(n) * wrb + (int64_t)ks * K * 2 + (pc ^ chunk_swz(n)) * 16;
        }
    } else {
        // one 16-byte code chunk (the 32-element block) per B row; BN = 128 uses waves 0-1
        b_on = tid < BN;
        s_on = tid < BN;
        const int wr = wrow_of(b_on ? tid : 0);
        bsrc[0] = W + (int64_t)wr * wrb;
        ssrc = WS + (int64_t)wr * wsb;
    }

    auto issue = [&](int kt) {
        const int st = kt % NS;
        const int k0 = kt * BK;
#pragma unroll
        for (int i = 0; i < NA; ++i) {
            uint16_t* dA = &sA[st][0][(i * THREADS + wv * 64) * 8];
            dma16(asrc[i] + k0, dA);
            if (SPLIT) dma16(asrc[i] + p.lo_off + k0, &sA[st][NPL - 1][(i * THREADS + wv * 64) * 8]);
        }
        if (WT == 1) {
#pragma unroll
            for (int i = 0; i < NB; ++i)
                dma16(bsrc[i] + (int64_t)k0 * 2, &sB[st][(i * THREADS + wv * 64) * 8]);
        } else {
            if (b_on) dma16(bsrc[0] + k0 / 2, &sB[st][wv * 64 * 8]);
            if (s_on && (kt & 3) == 0)
                dma4(ssrc + kt, &sS[(kt >> 2) & 1][wv * 64]);
        }
    };

    f32x16_t acc[2][NT32];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < NT32; ++b)
#pragma unroll
            for (int j = 0; j < 16; ++j) acc[a][b][j] = 0.0f;

    // fragment addresses: rows r = (multiple of 32) + lane%32 all share chunk_swz(lane%32)
    const int l32 = lane & 31, hk = lane >> 5;
    const int fc0 = ((0 + hk) ^ chunk_swz(l32)) * 8, fc1 = ((2 + hk) ^ chunk_swz(l32)) * 8;

    const int nk = K / BK;
    // a wavefront whose 64 rows all lie past the group's end only loads and synchronises; its
    // matrix-core time goes to the other workgroup on the CU
    const bool live = wm * 64 < mrows;
    issue(0);
    if (NS == 3 && nk > 1) issue(1);
    for (int kt = 0; kt < nk; ++kt) {
        const int st = kt % NS;
        asm volatile("" ::: "memory");
        // three stages: stage kt + 1 stays in flight; two: every wait drains the ring
        if (NS == 3 && kt + 1 < nk) VM_WAIT(OPS);
        else VM_WAIT(0);
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        if (kt + NS - 1 < nk) issue(kt + NS - 1);
        if (!live) continue;

        uint32_t sc_w[NT32];
        if (WT == 2) {
#pragma unroll
            for (int ns = 0; ns < NT32; ++ns) sc_w[ns] = sS[(kt >> 2) & 1][wn * WN + ns * 32 + l32];
        }
#pragma unroll
        for (int kk = 0; kk < BK / 16; ++kk) {
            const int fc = kk ? fc1 : fc0;
            bf16x8v bfr[NT32];
#pragma unroll
            for (int ns = 0; ns < NT32; ++ns) {
                const int n = wn * WN + ns * 32 + l32;
                if (WT == 1) {
                    bfr[ns] = __builtin_bit_cast(bf16x8v, *reinterpret_cast<const uint4*>(&sB[st][n * BROW + fc]));
                } else {
                    const uint32_t cw = *reinterpret_cast<const uint32_t*>(&sB[st][n * BROW + kk * 4 + hk * 2]);
                    const uint32_t s8 = (sc_w[ns] >> (8 * (kt & 3))) & 0xFFu;
                    bfr[ns] = __builtin_bit_cast(bf16x8v, fp4x8_to_bf16(cw, s8));
                }
            }
#pragma unroll
            for (int pl = 0; pl < NPL; ++pl) {
                bf16x8v af[2];
#pragma unroll
                for (int ms = 0; ms < 2; ++ms)
                    af[ms] = __builtin_bit_cast(bf16x8v, *reinterpret_cast<const uint4*>(
                        &sA[st][pl][(wm * 64 + ms * 32 + l32) * ROWE + fc]));
#pragma unroll
                for (int ms = 0; ms < 2; ++ms)
#pragma unroll
                    for (int ns = 0; ns < NT32; ++ns)
                        acc[ms][ns] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[ms], bfr[ns], acc[ms][ns], 0, 0, 0);
            }
        }
    }

    // ---- epilogue: accumulator j of lane l is row 8*(j/4) + 4*(l/32) + j%4, column l%32
    if constexpr (MODE == MODE_ROUTER) {
#pragma unroll
        for (int ms = 0; ms < 2; ++ms)
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const int r = wm * 64 + ms * 32 + (j >> 2) * 8 + (lane >> 5) * 4 + (j & 3);
                if (r >= mrows) continue;
                float* o = reinterpret_cast<float*>(p.out) + ((int64_t)ks * p.T + m0 + r) * p.E;
                const bool part = p.ksplit > 1;
#pragma unroll
                for (int ns = 0; ns < NT32; ++ns) {
                    const int n = nt * BN + wn * WN + ns * 32 + (lane & 31);
                    if (n < N) o[n] = acc[ms][ns][j] + (!part && p.bias ? p.bias[n] : 0.0f);
                }
            }
    } else {
        // Stage the tile's bf16 outputs in LDS (the ring is free once every wavefront is past
        // its last fragment read), one plane at a time, then store whole 16-byte row chunks.
        uint16_t* o_st = reinterpret_cast<uint16_t*>(smem);
        if constexpr (MODE == MODE_W13) {
            // SwiGLU in place of the gate accumulators
#pragma unroll
            for (int ms = 0; ms < 2; ++ms)
#pragma unroll
                for (int ns = 0; ns < NT32 / 2; ++ns)
#pragma unroll
                    for (int j = 0; j < 16; ++j) {
                        const float gt = acc[ms][ns][j], up = acc[ms][ns + NT32 / 2][j];
                        acc[ms][ns][j] = silu_hw(gt) * up;
                    }
        }
        constexpr int CH = NCOL / 8;  // 16-byte chunks per staged row
        const int col0 = nt * NCOL;
        const int lim = (MODE == MODE_W13) ? fg : N;  // columns of this group's output rows
#pragma unroll
        for (int pl = 0; pl < (MODE == MODE_W13 ? 2 : 1); ++pl) {
            __syncthreads();
#pragma unroll
            for (int ms = 0; ms < 2; ++ms)
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    const int r = wm * 64 + ms * 32 + (j >> 2) * 8 + (lane >> 5) * 4 + (j & 3);
                    if constexpr (MODE == MODE_W13) {
#pragma unroll
                        for (int ns = 0; ns < NT32 / 2; ++ns) {
                            const float av = acc[ms][ns][j];
                            const uint16_t hi = f32_to_bf16(av);
                            o_st[r * OP + wn * (WN / 2) + ns * 32 + (lane & 31)] =
                                pl == 0 ? hi : f32_to_bf16(av - bf16_to_f32(hi));
                        }
                    } else {
#pragma unroll
                        for (int ns = 0; ns < NT32; ++ns) o_st[r * OP + wn * WN + ns * 32 + (lane & 31)] = f32_to_bf16(acc[ms][ns][j]);
                    }
                }
            __syncthreads();
            for (int i = tid; i < BM * CH; i += THREADS) {
                const int r = i / CH, ch = i % CH;
                if (r >= mrows || col0 + ch * 8 >= lim) continue;
                const int row = m0 + r;
                const uint4 v = *reinterpret_cast<const uint4*>(&o_st[r * OP + ch * 8]);
                uint16_t* o;
                if constexpr (MODE == MODE_W13)
                    o = reinterpret_cast<uint16_t*>(p.out) + (pl ? p.lo_off : 0) +
                        (shared ? (int64_t)P * p.f + (int64_t)row * p.fs : (int64_t)(base + row) * p.f) + col0 + ch * 8;
                else
                    o = (shared ? p.out_sh + (int64_t)row * p.d
                                : reinterpret_cast<uint16_t*>(p.out) + (int64_t)(base + row) * p.d) + col0 + ch * 8;
                *reinterpret_cast<uint4*>(o) = v;
            }
        }
    }
}

static unsigned grid8(int64_t tiles) {
    int64_t g = (tiles + 7) / 8 * 8;
    return (unsigned)(g < 8 ? 8 : g);
}

// Router partial sums of a K split, added in split order (then the bias): deterministic.
__global__ void __launch_bounds__(256) router_reduce(const float* __restrict__ part, const float* __restrict__ b,
                                                     float* __restrict__ logits, int64_t n, int E, int ks) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
        float v = 0.0f;
        for (int q = 0; q < ks; ++q) v += part[(int64_t)q * n + i];
        logits[i] = v + (b ? b[i % E] : 0.0f);
    }
}

hipError_t launch_route_logits_mfma(const void* x, const void* wr, const float* b, float* logits, int T, int d,
                                    int E, float* part, size_t part_bytes, hipStream_t st) {
    // T/128 x E/128 tiles alone leave most CUs idle: split K (>= 4 steps of 32 each) over up to 8
    // workgroups when the partials fit the scratch given, but not beyond one round of the device's
    // workgroup slots (two per CU): a second round and its larger partials cost more than they
    // save (c3 prefill router 53 + 15 us at 8 ways against 41 + 10 us at 4).
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
        cus = 256;
    const int64_t slots = 2 * (int64_t)cus;
    const int64_t tiles = (int64_t)((T + TBM - 1) / TBM) * ((E + 127) / 128);
    int ks = 1;
    while (ks < 8 && tiles * ks * 2 <= slots && d % (32 * ks * 2) == 0 && d / (ks * 2) >= 128 &&
           (size_t)ks * 2 * T * E * 4 <= part_bytes)
        ks *= 2;
    GemmArgs p{};
    p.A = (const uint16_t*)x;
    p.w = (const uint8_t*)wr;
    p.bias = b;
    p.out = ks > 1 ? (void*)part : (void*)logits;
    p.T = T; p.d = d; p.E = E; p.k = 1;
    p.ksplit = ks;
    hipLaunchKernelGGL((ggemm<MODE_ROUTER, 1, 128, false, 2>), dim3(grid8(tiles * ks)), dim3(256), 0, st, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || ks == 1) return e;
    const int64_t n = (int64_t)T * E;
    const unsigned grid = (unsigned)((n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096);
    hipLaunchKernelGGL(router_reduce, dim3(grid), dim3(256), 0, st, part, b, logits, n, E, ks);
    return hipGetLastError();
}

// The SwiGLU activation is stored as two bf16 planes (hi, then lo) of P*f + T*fs elements each.
static int64_t a_lo_offset(int T, int k, int f, int fs, int n_shared) {
    return (int64_t)T * k * f + (n_shared ? (int64_t)T * fs : 0);
}

static int64_t max_tiles(int T, int k, int E, int n_shared, int rows_nt, int shared_nt) {
    const int64_t P = (int64_t)T * k;
    const int64_t routed_mt = (P + TBM - 1) / TBM + (P < E ? P : E);
    const int64_t shared_mt = n_shared ? (T + TBM - 1) / TBM : 0;
    return routed_mt * rows_nt + shared_mt * shared_nt;
}

hipError_t launch_ggemm_w13(int wt, const uint16_t* x, const int32_t* perm, const int32_t* offsets,
                            const int32_t*, const int32_t*, const void* w13, const uint8_t* w13s, const void* s13,
                            const uint8_t* s13s, uint16_t* a, int T, int d, int f, int fs, int k, int E, int n_shared,
                            const uint8_t* mask, hipStream_t st) {
    GemmArgs p{x, perm, offsets, (const uint8_t*)w13, w13s, (const uint8_t*)s13, s13s, nullptr, a, nullptr,
               a_lo_offset(T, k, f, fs, n_shared), T, d, f, fs, k, E, n_shared, mask, 1};
    if (wt == 2 && f % 256 == 0 && (!n_shared || fs % 256 == 0)) {
        // MXFP4 weights: 16 code bytes per row and stage, so a 128 x 512 tile (8 wavefronts, one
        // workgroup per CU) halves the activation reads per weight row at little LDS cost
        constexpr int BN = 512, NWN = 4;
        const unsigned grid = grid8(max_tiles(T, k, E, n_shared, f / (BN / 2), n_shared ? fs / (BN / 2) : 0));
        MOE_LAUNCH(PROF_FFN_UP, (ggemm<MODE_W13, 2, BN, false, NWN>), dim3(grid), dim3(128 * NWN), 0, st, p);
        return hipGetLastError();
    }
    constexpr int BN = 256, NWN = 2;  // 128 gate/up column pairs per tile, 4 wavefronts
    const unsigned grid = grid8(max_tiles(T, k, E, n_shared, (f + BN / 2 - 1) / (BN / 2), n_shared ? (fs + BN / 2 - 1) / (BN / 2) : 0));
    if (wt == 1) MOE_LAUNCH(PROF_FFN_UP, (ggemm<MODE_W13, 1, BN, false, NWN>), dim3(grid), dim3(128 * NWN), 0, st, p);
    else MOE_LAUNCH(PROF_FFN_UP, (ggemm<MODE_W13, 2, BN, false, NWN>), dim3(grid), dim3(128 * NWN), 0, st, p);
    return hipGetLastError();
}

hipError_t launch_ggemm_w2(int wt, const uint16_t* a, const int32_t* offsets, const int32_t*, const int32_t*,
                           const void* w2, const uint8_t* w2s, const void* s2, const uint8_t* s2s, uint16_t* y,
                           uint16_t* y_shared, int T, int d, int f, int fs, int k, int E, int n_shared,
                           const uint8_t* mask, hipStream_t st) {
    GemmArgs p{a, nullptr, offsets, (const uint8_t*)w2, w2s, (const uint8_t*)s2, s2s, nullptr, y, y_shared,
               a_lo_offset(T, k, f, fs, n_shared), T, d, f, fs, k, E, n_shared, mask, 1};
    constexpr int NWN = 2;
    if (d % 256 == 0) {
        // 256 output columns per tile, two stages (the lo/hi A planes and 256 B rows fill 64 KB
        // per stage pair; two workgroups per CU)
        constexpr int BN = 256;
        const int nt = d / BN;
        const unsigned grid = grid8(max_tiles(T, k, E, n_shared, nt, nt));
        if (wt == 1) MOE_LAUNCH(PROF_FFN_DOWN, (ggemm<MODE_W2, 1, BN, true, NWN, 2>), dim3(grid), dim3(128 * NWN), 0, st, p);
        else MOE_LAUNCH(PROF_FFN_DOWN, (ggemm<MODE_W2, 2, BN, true, NWN, 2>), dim3(grid), dim3(128 * NWN), 0, st, p);
        return hipGetLastError();
    }
    constexpr int BN = 128;
    const int nt = (d + BN - 1) / BN;
    const unsigned grid = grid8(max_tiles(T, k, E, n_shared, nt, nt));
    if (wt == 1) MOE_LAUNCH(PROF_FFN_DOWN, (ggemm<MODE_W2, 1, BN, true, NWN>), dim3(grid), dim3(128 * NWN), 0, st, p);
    else MOE_LAUNCH(PROF_FFN_DOWN, (ggemm<MODE_W2, 2, BN, true, NWN>), dim3(grid), dim3(128 * NWN), 0, st, p);
    return hipGetLastError();
}

}  // namespace moe
