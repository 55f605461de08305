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
#include "mxfp8.h"
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
    void* out;                // W13: a hi plane (bf16); W2: y (bf16 or f32) [P, d]; ROUTER: logits (f32) [T, E]
    void* out_sh;             // W2: y_shared [T, d], the dtype of y
    int64_t lo_off;           // elements from the a hi plane to the a lo plane
    int T, d, f, fs, k, E, n_shared;
    const uint8_t* mask;      // nullable [E + 1]: groups whose byte is 0 get no tiles
    int ksplit;               // ROUTER: K split over this many workgroups (fp32 partials, no bias) when > 1
    uint8_t* lo_q;            // W13 with LOQ, and ggemm_w2q: the lo plane as E4M3 codes (32-column blocks,
    uint8_t* lo_s;            //   as the hi plane) and its E8M0 scales [rows][K/32] (routed rows, then shared)
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

// LDS swizzles of the long-stage tiles: x rows of BK bf16 (128 or 256 bytes), chunk c of row r at
// c ^ a_swz(r); MXFP4 code rows of BK/2 bytes, chunk h of row n at h ^ b_swz(n).  Each spreads
// the rows that 8 consecutive lanes read over distinct banks.
template <int BK>
__device__ __forceinline__ int a_swz(int r) { return BK == 64 ? ((r >> 1) & 7) : (r & 15); }
template <int BK>
__device__ __forceinline__ int b_swz(int n) { return BK == 64 ? ((n >> 3) & 1) : chunk_swz(n); }

// 8 E2M1 codes (one 32-bit word) -> 8 bf16 (uint4).  A 0xFF scale (NaN by the MX rule) is an
// infinite fp32 scale here, and the scaled convert returns NaN for every code under an infinite
// or NaN scale (checked over all 16 codes on gfx950), so the block comes out NaN with no select.
__device__ __forceinline__ uint4 fp4x8_to_bf16(uint32_t w, uint32_t s) {
    const float sc = e8m0_to_f32(s);
    uint4 r;
    r.x = cvt2(w, sc, 0);
    r.y = cvt2(w, sc, 1);
    r.z = cvt2(w, sc, 2);
    r.w = cvt2(w, sc, 3);
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
// KB = 64 or 128 (gate/up): long stages, x rows of 128 or 256 bytes and 2 or 4 MXFP4 code
// chunks per weight row (swizzled by a_swz / b_swz), the scale dword every second or every
// stage; inside each 64 of a stage K is permuted so that MFMA c of lane half h takes
// K = 32h + 8c .. +7: the lane's 32 codes of one block feed four of its MFMAs.  bf16 weight
// rows of 128 bytes are laid out and read as the x rows.  TM = 256 (bf16 gate/up): tiles of
// 256 token rows, 4 x NWN wavefronts.
// SPLIT: the A operand comes as two bf16 planes a = hi + lo (lo = a - hi rounded to bf16), and
// every B fragment is applied to both, so the fp32 SwiGLU output keeps ~16 significant bits
// through the bf16 matrix cores.
typedef __bf16 bf16x8v __attribute__((ext_vector_type(8)));
typedef unsigned v4u_t __attribute__((ext_vector_type(4)));
typedef int v8i_t __attribute__((ext_vector_type(8)));

// YF32 (down projection only): y is written in fp32 straight from the accumulators, so the
// combine that follows sums unrounded expert outputs.
// LOQ (gate/up only): the lo plane is written as MXFP8 (E4M3 codes with an E8M0 scale per 32
// columns) for ggemm_w2q instead of as bf16.
template <int MODE, int WT, int BN, bool SPLIT, int NWN, int NS = 3, bool YF32 = false, bool LOQ = false, int KB = 32,
          int TM = TBM>
__global__ void __launch_bounds__(TM / 64 * 64 * NWN, TM / 64 * NWN >= 8 ? 1 : 2) ggemm(GemmArgs p) {  // <= 256 registers
    constexpr int BM = TM, BK = KB;
    static_assert(TM == 128 || (TM == 256 && KB == 64 && WT == 1), "256-row tiles: bf16 gate/up on 64-element stages");
    // 64-element stages: MXFP4 gate/up only (x rows of 128 bytes, 32 code bytes per weight row)
    static_assert(KB == 32 || ((KB == 64 || (KB == 128 && WT == 2)) && MODE == MODE_W13 && !SPLIT) ||
                      (KB == 64 && MODE == MODE_ROUTER && WT == 1), "stage depth");
    constexpr int SPG = 128 / BK;                   // stages per MXFP4 scale dword (4 blocks of 32)
    constexpr int CPR = BK / 32;                    // MXFP4 code chunks (blocks) per weight row and stage
    static_assert(NS == 2 || NS == 3, "ring depth");
    constexpr int THREADS = BM / 64 * 64 * NWN;     // BM / 64 wavefronts along M x NWN along N
    constexpr int NPL = SPLIT ? 2 : 1;              // A planes
    constexpr int WN = BN / NWN;                    // wave tile columns
    constexpr int NT32 = WN / 32;                   // 32-wide MFMA column tiles per wave (2 or 4)
    constexpr int ROWE = BK;                        // bf16 elements per LDS tile row (64 or 128 B)
    constexpr int BROW = (WT == 1) ? BK : BK / 4;   // uint16 per LDS B row (bf16: 64 or 128 B, MXFP4 codes: 16, 32 or 64 B)
    constexpr int NA = BM * (BK / 8) / THREADS;     // A chunks per thread per plane
    constexpr int NB = (WT == 1) ? BN * (BK / 8) / THREADS : (BN * CPR + THREADS - 1) / THREADS;  // B chunks per thread (max)
    static_assert(BK == 32 || WT == 1 || (BN * CPR) % THREADS == 0, "long stages: every thread loads whole B chunks");
    static_assert(NA >= 1 && (WT != 1 || NB >= 1), "tile / thread count");
    // vector-memory ops one stage adds per thread, counted for the wave that issues the fewest
    constexpr int OPS = NPL * NA + ((WT == 1) ? NB : (BK > 32 ? NB : (BN >= THREADS ? 1 : 0)));
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
    if (wv == 0) wave_tile_prefix<(MOE_MAX_E + 64) / 64>(G, s_pref, tiles_of);
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

    // `a` (the gate/up output, the down projection's A) is stored in 32-column stage blocks: block
    // s of the routed rows holds all P sorted rows' columns 32s .. 32s+31 (64 bytes a row), so a
    // down-projection stage of an m-tile is one contiguous 8 KB run of whole 128-byte lines
    // instead of 128 half-lines of separate rows; the shared expert's T rows follow in fs/32
    // blocks of their own.  a_row0: element of row 0 of the group in block 0; a_blk: elements
    // from one block to the next.
    const int64_t a_row0 = shared ? (int64_t)P * p.f : (int64_t)base * 32;
    const int64_t a_blk = shared ? (int64_t)p.T * 32 : (int64_t)P * 32;

    // ---- this thread's global sources.  A chunk slot s = i*256 + tid holds row s/4 at physical
    // chunk s%4; rows past the group's end re-read the tile's first row (their results are
    // never stored).
    const int pc = tid & 3;
    const uint16_t* asrc[NA];
#pragma unroll
    for (int i = 0; i < NA; ++i) {
        // 64-byte rows: chunk c of row r at c ^ chunk_swz(r); 128-byte rows: at c ^ ((r >> 1) & 7);
        // 256-byte rows: at c ^ (r & 15)
        int r = BK == 32 ? i * (THREADS / 4) + (tid >> 2) : (i * THREADS + tid) / (BK / 8);
        const int c = BK == 32 ? (pc ^ chunk_swz(r)) : ((tid % (BK / 8)) ^ a_swz<BK>(r));
        if (r >= mrows) r = 0;
        int64_t src;
        if (MODE == MODE_W13) src = shared ? (int64_t)(m0 + r) * p.d : (int64_t)(p.perm[base + m0 + r] / p.k) * p.d;
        else if (MODE == MODE_W2) src = a_row0 + (int64_t)(m0 + r) * 32;
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
    if (WT == 1 && BK == 64) {
        // bf16 weight rows of 128 bytes a stage, laid out as the x rows (chunk c at c ^ a_swz(n))
#pragma unroll
        for (int i = 0; i < NB; ++i) {
            const int n = (i * THREADS + tid) >> 3, c = (tid & 7) ^ a_swz<64>(n);
            bsrc[i] = W + (int64_t)wrow_of(n) * wrb + (int64_t)ks * K * 2 + c * 16;
        }
    } else if (WT == 1) {
#pragma unroll
        for (int i = 0; i < NB; ++i) {
            const int n = i * (THREADS / 4) + (tid >> 2);
            bsrc[i] = W + (int64_t)wrow_of(n) * wrb + (int64_t)ks * K * 2 + (pc ^ chunk_swz(n)) * 16;
        }
    } else if (BK > 32) {
        // CPR 16-byte code chunks (32-element blocks) per B row, chunk h of row n at
        // h ^ b_swz(n); the row's scale dword (4 blocks) every SPG stages
#pragma unroll
        for (int i = 0; i < NB; ++i) {
            const int sidx = i * THREADS + tid, n = sidx / CPR, h = (sidx % CPR) ^ b_swz<BK>(n);
            bsrc[i] = W + (int64_t)wrow_of(n) * wrb + h * 16;
        }
        s_on = tid < BN;
        ssrc = WS + (int64_t)wrow_of(s_on ? tid : 0) * wsb;
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
        const int64_t ka = (MODE == MODE_W2) ? (int64_t)kt * a_blk : k0;  // A: the next stage block, else 32 columns on
#pragma unroll
        for (int i = 0; i < NA; ++i) {
            uint16_t* dA = &sA[st][0][(i * THREADS + wv * 64) * 8];
            dma16(asrc[i] + ka, dA);
            if (SPLIT) dma16(asrc[i] + p.lo_off + ka, &sA[st][NPL - 1][(i * THREADS + wv * 64) * 8]);
        }
        if (WT == 1 || BK > 32) {
#pragma unroll
            for (int i = 0; i < NB; ++i)
                dma16(bsrc[i] + (WT == 1 ? (int64_t)k0 * 2 : (int64_t)k0 / 2), &sB[st][(i * THREADS + wv * 64) * 8]);
        } else {
            if (b_on) dma16(bsrc[0] + k0 / 2, &sB[st][wv * 64 * 8]);
        }
        if (WT == 2 && s_on && (kt % SPG) == 0)
            dma4(ssrc + k0 / 32, &sS[(kt / SPG) & 1][wv * 64]);
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
            for (int ns = 0; ns < NT32; ++ns) sc_w[ns] = sS[(kt / SPG) & 1][wn * WN + ns * 32 + l32];
        }
        if constexpr (BK > 32) {
            // long stage, K permuted inside each 64 of it as the down projection's kernel does:
            // MFMA c of 64-group q and lane half h covers K = 64q + 32h + 8c .. +7, so a lane's 32
            // codes (one 16-byte chunk: block 2q + h of the stage) serve four MFMAs, and the A
            // fragment of that MFMA is chunk 8q + 4h + c of the row
            const uint8_t* const sBs = reinterpret_cast<const uint8_t*>(&sB[st][0]);
            const uint8_t* const sAs = reinterpret_cast<const uint8_t*>(&sA[st][0][0]);
            const int blk0 = BK == 64 ? 2 * (kt & 1) : 0;  // the stage's first block in the scale dword
#pragma unroll
            for (int q = 0; q < BK / 64; ++q) {
                v4u_t bq[NT32];
                uint32_t bsc[NT32];
#pragma unroll
                for (int ns = 0; ns < NT32; ++ns) {
                    const int n = wn * WN + ns * 32 + l32;
                    if (WT == 2) {
                        bq[ns] = *reinterpret_cast<const v4u_t*>(sBs + n * (BK / 2) + (((2 * q + hk) ^ b_swz<BK>(n)) * 16));
                        bsc[ns] = (sc_w[ns] >> (8 * (blk0 + 2 * q + hk))) & 0xFFu;
                    }
                }
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    bf16x8v bfr[NT32];
#pragma unroll
                    for (int ns = 0; ns < NT32; ++ns) {
                        const int n = wn * WN + ns * 32 + l32;
                        if (WT == 1)  // bf16 rows: chunk 4h + c, as the x fragment
                            bfr[ns] = __builtin_bit_cast(bf16x8v, *reinterpret_cast<const v4u_t*>(
                                sBs + n * 128 + (((4 * hk + c) ^ a_swz<64>(n)) * 16)));
                        else
                            bfr[ns] = __builtin_bit_cast(bf16x8v, fp4x8_to_bf16(bq[ns][c], bsc[ns]));
                    }
                    bf16x8v af[2];
#pragma unroll
                    for (int ms = 0; ms < 2; ++ms) {
                        const int r = wm * 64 + ms * 32 + l32;
                        af[ms] = __builtin_bit_cast(bf16x8v, *reinterpret_cast<const v4u_t*>(
                            sAs + r * (BK * 2) + (((8 * q + 4 * hk + c) ^ a_swz<BK>(r)) * 16)));
                    }
#pragma unroll
                    for (int ms = 0; ms < 2; ++ms)
#pragma unroll
                        for (int ns = 0; ns < NT32; ++ns)
                            acc[ms][ns] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[ms], bfr[ns], acc[ms][ns], 0, 0, 0);
                }
            }
            continue;
        }
        // MXFP4: every code word of the stage read from LDS up front (the two K halves of a
        // lane's row are 8 bytes apart: one ds_read2 each), then expanded per K half
        uint32_t cw[BK / 16][NT32];
        if (WT == 2) {
#pragma unroll
            for (int ns = 0; ns < NT32; ++ns)
#pragma unroll
                for (int kk = 0; kk < BK / 16; ++kk)
                    cw[kk][ns] = *reinterpret_cast<const uint32_t*>(&sB[st][(wn * WN + ns * 32 + l32) * BROW + kk * 4 + hk * 2]);
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
                    const uint32_t s8 = (sc_w[ns] >> (8 * (kt & 3))) & 0xFFu;
                    bfr[ns] = __builtin_bit_cast(bf16x8v, fp4x8_to_bf16(cw[kk][ns], s8));
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
    } else if constexpr (MODE == MODE_W2 && YF32) {
        // fp32 y from the accumulators: the 32 lanes holding one row write 128 contiguous bytes
#pragma unroll
        for (int ms = 0; ms < 2; ++ms)
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const int r = wm * 64 + ms * 32 + (j >> 2) * 8 + (lane >> 5) * 4 + (j & 3);
                if (r >= mrows) continue;
                const int row = m0 + r;
                float* o = shared ? reinterpret_cast<float*>(p.out_sh) + (int64_t)row * p.d
                                  : reinterpret_cast<float*>(p.out) + (int64_t)(base + row) * p.d;
#pragma unroll
                for (int ns = 0; ns < NT32; ++ns) {
                    const int n = nt * BN + wn * WN + ns * 32 + (lane & 31);
                    if (n < N) o[n] = acc[ms][ns][j];
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
        static_assert(MODE != MODE_W13 || NCOL % 32 == 0, "gate/up tiles cover whole 32-column blocks of a");
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
            if (MODE == MODE_W13 && LOQ && pl == 1) {
                // lo as MXFP8: one thread per (row, 32-column block) of the tile
                for (int i = tid; i < BM * (NCOL / 32); i += THREADS) {
                    const int r = i % BM, sl = i / BM;
                    const int col = col0 + sl * 32;
                    if (r >= mrows || col >= lim) continue;
                    float v[32];
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const uint4 t = *reinterpret_cast<const uint4*>(&o_st[r * OP + sl * 32 + q * 8]);
                        v[8 * q] = bf16_lo(t.x); v[8 * q + 1] = bf16_hi(t.x);
                        v[8 * q + 2] = bf16_lo(t.y); v[8 * q + 3] = bf16_hi(t.y);
                        v[8 * q + 4] = bf16_lo(t.z); v[8 * q + 5] = bf16_hi(t.z);
                        v[8 * q + 6] = bf16_lo(t.w); v[8 * q + 7] = bf16_hi(t.w);
                    }
                    uint32_t code[8];
                    const uint32_t sb = mx_block(v, code);
                    uint4* o = reinterpret_cast<uint4*>(p.lo_q + a_row0 + (int64_t)(col / 32) * a_blk + (int64_t)(m0 + r) * 32);
                    o[0] = make_uint4(code[0], code[1], code[2], code[3]);
                    o[1] = make_uint4(code[4], code[5], code[6], code[7]);
                    const int64_t srow = shared ? (int64_t)P * (p.f / 32) + (int64_t)(m0 + r) * (p.fs / 32)
                                                : (int64_t)(base + m0 + r) * (p.f / 32);
                    p.lo_s[srow + col / 32] = (uint8_t)sb;
                }
            } else if constexpr (MODE == MODE_W13) {
                // a in its 32-column blocks: consecutive threads write each block's rows in order
                for (int i = tid; i < BM * CH; i += THREADS) {
                    const int sl = i / (BM * 4), r = (i / 4) % BM, c4 = i % 4;
                    const int col = col0 + sl * 32 + c4 * 8;
                    if (r >= mrows || col >= lim) continue;
                    const uint4 v = *reinterpret_cast<const uint4*>(&o_st[r * OP + sl * 32 + c4 * 8]);
                    uint16_t* o = reinterpret_cast<uint16_t*>(p.out) + (pl ? p.lo_off : 0) + a_row0 +
                                  (int64_t)(col / 32) * a_blk + (int64_t)(m0 + r) * 32 + c4 * 8;
                    *reinterpret_cast<uint4*>(o) = v;
                }
            } else {
                for (int i = tid; i < BM * CH; i += THREADS) {
                    const int r = i / CH, ch = i % CH;
                    if (r >= mrows || col0 + ch * 8 >= lim) continue;
                    const int row = m0 + r;
                    const uint4 v = *reinterpret_cast<const uint4*>(&o_st[r * OP + ch * 8]);
                    uint16_t* o = (shared ? reinterpret_cast<uint16_t*>(p.out_sh) + (int64_t)row * p.d
                                          : reinterpret_cast<uint16_t*>(p.out) + (int64_t)(base + row) * p.d) + col0 + ch * 8;
                    *reinterpret_cast<uint4*>(o) = v;
                }
            }
        }
    }
}

// ------------------------------------------------------------------------------------------------
// ggemm_w2q: the down projection of the bf16 path with MXFP4 weights, y = a_hi . W + a_lo . W.
// a_hi (bf16) meets the weights on the bf16 matrix cores as in ggemm<W2>; the correction a_lo =
// a - a_hi, about 2^-8 of a, needs only a few significant bits and comes as MXFP8 (E4M3 codes,
// one E8M0 scale per 32 columns), so it meets the stored E2M1 codes directly on the scaled
// fp8 x fp4 matrix cores (v_mfma_scale_f32_32x32x64_f8f6f4): one 64-K instruction per 32 x 32
// sub-tile instead of four bf16 ones, and half the bytes of a bf16 lo plane.  The quantised
// correction keeps the error of a within 2^-4 of the largest |a_lo| of its 32-column block
// (≈ 2^-12 of the block's |a|).
//
// K stages of 64: per stage and 128 x 256 tile, a_hi rows of 128 bytes (two 32-column blocks,
// 16-byte chunk c of row r at c ^ ((r >> 1) & 7)), a_lo rows of 64 bytes (chunk_swz) and weight
// rows of 32 code bytes (chunk h of row n at h ^ ((n >> 3) & 1)); E8M0 scales of two stages
// (four 32-element blocks, one dword per row) every second stage; a two-stage ring.
// The 64 K elements of a stage are assigned to the bf16 instructions so that lane half h of
// instruction c holds K = 32h + 8c .. +7: the four instructions of a lane then use exactly the
// 32 codes (K = 32h .. 32h+31) that the lane hands to the scaled instruction, expanded per
// dword, and one scale byte covers them.
// ------------------------------------------------------------------------------------------------
template <bool YF32>
__global__ void __launch_bounds__(256, 2) ggemm_w2q(GemmArgs p) {
    constexpr int BM = TBM, BN = 256, BK = 64, NWN = 2, THREADS = 256;
    constexpr int WN = BN / NWN, NT32 = WN / 32;
    constexpr int SZ_AH = BM * 128, SZ_AL = BM * 64, SZ_B = BN * 32;
    constexpr int SZ_STAGE = SZ_AH + SZ_AL + SZ_B;
    constexpr int SZ_SC = 2 * (BN + BM) * 4;
    constexpr int OP = BN + 8;
    constexpr int SZ_O = YF32 ? 0 : BM * OP * 2;
    constexpr int SZ_RING = (2 * SZ_STAGE + SZ_SC) > SZ_O ? (2 * SZ_STAGE + SZ_SC) : SZ_O;
    __shared__ __attribute__((aligned(16))) uint8_t smem[SZ_RING + (MOE_MAX_E + 2) * 4];
    uint8_t* const sAH = smem;
    uint8_t* const sAL = smem + 2 * SZ_AH;
    uint8_t* const sB = smem + 2 * (SZ_AH + SZ_AL);
    uint32_t* const sSB = reinterpret_cast<uint32_t*>(smem + 2 * SZ_STAGE);  // [2][BN]
    uint32_t* const sSA = sSB + 2 * BN;                                       // [2][BM]
    int* s_pref = reinterpret_cast<int*>(smem + SZ_RING);

    const int tid = threadIdx.x, lane = tid & 63, wv = wave_id(), wm = wv / NWN, wn = wv % NWN;
    const int G = p.E + p.n_shared;
    const int P = p.T * p.k;

    // ---- the flat tile list of ggemm<W2>: group g has ceil(rows_g / BM) x ceil(d / BN) tiles
    auto tiles_of = [&](int g) -> int {
        const bool sh = g == p.E;
        const int rows = (p.mask && !p.mask[g]) ? 0 : (sh ? p.T : p.offsets[g + 1] - p.offsets[g]);
        return ((rows + BM - 1) / BM) * ((p.d + BN - 1) / BN);
    };
    if (wv == 0) wave_tile_prefix<(MOE_MAX_E + 64) / 64>(G, s_pref, tiles_of);
    __syncthreads();
    const int total = s_pref[G];
    const int xcd = blockIdx.x & 7, j = blockIdx.x >> 3;
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
    const bool shared = g == p.E;
    const int K = shared ? p.fs : p.f, N = p.d;
    const int rows_g = shared ? p.T : p.offsets[g + 1] - p.offsets[g];
    const int base = shared ? 0 : p.offsets[g];
    const int ntiles = (p.d + BN - 1) / BN;
    const int local = L - s_pref[g];
    const int mt = local / ntiles, nt = local % ntiles;
    const int m0 = mt * BM;
    const int mrows = min(BM, rows_g - m0);
    const int64_t wrb = K / 2, wsb = K / 32;
    const uint8_t* W = shared ? p.sw : p.w + (int64_t)g * N * wrb;
    const uint8_t* WS = shared ? p.swsc : p.wsc + (int64_t)g * N * wsb;
    // a in 32-column blocks (as ggemm writes it): element of the group's row 0 in block 0, and
    // elements from one block to the next; the lo plane's bytes follow the same offsets
    const int64_t a_row0 = shared ? (int64_t)P * p.f : (int64_t)base * 32;
    const int64_t a_blk = shared ? (int64_t)p.T * 32 : (int64_t)P * 32;

    // ---- this thread's global sources (rows past the group's end re-read the tile's first row)
    const uint16_t* ahsrc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int s = i * THREADS + tid, r = s >> 3, c = (s & 7) ^ ((r >> 1) & 7);
        const int rr = r < mrows ? r : 0;
        ahsrc[i] = p.A + a_row0 + (int64_t)(c >> 2) * a_blk + (int64_t)(m0 + rr) * 32 + (c & 3) * 8;
    }
    const uint8_t* alsrc[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int s = i * THREADS + tid, r = s >> 2, c = (s & 3) ^ chunk_swz(r);
        const int rr = r < mrows ? r : 0;
        alsrc[i] = p.lo_q + a_row0 + (int64_t)(c >> 1) * a_blk + (int64_t)(m0 + rr) * 32 + (c & 1) * 16;
    }
    const uint8_t* bsrc[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int s = i * THREADS + tid, n = s >> 1, h = (s & 1) ^ ((n >> 3) & 1);
        const int r = nt * BN + n;
        bsrc[i] = W + (int64_t)(r < N ? r : 0) * wrb + h * 16;
    }
    const int rb = nt * BN + tid;
    const uint8_t* bssrc = WS + (int64_t)(rb < N ? rb : 0) * wsb;
    const int ra = tid < mrows ? tid : 0;
    const uint8_t* assrc = p.lo_s + (shared ? (int64_t)P * (p.f / 32) + (int64_t)(m0 + ra) * (p.fs / 32)
                                            : (int64_t)(base + m0 + ra) * (p.f / 32));

    auto issue = [&](int kt) {
        const int st = kt & 1;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            dma16(ahsrc[i] + (int64_t)(2 * kt) * a_blk, sAH + st * SZ_AH + (i * THREADS + wv * 64) * 16);
#pragma unroll
        for (int i = 0; i < 2; ++i)
            dma16(alsrc[i] + (int64_t)(2 * kt) * a_blk, sAL + st * SZ_AL + (i * THREADS + wv * 64) * 16);
#pragma unroll
        for (int i = 0; i < 2; ++i) dma16(bsrc[i] + kt * 32, sB + st * SZ_B + (i * THREADS + wv * 64) * 16);
        if ((kt & 1) == 0) {
            dma4(bssrc + 2 * kt, &sSB[((kt >> 1) & 1) * BN + wv * 64]);
            if (tid < BM) dma4(assrc + 2 * kt, &sSA[((kt >> 1) & 1) * BM + wv * 64]);
        }
    };

    f32x16_t acc[2][NT32];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < NT32; ++b)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[a][b][e] = 0.0f;

    const int l32 = lane & 31, hk = lane >> 5;
    const int nk = K / BK;
    const bool live = wm * 64 < mrows;
    issue(0);
    for (int kt = 0; kt < nk; ++kt) {
        const int st = kt & 1;
        asm volatile("" ::: "memory");
        VM_WAIT(0);
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        if (kt + 1 < nk) issue(kt + 1);
        if (!live) continue;
        const int sbuf = (kt >> 1) & 1, sh8 = 8 * (2 * (kt & 1) + hk);
        // the lane's 32 weight codes (K = 32hk .. +31 of this stage) and their scale, per column tile
        v4u_t bq[NT32];
        uint32_t bsc[NT32];
#pragma unroll
        for (int ns = 0; ns < NT32; ++ns) {
            const int n = wn * WN + ns * 32 + l32;
            bq[ns] = *reinterpret_cast<const v4u_t*>(sB + st * SZ_B + n * 32 + ((hk ^ ((n >> 3) & 1)) * 16));
            bsc[ns] = (sSB[sbuf * BN + n] >> sh8) & 0xFFu;
        }
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            bf16x8v bfr[NT32];
#pragma unroll
            for (int ns = 0; ns < NT32; ++ns) bfr[ns] = __builtin_bit_cast(bf16x8v, fp4x8_to_bf16(bq[ns][c], bsc[ns]));
            bf16x8v af[2];
#pragma unroll
            for (int ms = 0; ms < 2; ++ms) {
                const int r = wm * 64 + ms * 32 + l32;
                af[ms] = __builtin_bit_cast(bf16x8v, *reinterpret_cast<const v4u_t*>(
                    sAH + st * SZ_AH + r * 128 + (((4 * hk + c) ^ ((r >> 1) & 7)) * 16)));
            }
#pragma unroll
            for (int ms = 0; ms < 2; ++ms)
#pragma unroll
                for (int ns = 0; ns < NT32; ++ns)
                    acc[ms][ns] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[ms], bfr[ns], acc[ms][ns], 0, 0, 0);
        }
        // the correction: E4M3 bytes 0..15 at K = 16hk + 0..15 and 16..31 at K = 32 + 16hk + 0..15
#pragma unroll
        for (int ms = 0; ms < 2; ++ms) {
            const int r = wm * 64 + ms * 32 + l32;
            const uint8_t* row = sAL + st * SZ_AL + r * 64;
            const v4u_t lo = *reinterpret_cast<const v4u_t*>(row + ((hk ^ chunk_swz(r)) * 16));
            const v4u_t hi = *reinterpret_cast<const v4u_t*>(row + (((2 + hk) ^ chunk_swz(r)) * 16));
            const v8i_t aq = v8i_t{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
            const int sa = (int)((sSA[sbuf * BM + r] >> sh8) & 0xFFu);
#pragma unroll
            for (int ns = 0; ns < NT32; ++ns) {
                const v8i_t bf = v8i_t{(int)bq[ns].x, (int)bq[ns].y, (int)bq[ns].z, (int)bq[ns].w, 0, 0, 0, 0};
                acc[ms][ns] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(aq, bf, acc[ms][ns], 0, 4, 0, sa, 0,
                                                                              (int)bsc[ns]);
            }
        }
    }

    // ---- epilogue: accumulator j of lane l is row 8*(j/4) + 4*(l/32) + j%4, column l%32
    if constexpr (YF32) {
#pragma unroll
        for (int ms = 0; ms < 2; ++ms)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int r = wm * 64 + ms * 32 + (e >> 2) * 8 + (lane >> 5) * 4 + (e & 3);
                if (r >= mrows) continue;
                const int row = m0 + r;
                float* o = shared ? reinterpret_cast<float*>(p.out_sh) + (int64_t)row * p.d
                                  : reinterpret_cast<float*>(p.out) + (int64_t)(base + row) * p.d;
#pragma unroll
                for (int ns = 0; ns < NT32; ++ns) {
                    const int n = nt * BN + wn * WN + ns * 32 + (lane & 31);
                    if (n < N) o[n] = acc[ms][ns][e];
                }
            }
    } else {
        uint16_t* o_st = reinterpret_cast<uint16_t*>(smem);
        __syncthreads();
#pragma unroll
        for (int ms = 0; ms < 2; ++ms)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int r = wm * 64 + ms * 32 + (e >> 2) * 8 + (lane >> 5) * 4 + (e & 3);
#pragma unroll
                for (int ns = 0; ns < NT32; ++ns) o_st[r * OP + wn * WN + ns * 32 + (lane & 31)] = f32_to_bf16(acc[ms][ns][e]);
            }
        __syncthreads();
        constexpr int CH = BN / 8;
        const int col0 = nt * BN;
        for (int i = tid; i < BM * CH; i += THREADS) {
            const int r = i / CH, ch = i % CH;
            if (r >= mrows || col0 + ch * 8 >= N) continue;
            const int row = m0 + r;
            const uint4 v = *reinterpret_cast<const uint4*>(&o_st[r * OP + ch * 8]);
            uint16_t* o = (shared ? reinterpret_cast<uint16_t*>(p.out_sh) + (int64_t)row * p.d
                                  : reinterpret_cast<uint16_t*>(p.out) + (int64_t)(base + row) * p.d) + col0 + ch * 8;
            *reinterpret_cast<uint4*>(o) = v;
        }
    }
}

static unsigned grid8(int64_t tiles) {
    int64_t g = (tiles + 7) / 8 * 8;
    return (unsigned)(g < 8 ? 8 : g);
}

hipError_t launch_route_logits_mfma(const void* x, const void* wr, const float* b, float* logits, int T, int d,
                                    int E, float* part, size_t part_bytes, hipStream_t st, RouterPartials* rp) {
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
    while (ks < ROUTER_MAX_SPLIT && tiles * ks * 2 <= slots && d % (32 * ks * 2) == 0 && d / (ks * 2) >= 128 &&
           (size_t)ks * 2 * T * E * 4 <= part_bytes)
        ks *= 2;
    GemmArgs p{};
    p.A = (const uint16_t*)x;
    p.w = (const uint8_t*)wr;
    p.bias = b;
    p.out = ks > 1 ? (void*)part : (void*)logits;
    p.T = T; p.d = d; p.E = E; p.k = 1;
    p.ksplit = ks;
    // 64-element K stages two deep when every split is whole 64s (half the waits and barriers of
    // 32-element stages, whole 128-byte row pieces), else 32-element stages three deep
    if ((d / ks) % 64 == 0)
        hipLaunchKernelGGL((ggemm<MODE_ROUTER, 1, 128, false, 2, 2, false, false, 64>), dim3(grid8(tiles * ks)),
                           dim3(256), 0, st, p);
    else
        hipLaunchKernelGGL((ggemm<MODE_ROUTER, 1, 128, false, 2>), dim3(grid8(tiles * ks)), dim3(256), 0, st, p);
    *rp = RouterPartials{ks > 1 ? part : nullptr, ks, b, logits};
    return hipGetLastError();
}

// The SwiGLU activation is stored as two bf16 planes (hi, then lo) of P*f + T*fs elements each,
// each in 32-column blocks (routed rows, then the shared expert's; see the kernel).
static int64_t a_lo_offset(int T, int k, int f, int fs, int n_shared) {
    return (int64_t)T * k * f + (n_shared ? (int64_t)T * fs : 0);
}

static int64_t max_tiles(int T, int k, int E, int n_shared, int rows_nt, int shared_nt, int bm = TBM) {
    const int64_t P = (int64_t)T * k;
    const int64_t routed_mt = (P + bm - 1) / bm + (P < E ? P : E);
    const int64_t shared_mt = n_shared ? (T + bm - 1) / bm : 0;
    return routed_mt * rows_nt + shared_mt * shared_nt;
}

// With MXFP4 weights and whole 256-column tiles, the lo plane of a goes to the down projection
// as MXFP8 (ggemm_w2q); its codes follow the hi plane in the workspace, then its scales.
static bool lo_fp8(int wt, int d, int f, int fs, int n_shared) {
    return wt == 2 && d % 256 == 0 && f % 256 == 0 && (!n_shared || fs % 256 == 0);
}
static void lo_planes(GemmArgs& p, uint16_t* a, int T, int k, int f, int fs, int n_shared) {
    const int64_t plane = a_lo_offset(T, k, f, fs, n_shared);
    p.lo_q = reinterpret_cast<uint8_t*>(a + plane);
    p.lo_s = p.lo_q + plane;
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
        // 128-element K stages (256-byte x rows, 64 code bytes per weight row, a quarter of the
        // barriers per flop of 32-element stages; two of them fill 128 KB of LDS) when K = d is a
        // whole number of stages: c3 gate/up 2349 -> 1899 us with 64-element stages three deep,
        // 1882 us with these
        const bool kb_long = d % 128 == 0;
        if (lo_fp8(wt, d, f, fs, n_shared)) {
            lo_planes(p, a, T, k, f, fs, n_shared);
            if (kb_long)
                MOE_LAUNCH(PROF_FFN_UP, (ggemm<MODE_W13, 2, BN, false, NWN, 2, false, true, 128>), dim3(grid),
                           dim3(128 * NWN), 0, st, p);
            else
                MOE_LAUNCH(PROF_FFN_UP, (ggemm<MODE_W13, 2, BN, false, NWN, 3, false, true>), dim3(grid), dim3(128 * NWN),
                           0, st, p);
        } else if (kb_long) {
            MOE_LAUNCH(PROF_FFN_UP, (ggemm<MODE_W13, 2, BN, false, NWN, 2, false, false, 128>), dim3(grid),
                       dim3(128 * NWN), 0, st, p);
        } else {
            MOE_LAUNCH(PROF_FFN_UP, (ggemm<MODE_W13, 2, BN, false, NWN>), dim3(grid), dim3(128 * NWN), 0, st, p);
        }
        return hipGetLastError();
    }
    constexpr int BN = 256, NWN = 2;  // 128 gate/up column pairs per tile, 4 wavefronts
    const unsigned grid = grid8(max_tiles(T, k, E, n_shared, (f + BN / 2 - 1) / (BN / 2), n_shared ? (fs + BN / 2 - 1) / (BN / 2) : 0));
    if (wt == 1 && d % 64 == 0) {
        // bf16 weights: 256 x 256 tiles of 8 wavefronts on 64-element stages two deep (128-byte
        // x and weight rows, 128 KB of LDS, one workgroup per CU): half the barriers per flop of
        // the 128 x 256 tiles on 32-element stages (c2 gate/up 358 -> 333 us)
        const unsigned grid2 = grid8(max_tiles(T, k, E, n_shared, (f + BN / 2 - 1) / (BN / 2),
                                               n_shared ? (fs + BN / 2 - 1) / (BN / 2) : 0, 256));
        MOE_LAUNCH(PROF_FFN_UP, (ggemm<MODE_W13, 1, BN, false, NWN, 2, false, false, 64, 256>), dim3(grid2),
                   dim3(256 * NWN), 0, st, p);
    } else if (wt == 1) MOE_LAUNCH(PROF_FFN_UP, (ggemm<MODE_W13, 1, BN, false, NWN>), dim3(grid), dim3(128 * NWN), 0, st, p);
    else MOE_LAUNCH(PROF_FFN_UP, (ggemm<MODE_W13, 2, BN, false, NWN>), dim3(grid), dim3(128 * NWN), 0, st, p);
    return hipGetLastError();
}

hipError_t launch_ggemm_w2(int wt, const uint16_t* a, const int32_t* offsets, const int32_t*, const int32_t*,
                           const void* w2, const uint8_t* w2s, const void* s2, const uint8_t* s2s, void* y,
                           void* y_shared, bool y_f32, int T, int d, int f, int fs, int k, int E, int n_shared,
                           const uint8_t* mask, hipStream_t st) {
    GemmArgs p{a, nullptr, offsets, (const uint8_t*)w2, w2s, (const uint8_t*)s2, s2s, nullptr, y, y_shared,
               a_lo_offset(T, k, f, fs, n_shared), T, d, f, fs, k, E, n_shared, mask, 1};
    if (lo_fp8(wt, d, f, fs, n_shared)) {
        lo_planes(p, const_cast<uint16_t*>(a), T, k, f, fs, n_shared);
        const unsigned grid = grid8(max_tiles(T, k, E, n_shared, d / 256, d / 256));
        if (y_f32) MOE_LAUNCH(PROF_FFN_DOWN, (ggemm_w2q<true>), dim3(grid), dim3(256), 0, st, p);
        else MOE_LAUNCH(PROF_FFN_DOWN, (ggemm_w2q<false>), dim3(grid), dim3(256), 0, st, p);
        return hipGetLastError();
    }
    constexpr int NWN = 2;
#define MOE_W2(BNV, NSV)                                                                                         \
    do {                                                                                                         \
        const unsigned grid = grid8(max_tiles(T, k, E, n_shared, (d + BNV - 1) / BNV, (d + BNV - 1) / BNV));     \
        if (wt == 1 && y_f32)                                                                                    \
            MOE_LAUNCH(PROF_FFN_DOWN, (ggemm<MODE_W2, 1, BNV, true, NWN, NSV, true>), dim3(grid), dim3(128 * NWN), 0, st, p); \
        else if (wt == 1)                                                                                        \
            MOE_LAUNCH(PROF_FFN_DOWN, (ggemm<MODE_W2, 1, BNV, true, NWN, NSV>), dim3(grid), dim3(128 * NWN), 0, st, p); \
        else if (y_f32)                                                                                          \
            MOE_LAUNCH(PROF_FFN_DOWN, (ggemm<MODE_W2, 2, BNV, true, NWN, NSV, true>), dim3(grid), dim3(128 * NWN), 0, st, p); \
        else MOE_LAUNCH(PROF_FFN_DOWN, (ggemm<MODE_W2, 2, BNV, true, NWN, NSV>), dim3(grid), dim3(128 * NWN), 0, st, p); \
    } while (0)
    // 256 output columns per tile, two stages (the lo/hi A planes and 256 B rows fill 64 KB per
    // stage pair; two workgroups per CU); else 128 columns three deep
    if (d % 256 == 0) MOE_W2(256, 2);
    else MOE_W2(128, 3);
#undef MOE_W2
    return hipGetLastError();
}

}  // namespace moe
