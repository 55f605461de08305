// Prefill grouped GEMM on the gfx950 scaled matrix cores (MOE_F_MX_GEMM): MXFP4 expert weights
// enter v_mfma_scale_f32_32x32x64_f8f6f4 as they are stored, and the activations are quantised
// on the fly to MXFP8 (E4M3 elements, one E8M0 scale per 32 along K; OCP Microscaling Formats
// v1.0): x by mx_quant_rows before gate/up, the SwiGLU output a inside the gate/up epilogue.
// The pages run their DeepSeek-V4-Flash build on MXFP4 experts (dothoosh.com FreeToken article,
// "Benchmarks and real performance"); at prefill every expert's weights meet thousands of
// tokens, and the fp8 x fp4 matrix cores do twice the work per cycle of the bf16 ones with no
// per-fragment expansion of the codes.
//
// Operand layout of the scaled MFMA (measured on gfx950): A (E4M3, 32 bytes per lane): lane l
// holds row l%32; its bytes 0..15 are K = 16*(l/32) + 0..15 and bytes 16..31 are
// K = 32 + 16*(l/32) + 0..15.  B (E2M1, 16 bytes per lane): lane l holds column l%32,
// K = 32*(l/32) + 0..31, element 2i in the low nibble of byte i.  Scales: byte 0 of lane l's
// scale operand is the E8M0 scale of row (column) l%32 for the K block l/32.  Accumulator j of
// lane l: row 8*(j/4) + 4*(l/32) + j%4, column l%32.
//
// Tile: 128 token rows x 256 weight rows, K in stages of 128 (two MFMAs per 32x32 sub-tile), 4
// wavefronts as 2 x 2, each owning 64 x 128.  Stages stream through a double-buffered LDS ring by
// global_load_lds (A rows 128 bytes, B rows 64 bytes, both chunk-swizzled so fragment reads are
// conflict-free); the E8M0 scales of four stages (16 blocks) travel as 16 bytes per row into a
// double-buffered row list.  Tiles come from the flat (expert, m-tile, n-tile) list of the bf16
// kernel.  A down projection with d not a multiple of 256 uses 128-column tiles with 64-element
// stages three deep.
#include "common.h"
#include "kernels.h"
#include "lds_dma.h"
#include "mxfp8.h"

namespace moe {

typedef int v8i_t __attribute__((ext_vector_type(8)));
// Fragment reads from LDS are loads of this vector type, not of a struct: a load that carries no
// type-based alias information makes the compiler's wait insertion drain every global -> LDS
// load in flight before it, which would serialise the ring (the explicit vmcnt waits and
// barriers below already order each stage's loads before its reads).
typedef unsigned v4u_t __attribute__((ext_vector_type(4)));

enum { MX_W13 = 0, MX_W2 = 1 };


// rows [rows, d] (bf16 or f32) -> codes [rows, d], scales [rows, d/32]; one thread per block.
template <typename X>
__global__ void __launch_bounds__(256) mx_quant_rows(const X* __restrict__ x, uint8_t* __restrict__ q,
                                                     uint8_t* __restrict__ sc, int64_t nblk) {
    for (int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; b < nblk; b += (int64_t)gridDim.x * blockDim.x) {
        float v[32];
        if constexpr (sizeof(X) == 2) {
            const uint4* src = reinterpret_cast<const uint4*>(x + b * 32);
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const uint4 u = src[c];
                const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
                for (int h = 0; h < 4; ++h) {
                    v[8 * c + 2 * h] = bf16_lo(w[h]);
                    v[8 * c + 2 * h + 1] = bf16_hi(w[h]);
                }
            }
        } else {
            const float4* src = reinterpret_cast<const float4*>(x + b * 32);
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                const float4 u = src[c];
                v[4 * c] = u.x;
                v[4 * c + 1] = u.y;
                v[4 * c + 2] = u.z;
                v[4 * c + 3] = u.w;
            }
        }
        uint32_t code[8];
        sc[b] = (uint8_t)mx_block(v, code);
        uint4* dst = reinterpret_cast<uint4*>(q + b * 32);
        dst[0] = make_uint4(code[0], code[1], code[2], code[3]);
        dst[1] = make_uint4(code[4], code[5], code[6], code[7]);
    }
}

hipError_t launch_mx_quant_rows(int x_dtype, const void* x, uint8_t* q, uint8_t* sc, int64_t rows, int64_t K,
                                hipStream_t st) {
    const int64_t nblk = rows * (K / 32);
    if (nblk == 0) return hipSuccess;
    int64_t blocks = (nblk + 255) / 256;
    if (blocks > 8192) blocks = 8192;
    if (x_dtype == 0)
        hipLaunchKernelGGL(mx_quant_rows<float>, dim3((unsigned)blocks), dim3(256), 0, st, (const float*)x, q, sc, nblk);
    else
        hipLaunchKernelGGL(mx_quant_rows<uint16_t>, dim3((unsigned)blocks), dim3(256), 0, st, (const uint16_t*)x, q, sc,
                           nblk);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------
// The grouped GEMM
// ---------------------------------------------------------------------------------------------
struct MxGemmArgs {
    const uint8_t* A;        // W13: x codes [T, d]; W2: a codes (routed [P, f], shared at +P*f as [T, fs])
    const uint8_t* As;       // A scales: W13 [T, d/32]; W2 routed [P, f/32], shared at +P*f/32 as [T, fs/32]
    const int32_t* perm;     // W13: sorted slot -> pair
    const int32_t* offsets;  // [E+1]
    const uint8_t* w;        // routed MXFP4 codes [E, N, K/2]
    const uint8_t* wsc;      // routed E8M0 scales [E, N, K/32]
    const uint8_t* sw;       // shared expert
    const uint8_t* swsc;
    uint8_t* aq;             // W13 out: a codes, laid out as the W2 A operand
    uint8_t* aqs;            // W13 out: a scales
    void* y;                 // W2 out: y_sorted [P, d] bf16 (f32 with YF32)
    void* y_sh;              // W2 out: y_shared [T, d], the dtype of y
    int T, d, f, fs, k, E, n_shared;
    const uint8_t* mask;     // nullable [E + 1]: groups whose byte is 0 get no tiles
};

// Chunk swizzles of the LDS tiles: 16-byte chunk c of row r sits at physical chunk c ^ swz(r), so
// that a wavefront's fragment reads (consecutive rows, one chunk each) fall on distinct banks.
template <int CH>  // chunks per row
__device__ __forceinline__ int tile_swz(int r) {
    if constexpr (CH == 8) return (r >> 1) & 7;   // 128-byte rows
    else if constexpr (CH == 4) return chunk_swz(r);
    else return 0;                                // 32-byte rows: two chunks, no conflict to remove
}
template <int CH>  // B rows (weights) of CH chunks
__device__ __forceinline__ int btile_swz(int r) {
    if constexpr (CH == 4) return (r >> 2) & 3;   // 64-byte rows
    else return 0;
}

// BM x BN output tile: BM / 64 rows of two wavefronts, each 64 x BN/2 (BM = 128: 256 threads, two
// workgroups per CU; BM = 256: 512 threads, one per CU).  BK: K elements per stage (64: A rows of
// 64 bytes, B rows of 32; 128: 128 and 64).  NS: ring depth.  SCB: scale bytes fetched per row at a
// time (4 or 16; 16 needs K % 512 == 0).
// YF32 (down projection only): y in fp32 straight from the accumulators.
template <int MODE, int BM, int BN, int NS, int SCB, int BK, bool YF32 = false>
__global__ void __launch_bounds__(BM * 2, 256 / BM) mxgemm(MxGemmArgs p) {
    constexpr int NWN = 2, THREADS = BM * 2;
    static_assert(BM == 128 || BM == 256, "tile rows");
    static_assert(NS >= 2 && NS <= 4, "ring depth");
    static_assert(SCB == 4 || SCB == 16, "scale fetch");
    static_assert(BK == 64 || BK == 128, "stage depth");
    constexpr int KS = BK / 64;                               // MFMA K steps per stage
    constexpr int ACH = BK / 16, BCH = BK / 32;               // 16-byte chunks per A row / B row
    constexpr int SBK = BK / 32;                              // scale blocks per row per stage
    static_assert(SCB % SBK == 0, "scale groups hold whole stages");
    constexpr int SST = SCB / SBK;                            // stages covered by one scale fetch
    // scale groups in flight at once: a group's buffer is refilled NS - 1 stages ahead of its first
    // use, so it must not be the buffer of a group still being read
    constexpr int SB = 1 + (NS - 2 + SST) / SST;              // 1 + ceil((NS - 1) / SST)
    constexpr int SW = SCB / 4;                               // scale dwords per row per group
    constexpr int WN = BN / NWN, NT32 = WN / 32;
    constexpr int NA = BM * ACH / THREADS;                    // A chunks per thread per stage
    constexpr int NB = BN * BCH / THREADS;                    // B chunks per thread per stage
    constexpr int OPS = NA + NB;                              // loads one stage adds (scale fetches not counted)
    static_assert(NA >= 1 && NB >= 1 && (NS - 2) * OPS < 16, "tile / thread count");
    constexpr int SZ_A = NS * BM * BK, SZ_B = NS * BN * BK / 2, SZ_SA = SB * BM * SCB, SZ_SB = SB * BN * SCB;
    // epilogue: the output tile passes through LDS EPR rows at a time (gate/up: one thread per
    // (row, 32-column block) of the 128 a-columns)
    constexpr int EPR = (MODE == MX_W13) ? THREADS / 4 : 128;
    static_assert(MODE != MX_W13 || BN == 256, "gate/up tiles give 128 a-columns");
    constexpr int APITCH = 132;  // fp32 a-values per staged row (gate/up)
    constexpr int OP = BN + 8;   // bf16 per staged output row (down)
    constexpr int SZ_EP = (MODE == MX_W13) ? EPR * APITCH * 4 : EPR * OP * 2;
    constexpr int SZ_RING = SZ_A + SZ_B + SZ_SA + SZ_SB;
    constexpr int SZ_LIST = (MOE_MAX_E + 2) * 4;  // the tile list prefix, read before the ring fills
    constexpr int SZ0 = SZ_RING > SZ_EP ? SZ_RING : SZ_EP;
    constexpr int SZ = SZ0 > SZ_LIST ? SZ0 : SZ_LIST;
    __shared__ __attribute__((aligned(16))) uint8_t smem[SZ];
    uint8_t* sA = smem;
    uint8_t* sB = smem + SZ_A;
    uint32_t* sSA = reinterpret_cast<uint32_t*>(smem + SZ_A + SZ_B);
    uint32_t* sSB = reinterpret_cast<uint32_t*>(smem + SZ_A + SZ_B + SZ_SA);
    int* s_pref = reinterpret_cast<int*>(smem);

    const int tid = threadIdx.x, lane = tid & 63, wv = wave_id(), wm = wv / NWN, wn = wv % NWN;
    const int G = p.E + p.n_shared;
    const int P = p.T * p.k;

    // ---- flat tile list: tiles of group g = ceil(rows_g / BM) * ntiles_g
    auto tiles_of = [&](int g) -> int {
        const bool sh = g == p.E;
        const int rows = (p.mask && !p.mask[g]) ? 0 : (sh ? p.T : p.offsets[g + 1] - p.offsets[g]);
        const int nt = (MODE == MX_W13) ? (sh ? p.fs : p.f) / (BN / 2) : p.d / BN;
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
    const int local = L - s_pref[g];
    __syncthreads();  // the list shares its LDS with the ring filled below
    const bool shared = g == p.E;
    const int fg = shared ? p.fs : p.f;
    const int rows_g = shared ? p.T : p.offsets[g + 1] - p.offsets[g];
    const int base = shared ? 0 : p.offsets[g];
    const int K = (MODE == MX_W13) ? p.d : fg, N = (MODE == MX_W13) ? 2 * fg : p.d;
    const int ntiles = (MODE == MX_W13) ? fg / (BN / 2) : p.d / BN;
    const int64_t wrb = K / 2, wsb = K / 32;
    const uint8_t* W = shared ? p.sw : p.w + (int64_t)g * N * wrb;
    const uint8_t* WS = shared ? p.swsc : p.wsc + (int64_t)g * N * wsb;
    const int mt = local / ntiles, nt = local % ntiles;
    const int m0 = mt * BM;
    const int mrows = min(BM, rows_g - m0);

    // ---- A sources: chunk slot s = i*THREADS + tid holds row s/ACH at physical chunk s%ACH; rows
    // past the group's end re-read the tile's first row (their results are never stored), or, with
    // a two-stage ring (whose every wait drains all loads), are not loaded at all.
    auto a_row = [&](int r) -> int64_t {  // byte offset of row r's codes; scales at /32
        if (r >= mrows) r = 0;
        if (MODE == MX_W13) return (int64_t)(shared ? m0 + r : p.perm[base + m0 + r] / p.k) * p.d;
        return shared ? (int64_t)P * p.f + (int64_t)(m0 + r) * p.fs : (int64_t)(base + m0 + r) * p.f;
    };
    const uint8_t* asrc[NA];
    bool alive[NA];
#pragma unroll
    for (int i = 0; i < NA; ++i) {
        const int slot = i * THREADS + tid, r = slot / ACH;
        asrc[i] = p.A + a_row(r) + ((slot % ACH) ^ tile_swz<ACH>(r)) * 16;
        alive[i] = NS != 2 || r < mrows;
    }
    const uint8_t* assrc = p.As + a_row(tid < BM ? tid : 0) / 32;
    // ---- B sources.  Gate/up: each wavefront column holds BN/4 gate rows and the matching
    // BN/4 up rows, so SwiGLU pairs meet in the same lane.
    auto wrow_of = [&](int n) -> int {
        if (MODE == MX_W13) {
            constexpr int H = BN / (2 * NWN);
            const int h = n / (2 * H), w = n % (2 * H);
            const int j = nt * (BN / 2) + h * H + (w < H ? w : w - H);
            return w < H ? j : fg + j;
        }
        return nt * BN + n;
    };
    const uint8_t* bsrc[NB];
#pragma unroll
    for (int i = 0; i < NB; ++i) {
        const int slot = i * THREADS + tid, n = slot / BCH;
        bsrc[i] = W + (int64_t)wrow_of(n) * wrb + ((slot % BCH) ^ btile_swz<BCH>(n)) * 16;
    }
    const uint8_t* bssrc = WS + (int64_t)wrow_of(tid < BN ? tid : 0) * wsb;

    // stage kt's A and B codes, and at a scale group's first stage the group's scales (SCB blocks
    // of each row for stages kt .. kt+SST-1)
    auto issue = [&](int kt) {
        const int st = kt % NS;
#pragma unroll
        for (int i = 0; i < NA; ++i)
            if (alive[i]) dma16(asrc[i] + kt * BK, sA + st * BM * BK + (i * THREADS + wv * 64) * 16);
#pragma unroll
        for (int i = 0; i < NB; ++i)
            dma16(bsrc[i] + kt * (BK / 2), sB + st * BN * (BK / 2) + (i * THREADS + wv * 64) * 16);
        if (kt % SST == 0) {
            const int grp = kt / SST, sbuf = grp % SB;
            if constexpr (SCB == 16) {
                if (tid < BM) dma16(assrc + grp * 16, sSA + (sbuf * BM + wv * 64) * SW);
                if (tid < BN) dma16(bssrc + grp * 16, sSB + (sbuf * BN + wv * 64) * SW);
            } else {
                if (tid < BM) dma4(assrc + grp * 4, sSA + sbuf * BM + wv * 64);
                if (tid < BN) dma4(bssrc + grp * 4, sSB + sbuf * BN + wv * 64);
            }
        }
    };

    f32x16_t acc[2][NT32];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < NT32; ++b)
#pragma unroll
            for (int j = 0; j < 16; ++j) acc[a][b][j] = 0.0f;

    const int l32 = lane & 31, hk = lane >> 5;
    const int nk = K / BK;
    // a wavefront whose 64 rows all lie past the group's end only loads and synchronises; its
    // matrix-core time goes to the other workgroup on the CU
    const bool live = wm * 64 < mrows;
#pragma unroll
    for (int i = 0; i < NS - 1; ++i)
        if (i < nk) issue(i);
    for (int kt = 0; kt < nk; ++kt) {
        const int st = kt % NS;
        // wait for stage kt; the stages issued after it (up to NS - 2) stay in flight.  A stage adds
        // OPS loads plus any scale loads, so waiting down to OPS (2 * OPS) outstanding leaves only
        // loads of the newer stages.
        asm volatile("" ::: "memory");
        const int newer = min(NS - 2, nk - 1 - kt);
        if (newer >= 2) VM_WAIT(2 * OPS);
        else if (newer == 1) VM_WAIT(OPS);
        else VM_WAIT(0);
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        if (kt + NS - 1 < nk) issue(kt + NS - 1);

        if (!live) continue;
        const int sbuf = (kt / SST) % SB;
#pragma unroll
        for (int u = 0; u < KS; ++u) {
            // this lane's block inside its row's scale group: (kt % SST) * SBK + 2u + hk
            const int sblk = (kt % SST) * SBK + 2 * u + hk;
            const int sw = sblk >> 2, sh8 = 8 * (sblk & 3);
            v8i_t af[2];
            int sa[2];
#pragma unroll
            for (int ms = 0; ms < 2; ++ms) {
                const int r = wm * 64 + ms * 32 + l32;
                const uint8_t* row = sA + st * BM * BK + r * BK;
                const v4u_t lo = *reinterpret_cast<const v4u_t*>(row + ((4 * u + hk) ^ tile_swz<ACH>(r)) * 16);
                const v4u_t hi = *reinterpret_cast<const v4u_t*>(row + ((4 * u + 2 + hk) ^ tile_swz<ACH>(r)) * 16);
                af[ms] = v8i_t{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
                sa[ms] = (int)((sSA[(sbuf * BM + r) * SW + sw] >> sh8) & 0xFFu);
            }
#pragma unroll
            for (int ns = 0; ns < NT32; ++ns) {
                const int n = wn * WN + ns * 32 + l32;
                const v4u_t b = *reinterpret_cast<const v4u_t*>(sB + st * BN * (BK / 2) + n * (BK / 2) +
                                                                ((2 * u + hk) ^ btile_swz<BCH>(n)) * 16);
                const v8i_t bf = v8i_t{(int)b.x, (int)b.y, (int)b.z, (int)b.w, 0, 0, 0, 0};
                const int sb = (int)((sSB[(sbuf * BN + n) * SW + sw] >> sh8) & 0xFFu);
#pragma unroll
                for (int ms = 0; ms < 2; ++ms)
                    acc[ms][ns] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af[ms], bf, acc[ms][ns], 0, 4, 0,
                                                                                  sa[ms], 0, sb);
            }
        }
    }

    // ---- epilogue: accumulator j of lane l is row 8*(j/4) + 4*(l/32) + j%4, column l%32
    if constexpr (MODE == MX_W13) {
        // SwiGLU in place of the gate accumulators, then MXFP8 quantisation of a: the tile's
        // 128 a-columns of 64 rows at a time are staged in LDS as fp32, and each thread
        // quantises one (row, 32-column block).
#pragma unroll
        for (int ms = 0; ms < 2; ++ms)
#pragma unroll
            for (int ns = 0; ns < NT32 / 2; ++ns)
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    const float gt = acc[ms][ns][j], up = acc[ms][ns + NT32 / 2][j];
                    acc[ms][ns][j] = silu_hw(gt) * up;
                }
        float* o_st = reinterpret_cast<float*>(smem);
        const int col0 = nt * (BN / 2);
        const int64_t rowbytes = shared ? p.fs : p.f;
        uint8_t* qbase = p.aq + (shared ? (int64_t)P * p.f : 0);
        uint8_t* sbase = p.aqs + (shared ? (int64_t)P * (p.f / 32) : 0);
        const int qrow0 = shared ? m0 : base + m0;
#pragma unroll
        for (int pass = 0; pass < BM / EPR; ++pass) {
            if (pass * EPR >= mrows) break;  // uniform over the workgroup
            __syncthreads();
            if (wm * 64 / EPR == pass) {
#pragma unroll
                for (int ms = 0; ms < 2; ++ms)
#pragma unroll
                    for (int j = 0; j < 16; ++j) {
                        const int r = (wm * 64) % EPR + ms * 32 + (j >> 2) * 8 + hk * 4 + (j & 3);
#pragma unroll
                        for (int ns = 0; ns < NT32 / 2; ++ns) o_st[r * APITCH + wn * (WN / 2) + ns * 32 + l32] = acc[ms][ns][j];
                    }
            }
            __syncthreads();
            const int rr = tid >> 2, cb = tid & 3;
            const int row = pass * EPR + rr;
            if (row < mrows) {
                float v[32];
#pragma unroll
                for (int q = 0; q < 8; ++q) {
                    const float4 t = *reinterpret_cast<const float4*>(&o_st[rr * APITCH + cb * 32 + q * 4]);
                    v[4 * q] = t.x;
                    v[4 * q + 1] = t.y;
                    v[4 * q + 2] = t.z;
                    v[4 * q + 3] = t.w;
                }
                uint32_t code[8];
                const uint32_t sb = mx_block(v, code);
                const int64_t qr = (int64_t)(qrow0 + row);
                uint4* dst = reinterpret_cast<uint4*>(qbase + qr * rowbytes + col0 + cb * 32);
                dst[0] = make_uint4(code[0], code[1], code[2], code[3]);
                dst[1] = make_uint4(code[4], code[5], code[6], code[7]);
                sbase[qr * (rowbytes / 32) + col0 / 32 + cb] = (uint8_t)sb;
            }
        }
    } else if constexpr (YF32) {
        // fp32 y from the accumulators: the 32 lanes holding one row write 128 contiguous bytes
#pragma unroll
        for (int ms = 0; ms < 2; ++ms)
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const int r = wm * 64 + ms * 32 + (j >> 2) * 8 + hk * 4 + (j & 3);
                if (r >= mrows) continue;
                const int row = m0 + r;
                float* o = (shared ? reinterpret_cast<float*>(p.y_sh) + (int64_t)row * p.d
                                   : reinterpret_cast<float*>(p.y) + (int64_t)(base + row) * p.d) + nt * BN;
#pragma unroll
                for (int ns = 0; ns < NT32; ++ns) o[wn * WN + ns * 32 + l32] = acc[ms][ns][j];
            }
    } else {
        // bf16 outputs staged in LDS, then whole 16-byte row chunks stored
        uint16_t* o_st = reinterpret_cast<uint16_t*>(smem);
        constexpr int CH = BN / 8;
        const int col0 = nt * BN;
#pragma unroll
        for (int pass = 0; pass < BM / EPR; ++pass) {
            if (pass * EPR >= mrows) break;  // uniform over the workgroup
            __syncthreads();
            if (wm * 64 / EPR == pass) {
#pragma unroll
                for (int ms = 0; ms < 2; ++ms)
#pragma unroll
                    for (int j = 0; j < 16; ++j) {
                        const int r = (wm * 64) % EPR + ms * 32 + (j >> 2) * 8 + hk * 4 + (j & 3);
#pragma unroll
                        for (int ns = 0; ns < NT32; ++ns)
                            o_st[r * OP + wn * WN + ns * 32 + l32] = f32_to_bf16(acc[ms][ns][j]);
                    }
            }
            __syncthreads();
            for (int i = tid; i < EPR * CH; i += THREADS) {
                const int r = pass * EPR + i / CH, ch = i % CH;
                if (r >= mrows) continue;
                const int row = m0 + r;
                const uint4 v = *reinterpret_cast<const uint4*>(&o_st[(i / CH) * OP + ch * 8]);
                uint16_t* o = (shared ? reinterpret_cast<uint16_t*>(p.y_sh) + (int64_t)row * p.d
                                      : reinterpret_cast<uint16_t*>(p.y) + (int64_t)(base + row) * p.d) +
                              col0 + ch * 8;
                *reinterpret_cast<uint4*>(o) = v;
            }
        }
    }
}

// Stage shapes.  Both stages read 128-byte activation rows and 64-byte weight rows per stage into a
// double-buffered ring with 256-column tiles.  A down projection with d not a multiple of 256 takes
// 128 x 128 tiles with 64-element stages three deep, the faster of the shapes measured at that
// tile width.
// 256-row tiles (one 8-wavefront workgroup per CU) measured slower at every ring depth: the two
// independent workgroups of 128 rows hide each other's load waits.
constexpr int MX_BM = 128, MX_BK = 128, MX_NS = 2;

static unsigned mx_grid8(int64_t tiles) {
    int64_t g = (tiles + 7) / 8 * 8;
    return (unsigned)(g < 8 ? 8 : g);
}

// tiles of BM rows over all groups: at most ceil(P / BM) + one ragged tile per group
static int64_t mx_max_tiles(int BM, int T, int k, int E, int n_shared, int rows_nt, int shared_nt) {
    const int64_t P = (int64_t)T * k;
    const int64_t routed_mt = (P + BM - 1) / BM + (P < E ? P : E);
    const int64_t shared_mt = n_shared ? (T + BM - 1) / BM : 0;
    return routed_mt * rows_nt + shared_mt * shared_nt;
}

hipError_t launch_mxgemm_w13(const uint8_t* xq, const uint8_t* xs, const int32_t* perm, const int32_t* offsets,
                             const void* w13, const uint8_t* w13s, const void* s13, const uint8_t* s13s, uint8_t* aq,
                             uint8_t* aqs, int T, int d, int f, int fs, int k, int E, int n_shared,
                             const uint8_t* mask, hipStream_t st) {
    constexpr int BM = MX_BM, BN = 256;
    MxGemmArgs p{xq, xs, perm, offsets, (const uint8_t*)w13, w13s, (const uint8_t*)s13, s13s, aq, aqs,
                 nullptr, nullptr, T, d, f, fs, k, E, n_shared, mask};
    const unsigned grid =
        mx_grid8(mx_max_tiles(BM, T, k, E, n_shared, f / (BN / 2), n_shared ? fs / (BN / 2) : 0));
    if (d % 512 == 0)
        MOE_LAUNCH(PROF_FFN_UP, (mxgemm<MX_W13, BM, BN, MX_NS, 16, MX_BK>), dim3(grid), dim3(2 * BM), 0, st, p);
    else MOE_LAUNCH(PROF_FFN_UP, (mxgemm<MX_W13, BM, BN, MX_NS, 4, MX_BK>), dim3(grid), dim3(2 * BM), 0, st, p);
    return hipGetLastError();
}

hipError_t launch_mxgemm_w2(const uint8_t* aq, const uint8_t* aqs, const int32_t* offsets, const void* w2,
                            const uint8_t* w2s, const void* s2, const uint8_t* s2s, void* y, void* y_shared,
                            bool y_f32, int T, int d, int f, int fs, int k, int E, int n_shared, const uint8_t* mask,
                            hipStream_t st) {
    MxGemmArgs p{aq, aqs, nullptr, offsets, (const uint8_t*)w2, w2s, (const uint8_t*)s2, s2s, nullptr, nullptr,
                 y, y_shared, T, d, f, fs, k, E, n_shared, mask};
    const bool scb16 = f % 512 == 0 && (!n_shared || fs % 512 == 0);
#define MOE_MXW2(BMV, BNV, NSV, BKV)                                                                              \
    do {                                                                                                          \
        const unsigned grid = mx_grid8(mx_max_tiles(BMV, T, k, E, n_shared, d / BNV, d / BNV));                   \
        if (scb16 && y_f32)                                                                                       \
            MOE_LAUNCH(PROF_FFN_DOWN, (mxgemm<MX_W2, BMV, BNV, NSV, 16, BKV, true>), dim3(grid), dim3(2 * BMV), 0, st, p); \
        else if (scb16)                                                                                           \
            MOE_LAUNCH(PROF_FFN_DOWN, (mxgemm<MX_W2, BMV, BNV, NSV, 16, BKV>), dim3(grid), dim3(2 * BMV), 0, st, p); \
        else if (y_f32)                                                                                           \
            MOE_LAUNCH(PROF_FFN_DOWN, (mxgemm<MX_W2, BMV, BNV, NSV, 4, BKV, true>), dim3(grid), dim3(2 * BMV), 0, st, p); \
        else MOE_LAUNCH(PROF_FFN_DOWN, (mxgemm<MX_W2, BMV, BNV, NSV, 4, BKV>), dim3(grid), dim3(2 * BMV), 0, st, p); \
    } while (0)
    if (d % 256 == 0) MOE_MXW2(MX_BM, 256, MX_NS, MX_BK);
    else MOE_MXW2(128, 128, 3, 64);
#undef MOE_MXW2
    return hipGetLastError();
}

}  // namespace moe
