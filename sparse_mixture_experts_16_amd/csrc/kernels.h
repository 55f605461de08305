// Host-side launchers of the gfx950 kernels (internal to libmoe.so).
#pragma once
#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>
#include <stdint.h>

#define MOE_MAX_E 1024
#define MOE_MAX_K 64
#define PERMUTE_SMALL_MAX 4096
#define PERMUTE_MAX_COUNTS 16384  // chunk counts (nblk x E ints) every scatter workgroup reads
#define GEMM_BM 128  // token rows per grouped-GEMM tile (tile list granularity)

namespace moe {

// Pairs per chunk of the large-P permute: as many chunks as the scan can hold in LDS (at most
// 256), each a multiple of 64 pairs (one wavefront scatters a chunk).
inline int permute_chunk(int64_t P, int E) {
    int64_t nmax = PERMUTE_MAX_COUNTS / (E > 0 ? E : 1);
    if (nmax > 256) nmax = 256;
    if (nmax < 1) nmax = 1;
    int64_t c = (P + nmax - 1) / nmax;
    c = (c + 63) / 64 * 64;
    return (int)(c < 256 ? 256 : c);
}

// Timing hook: the launch of the kernel class being profiled carries the caller's start/stop
// events on its own dispatch packet (hipExtLaunchKernel), so they time that kernel alone.
enum { PROF_FFN_UP = 0, PROF_FFN_DOWN = 1 };
void prof_events(int cls, hipEvent_t* start, hipEvent_t* stop);
#define MOE_LAUNCH(CLS, KERNEL, GRID, BLOCK, SHMEM, STREAM, ...)                                  \
    do {                                                                                          \
        hipEvent_t moe_e0_ = nullptr, moe_e1_ = nullptr;                                          \
        ::moe::prof_events(CLS, &moe_e0_, &moe_e1_);                                              \
        hipExtLaunchKernelGGL(KERNEL, GRID, BLOCK, SHMEM, STREAM, moe_e0_, moe_e1_, 0, __VA_ARGS__); \
    } while (0)

hipError_t launch_route_logits(int act_dtype, const void* x, const void* wr, const float* b, float* logits,
                               int T, int d, int E, hipStream_t st);
// The MFMA router's K-split partial sums, left for the top-k kernel to add up (in split order,
// then the bias) into `logits`; at most ROUTER_MAX_SPLIT of them.
#define ROUTER_MAX_SPLIT 8
struct RouterPartials {
    const float* part;  // ks x [T, E]
    int ks;
    const float* bias;  // [E] or null
    float* logits;      // [T, E]: receives the summed logits
};
// part: scratch for the K-split partial sums (part_bytes of it; 0 = no split).  A split leaves
// the partials for launch_route_topk, described in *rp (rp->part null: no split, and logits
// already holds the logits).
hipError_t launch_route_logits_mfma(const void* x, const void* wr, const float* b, float* logits, int T, int d,
                                    int E, float* part, size_t part_bytes, hipStream_t st, RouterPartials* rp);
// rp (nullable): form the logits from the router GEMM's partial sums first (logits is then unused)
hipError_t launch_route_topk(const float* logits, int T, int E, int k, bool no_renorm, int32_t* idx, float* w,
                             int32_t* idx2, hipStream_t st, const RouterPartials* rp = nullptr);

hipError_t launch_permute(const int32_t* idx, int P, int E, int bm, int32_t* counts, int32_t* offsets,
                          int32_t* perm, int32_t* inv, int32_t* act_list, int32_t* tile_off, int32_t* meta,
                          int32_t* blk, hipStream_t st);
hipError_t launch_active_from_offsets(const int32_t* offsets, int E, int bm, int32_t* act_list, int32_t* tile_off,
                                      int32_t* meta, hipStream_t st);

hipError_t launch_gemv_w13(int wt, const void* x, const int32_t* perm, const int32_t* offsets,
                           const int32_t* act_list, const int32_t* meta, const void* w13, const uint8_t* w13s,
                           const void* s13, const uint8_t* s13s, float* a, int T, int d, int f, int fs, int k,
                           int E, int n_shared, float g_r, float g_s, hipStream_t st);
hipError_t launch_gemv_w2_combine(int wt, bool out_bf16, const float* a, const int32_t* perm, const int32_t* offsets,
                                  const int32_t* act_list, const int32_t* meta, const float* topk_w, const void* w2,
                                  const uint8_t* w2s, const void* s2, const uint8_t* s2s, void* out, int T, int d,
                                  int f, int fs, int k, int n_shared, bool accumulate, float g_r, float g_s,
                                  hipStream_t st);
hipError_t launch_gemv_w2_sorted(int wt, bool y_bf16, const float* a, const int32_t* perm, const int32_t* offsets,
                                 const int32_t* act_list, const int32_t* meta, const void* w2, const uint8_t* w2s,
                                 const void* s2, const uint8_t* s2s, void* y, void* y_shared, int T, int d, int f,
                                 int fs, int k, int E, int n_shared, float g_r, float g_s, hipStream_t st);

// Prefill grouped GEMM (MFMA).  a_bf16: routed [P, f] then shared [T, fs].
// mask (nullable, E + 1 bytes): groups whose byte is 0 get no tiles.
hipError_t launch_ggemm_w13(int wt, const uint16_t* x, const int32_t* perm, const int32_t* offsets,
                            const int32_t* tile_off, const int32_t* meta, const void* w13, const uint8_t* w13s,
                            const void* s13, const uint8_t* s13s, uint16_t* a, int T, int d, int f, int fs, int k,
                            int E, int n_shared, const uint8_t* mask, hipStream_t st);
hipError_t launch_ggemm_w2(int wt, const uint16_t* a, const int32_t* offsets, const int32_t* tile_off,
                           const int32_t* meta, const void* w2, const uint8_t* w2s, const void* s2,
                           const uint8_t* s2s, void* y, void* y_shared, bool y_f32, int T, int d, int f, int fs,
                           int k, int E, int n_shared, const uint8_t* mask, hipStream_t st);

// MX prefill (MXFP4 weights on the scaled fp8 x fp4 matrix cores, activations quantised to MXFP8):
// x -> codes [rows, d] + E8M0 scales [rows, d/32]; gate/up (+ SwiGLU, a quantised in the
// epilogue into codes [P*f + T*fs] and scales [(P*f + T*fs)/32]); down projection to bf16 or f32.
// x_dtype 0: f32 rows, 1: bf16 rows; K % 32 == 0
hipError_t launch_mx_quant_rows(int x_dtype, const void* x, uint8_t* q, uint8_t* sc, int64_t rows, int64_t K,
                                hipStream_t st);
hipError_t launch_mxgemm_w13(const uint8_t* xq, const uint8_t* xs, const int32_t* perm, const int32_t* offsets,
                             const void* w13, const uint8_t* w13s, const void* s13, const uint8_t* s13s, uint8_t* aq,
                             uint8_t* aqs, int T, int d, int f, int fs, int k, int E, int n_shared,
                             const uint8_t* mask, hipStream_t st);
hipError_t launch_mxgemm_w2(const uint8_t* aq, const uint8_t* aqs, const int32_t* offsets, const void* w2,
                            const uint8_t* w2s, const void* s2, const uint8_t* s2s, void* y, void* y_shared,
                            bool y_f32, int T, int d, int f, int fs, int k, int E, int n_shared, const uint8_t* mask,
                            hipStream_t st);

// Decode path (T <= 32, T*E <= 8192): router logits, then the FFN kernels (the gate/up kernel
// redoes the routing per workgroup in LDS; workgroup 0 publishes it).
bool dec_supported(int T, int E, int k);
hipError_t launch_dec_logits(int act_dtype, const void* x, const void* wr, const float* b, float* logits, void* xn,
                             int T, int d, int E, bool prenorm, hipStream_t st);
hipError_t launch_dec_ffn(int wt, bool out_bf16, const void* x, const float* logits, int32_t* topk_idx,
                          float* topk_w, int32_t* idx_out, int32_t* meta, int4* slots, float* pos_gate,
                          bool no_renorm, const void* w13, const uint8_t* w13s, const void* s13, const uint8_t* s13s,
                          const void* w2, const uint8_t* w2s, const void* s2, const uint8_t* s2s, float* a, void* out,
                          int T, int d, int f, int fs, int k, int E, int n_shared, bool accumulate,
                          const uint8_t* mask, const float* gsc, hipStream_t st);  // gsc: g13, g2, gs13, gs2

// mask (nullable, E + 1 bytes; needs idx): terms of experts whose byte is 0 are left out.
// The decode stack for one token in one cooperative launch (MXFP4 weights, bf16 activations).
struct StackLayerPtrs {
    const void* wr;
    const float* br;
    const void* w13;
    const uint8_t* w13s;
    const void* w2;
    const uint8_t* w2s;
};
constexpr int STACK_LAYERS_PER_LAUNCH = 48;
int dec_stack_bar_ints();
int dec_stack_err_index();
bool dec_stack_supported(int d, int f, int E, int k);
hipError_t launch_dec_stack(const StackLayerPtrs* layers, int n_layers, float* h, float* hbuf, float* logits,
                            uint16_t* xn, float* a, int32_t* idx_out, int* bar, int64_t sh_h, int64_t sh_lg,
                            int64_t sh_xn, int64_t sh_a, int d, int f, int E, int k, bool no_renorm, int spin_limit,
                            bool clear_err, hipStream_t st);
hipError_t launch_combine(int y_dtype, int out_dtype, const void* y, const int32_t* inv, const float* topk_w,
                          const void* ysh, void* out, int T, int d, int k, bool accumulate, const int32_t* idx,
                          const uint8_t* mask, int E, hipStream_t st);
hipError_t launch_mxfp4_dequant(const uint8_t* codes, const uint8_t* scales, float* out, int64_t rows, int64_t K,
                                hipStream_t st);
hipError_t launch_nvfp4_dequant(const uint8_t* codes, const uint8_t* scales, float gscale, float* out, int64_t rows,
                                int64_t K, hipStream_t st);
hipError_t launch_rmsnorm(int x_dtype, const float* h, void* x, int T, int d, float eps, hipStream_t st);

}  // namespace moe
