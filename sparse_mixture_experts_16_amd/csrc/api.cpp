// C-ABI of the MoE layer: host-side validation, workspace layout and kernel dispatch.
// Every entry point validates all arguments before it enqueues anything; see include/moe.h.
#include <hip/hip_runtime.h>

#include <stdint.h>
#include <string.h>

#include <mutex>

#include "../../include/moe.h"
#include "kernels.h"

using namespace moe;

namespace {

constexpr int DECODE_MAX_T = 32;  // at or below: grouped GEMV kernels (HBM-bound decode)
constexpr size_t ALIGN = 256;

size_t up(size_t v) { return (v + ALIGN - 1) / ALIGN * ALIGN; }

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
int ptr_ok(const void* p) { return p && aligned16(p); }

int act_bytes(int dt) { return dt == MOE_F32 ? 4 : 2; }

// Workspace regions (byte offsets from ws).
struct Layout {
    size_t logits, topk_idx, topk_w, counts, offsets, perm, inv, act_list, tile_off, meta, blk, slots, pos_tok,
        pos_gate, a, y, ysh, xn, total;
};

Layout layout(const moe_shape* s) {
    Layout L{};
    const size_t T = (size_t)s->T, E = (size_t)s->n_experts, k = (size_t)s->top_k, d = (size_t)s->d_model;
    const size_t f = (size_t)s->d_ff, fs = s->n_shared ? (size_t)s->shared_d_ff : 0;
    const size_t P = T * k;
    const size_t ab = (size_t)act_bytes(s->act_dtype);
    const size_t pc = (size_t)permute_chunk((int64_t)P, (int)E);
    const size_t nblk = P > PERMUTE_SMALL_MAX ? (P + pc - 1) / pc : 0;
    const size_t fmax = fs > f ? fs : f;
    size_t o = 0;
    L.logits = o; o = up(o + T * E * 4);
    L.topk_idx = o; o = up(o + P * 4);
    L.topk_w = o; o = up(o + P * 4);
    L.counts = o; o = up(o + E * 4);
    L.offsets = o; o = up(o + (E + 1) * 4);
    L.perm = o; o = up(o + P * 4);
    L.inv = o; o = up(o + P * 4);
    L.act_list = o; o = up(o + (E + 1) * 4);
    L.tile_off = o; o = up(o + (E + 2) * 4);
    L.meta = o; o = up(o + 16 * 4);
    L.blk = o; o = up(o + nblk * E * 4);
    L.slots = o; o = up(o + (E + 1) * 16);
    L.pos_tok = o; o = up(o + (P + T) * 4);
    L.pos_gate = o; o = up(o + (P + T) * 4);
    // fp32 rows of width fmax at decode, two bf16 planes at prefill
    const size_t a_dec = (P + T) * fmax * 4, a_pre = (P * f + T * fs) * 4;
    L.a = o; o = up(o + (a_dec > a_pre ? a_dec : a_pre));
    // y_sorted / y_shared: fp32 inside the layer at prefill (the combine sums unrounded expert
    // outputs), the act dtype for the step calls; also the router K-split scratch (written only
    // after routing) and the MX path's x codes
    L.y = o; o = up(o + P * d * 4);
    L.ysh = o; o = up(o + T * d * 4);
    L.xn = o; o = up(o + T * d * ab);
    L.total = o;
    return L;
}

template <typename T> T* at(void* ws, size_t off) { return reinterpret_cast<T*>(reinterpret_cast<char*>(ws) + off); }

// Shape checks shared by every entry point.
int check_shape(const moe_shape* s) {
    if (!s) return MOE_ERR_INVALID_ARG;
    if (s->T < 0 || s->d_model < 1 || s->d_ff < 1 || s->n_experts < 1) return MOE_ERR_INVALID_ARG;
    if (s->top_k < 1 || s->top_k > s->n_experts) return MOE_ERR_INVALID_ARG;
    if (s->n_shared < 0 || s->n_shared > 1) return MOE_ERR_INVALID_ARG;
    if (s->n_shared == 1 && s->shared_d_ff < 1) return MOE_ERR_INVALID_ARG;
    const bool pair_ok = (s->act_dtype == MOE_F32 && s->weight_dtype == MOE_F32) ||
                         (s->act_dtype == MOE_BF16 && (s->weight_dtype == MOE_BF16 || s->weight_dtype == MOE_MXFP4 ||
                                                       s->weight_dtype == MOE_NVFP4));
    if (s->act_dtype < MOE_F32 || s->act_dtype > MOE_BF16 || s->weight_dtype < MOE_F32 || s->weight_dtype > MOE_NVFP4)
        return MOE_ERR_INVALID_ARG;
    if (!pair_ok) return MOE_ERR_UNSUPPORTED;
    if (s->n_experts > MOE_MAX_EXPERTS || s->top_k > MOE_MAX_TOPK) return MOE_ERR_UNSUPPORTED;
    if ((int64_t)s->T * s->top_k > INT32_MAX / 2) return MOE_ERR_UNSUPPORTED;
    // 16-byte vector loads along every contiguous dimension.
    const int vec = s->act_dtype == MOE_F32 ? 4 : 8;
    const int fs = s->n_shared ? s->shared_d_ff : 32 * vec;  // no shared expert: nothing to check
    if (s->weight_dtype == MOE_MXFP4 || s->weight_dtype == MOE_NVFP4) {  // 32-element code chunks
        if (s->d_model % 32 || s->d_ff % 32 || fs % 32) return MOE_ERR_INVALID_ARG;
    } else {
        if (s->d_model % vec || s->d_ff % vec || fs % vec) return MOE_ERR_INVALID_ARG;
    }
    if (s->flags &
        ~(uint32_t)(MOE_F_NO_RENORM | MOE_F_ACCUMULATE | MOE_F_FORCE_GEMV | MOE_F_FORCE_GEMM | MOE_F_MX_GEMM))
        return MOE_ERR_INVALID_ARG;
    if ((s->flags & MOE_F_FORCE_GEMV) && (s->flags & MOE_F_FORCE_GEMM)) return MOE_ERR_INVALID_ARG;
    if ((s->flags & MOE_F_MX_GEMM) && s->weight_dtype != MOE_MXFP4) return MOE_ERR_UNSUPPORTED;
    return MOE_OK;
}

// The MFMA kernels tile K by 64 and the gate/up columns by 64.
bool gemm_shape_ok(const moe_shape* s) {
    // K steps of 32; MXFP4 scales move four 32-element blocks (one dword) at a time
    const int q = s->weight_dtype == MOE_MXFP4 ? 128 : 64;
    const int fs = s->n_shared ? s->shared_d_ff : q;
    // NVFP4 weights take the grouped-GEMV kernels at every T
    return s->act_dtype == MOE_BF16 && s->weight_dtype != MOE_NVFP4 && s->d_model % q == 0 && s->d_ff % q == 0 &&
           fs % q == 0;
}

// Which FFN kernels run: grouped GEMV (decode) or grouped MFMA GEMM (prefill).
bool use_gemm(const moe_shape* s) {
    if (s->flags & MOE_F_FORCE_GEMV) return false;
    if (!gemm_shape_ok(s)) return false;
    if (s->flags & MOE_F_FORCE_GEMM) return true;
    return s->T > DECODE_MAX_T;
}

int check_weights(const moe_shape* s, const moe_weights* w) {
    if (!w || !w->w13 || !w->w2) return MOE_ERR_INVALID_ARG;
    if (!aligned16(w->w13) || !aligned16(w->w2)) return MOE_ERR_INVALID_ARG;
    const bool scaled = s->weight_dtype == MOE_MXFP4 || s->weight_dtype == MOE_NVFP4;
    if (scaled && (!ptr_ok(w->w13_scale) || !ptr_ok(w->w2_scale))) return MOE_ERR_INVALID_ARG;
    if (s->n_shared) {
        if (!w->s13 || !w->s2 || !aligned16(w->s13) || !aligned16(w->s2)) return MOE_ERR_INVALID_ARG;
        if (scaled && (!ptr_ok(w->s13_scale) || !ptr_ok(w->s2_scale))) return MOE_ERR_INVALID_ARG;
    }
    return MOE_OK;
}


int hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

#define MOE_TRY(expr)                                  \
    do {                                               \
        hipError_t _e = (expr);                        \
        if (_e != hipSuccess) return MOE_ERR_HIP;      \
    } while (0)

// Optional timing hook (moe_profile_kernel): the events ride on the profiled class's launch.
hipEvent_t g_prof_start = nullptr, g_prof_stop = nullptr;
int g_prof_kernel = -1;
static_assert(MOE_KERNEL_FFN_UP == PROF_FFN_UP && MOE_KERNEL_FFN_DOWN == PROF_FFN_DOWN, "kernel classes");

// NVFP4 tensor scales {routed gate/up, routed down, shared gate/up, shared down}; 1 otherwise.
void tensor_scales(const moe_shape* s, const moe_weights* w, float g[4]) {
    const bool nv = s->weight_dtype == MOE_NVFP4;
    g[0] = nv ? w->w13_gscale : 1.0f;
    g[1] = nv ? w->w2_gscale : 1.0f;
    g[2] = nv ? w->s13_gscale : 1.0f;
    g[3] = nv ? w->s2_gscale : 1.0f;
}

// Routed + shared FFNs given ws-resident permute results: y_sorted / y_shared in the act dtype,
// or in fp32 (y_f32).
int run_ffn(const moe_shape* s, const void* x, const int32_t* perm, const int32_t* offsets, const int32_t* act_list,
            const int32_t* tile_off, const int32_t* meta, const moe_weights* w, void* ws, const Layout& L,
            void* y_sorted, void* y_shared, bool y_f32, const uint8_t* mask, hipStream_t st) {
    const int wt = s->weight_dtype;
    const int fs = s->n_shared ? s->shared_d_ff : 0;
    if (use_gemm(s) && (s->flags & MOE_F_MX_GEMM)) {
        // x codes and scales in the y region (consumed by gate/up before the down projection
        // writes y), a codes and scales in the a region
        const int64_t T = s->T, d = s->d_model, P = T * s->top_k;
        uint8_t* xq = at<uint8_t>(ws, L.y);
        uint8_t* xs = xq + T * d;
        uint8_t* aq = at<uint8_t>(ws, L.a);
        uint8_t* aqs = aq + P * s->d_ff + T * fs;
        MOE_TRY(launch_mx_quant_rows(MOE_BF16, x, xq, xs, T, d, st));
        MOE_TRY(launch_mxgemm_w13(xq, xs, perm, offsets, w->w13, w->w13_scale, w->s13, w->s13_scale, aq, aqs, s->T,
                                  s->d_model, s->d_ff, fs, s->top_k, s->n_experts, s->n_shared, mask, st));
        MOE_TRY(launch_mxgemm_w2(aq, aqs, offsets, w->w2, w->w2_scale, w->s2, w->s2_scale, y_sorted, y_shared,
                                 y_f32, s->T, s->d_model, s->d_ff, fs, s->top_k, s->n_experts, s->n_shared, mask,
                                 st));
        return MOE_OK;
    }
    if (use_gemm(s)) {
        uint16_t* a = at<uint16_t>(ws, L.a);
        MOE_TRY(launch_ggemm_w13(wt, (const uint16_t*)x, perm, offsets, tile_off, meta, w->w13, w->w13_scale,
                                 w->s13, w->s13_scale, a, s->T, s->d_model, s->d_ff, fs, s->top_k, s->n_experts,
                                 s->n_shared, mask, st));
        MOE_TRY(launch_ggemm_w2(wt, a, offsets, tile_off, meta, w->w2, w->w2_scale, w->s2, w->s2_scale, y_sorted,
                                y_shared, y_f32, s->T, s->d_model, s->d_ff, fs, s->top_k, s->n_experts,
                                s->n_shared, mask, st));
        return MOE_OK;
    }
    float* a = at<float>(ws, L.a);
    float gs[4];
    tensor_scales(s, w, gs);
    MOE_TRY(launch_gemv_w13(wt, x, perm, offsets, act_list, meta, w->w13, w->w13_scale, w->s13, w->s13_scale, a,
                            s->T, s->d_model, s->d_ff, fs, s->top_k, s->n_experts, s->n_shared, gs[0], gs[2], st));
    MOE_TRY(launch_gemv_w2_sorted(wt, s->act_dtype == MOE_BF16 && !y_f32, a, perm, offsets, act_list, meta, w->w2, w->w2_scale,
                                  w->s2, w->s2_scale, y_sorted, y_shared, s->T, s->d_model, s->d_ff, fs, s->top_k,
                                  s->n_experts, s->n_shared, gs[1], gs[3], st));
    return MOE_OK;
}

// Decode path: router logits, then gate/up (routing redone per workgroup) and down + combine.
// prenorm: x is the fp32 residual stream, normalised by the logits kernel into ws.xn.
int run_decode(const moe_shape* s, const void* x, const void* w_router, const float* b, const moe_weights* w,
               void* out, int out_dtype, bool accumulate, int32_t* idx_out, bool prenorm, void* ws, const Layout& L,
               const uint8_t* mask, hipStream_t st) {
    void* xn = at<void>(ws, L.xn);
    float gs[4];
    tensor_scales(s, w, gs);
    MOE_TRY(launch_dec_logits(s->act_dtype, x, w_router, b, at<float>(ws, L.logits), xn, s->T, s->d_model,
                              s->n_experts, prenorm, st));
    hipError_t e = launch_dec_ffn(
        s->weight_dtype, out_dtype == MOE_BF16, prenorm ? xn : x, at<float>(ws, L.logits), at<int32_t>(ws, L.topk_idx),
        at<float>(ws, L.topk_w), idx_out, at<int32_t>(ws, L.meta), at<int4>(ws, L.slots), at<float>(ws, L.pos_gate),
        (s->flags & MOE_F_NO_RENORM) != 0, w->w13, w->w13_scale, w->s13, w->s13_scale, w->w2, w->w2_scale, w->s2,
        w->s2_scale, at<float>(ws, L.a), out, s->T, s->d_model, s->d_ff, s->n_shared ? s->shared_d_ff : 0, s->top_k,
        s->n_experts, s->n_shared, accumulate, mask, gs, st);
    if (e != hipSuccess) return MOE_ERR_HIP;
    return MOE_OK;
}

bool use_decode(const moe_shape* s) {
    return !use_gemm(s) && s->T <= DECODE_MAX_T && dec_supported(s->T, s->n_experts, s->top_k);
}

// The whole layer on x; out has dtype out_dtype (act dtype for the layer API, f32 for the stack).
int run_layer(const moe_shape* s, const void* x, const void* w_router, const float* b, const moe_weights* w,
              void* out, int out_dtype, bool accumulate, int32_t* idx_out, void* ws, const Layout& L,
              const uint8_t* mask, hipStream_t st) {
    const int T = s->T, E = s->n_experts, k = s->top_k, d = s->d_model, P = T * k;
    const int fs = s->n_shared ? s->shared_d_ff : 0;
    float* logits = at<float>(ws, L.logits);
    int32_t* idx = at<int32_t>(ws, L.topk_idx);
    float* g = at<float>(ws, L.topk_w);
    int32_t* counts = at<int32_t>(ws, L.counts);
    int32_t* offsets = at<int32_t>(ws, L.offsets);
    int32_t* perm = at<int32_t>(ws, L.perm);
    int32_t* inv = at<int32_t>(ws, L.inv);
    int32_t* act_list = at<int32_t>(ws, L.act_list);
    int32_t* tile_off = at<int32_t>(ws, L.tile_off);
    int32_t* meta = at<int32_t>(ws, L.meta);
    int32_t* blk = at<int32_t>(ws, L.blk);
    const bool gemm = use_gemm(s);
    if (use_decode(s)) return run_decode(s, x, w_router, b, w, out, out_dtype, accumulate, idx_out, false, ws, L, mask, st);
    RouterPartials rp{};  // the MFMA router's K-split partials are added up by the top-k kernel
    if (gemm && T > DECODE_MAX_T)
        MOE_TRY(launch_route_logits_mfma(x, w_router, b, logits, T, d, E, at<float>(ws, L.y), L.ysh - L.y, st, &rp));
    else
        MOE_TRY(launch_route_logits(s->act_dtype, x, w_router, b, logits, T, d, E, st));
    MOE_TRY(launch_route_topk(logits, T, E, k, (s->flags & MOE_F_NO_RENORM) != 0, idx, g, idx_out, st,
                              rp.part ? &rp : nullptr));
    MOE_TRY(launch_permute(idx, P, E, GEMM_BM, counts, offsets, perm, inv, act_list, tile_off, meta, blk, st));
    if (!gemm && T <= 64 && !mask) {
        float* a = at<float>(ws, L.a);
        float gs[4];
        tensor_scales(s, w, gs);
        MOE_TRY(launch_gemv_w13(s->weight_dtype, x, perm, offsets, act_list, meta, w->w13, w->w13_scale, w->s13,
                                w->s13_scale, a, T, d, s->d_ff, fs, k, E, s->n_shared, gs[0], gs[2], st));
        MOE_TRY(launch_gemv_w2_combine(s->weight_dtype, out_dtype == MOE_BF16, a, perm, offsets, act_list, meta, g,
                                       w->w2, w->w2_scale, w->s2, w->s2_scale, out, T, d, s->d_ff, fs, k,
                                       s->n_shared, accumulate, gs[1], gs[3], st));
        return MOE_OK;
    }
    void* y = at<void>(ws, L.y);
    void* ysh = s->n_shared ? at<void>(ws, L.ysh) : nullptr;
    // the expert outputs reach the combine in fp32: rounding them to bf16 first would add an
    // error relative to each expert's output, which a near-cancelling sum can exceed
    int rc = run_ffn(s, x, perm, offsets, act_list, tile_off, meta, w, ws, L, y, ysh, true, mask, st);
    if (rc != MOE_OK) return rc;
    MOE_TRY(launch_combine(0, out_dtype == MOE_BF16 ? 1 : 0, y, inv, g, ysh, out, T, d, k, accumulate, idx, mask, E,
                           st));
    return MOE_OK;
}

}  // namespace

// Scratch area of moe_layer_forward_noalloc: one per GPU (each device holds its own copy of this
// array), looked up once per device; host code uses only the looked-up address.
static __device__ __align__(256) uint8_t scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int NOALLOC_MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[NOALLOC_MAX_DEVICES] = {};

// The current device's scratch address, looked up on the first call on that device.
hipError_t scratch_ptr(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= NOALLOC_MAX_DEVICES) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}
}  // namespace

namespace {
// Workspace of moe_stack_forward_persistent: the barrier words, then one region per layer of a
// launch for its logits, x, a and (between layers) h, each region 256-byte aligned.
struct StackLayout {
    size_t bar, logits, xn, a, hbuf, total;
    int64_t sh_lg, sh_xn, sh_a, sh_h;  // elements per region
    int lc;                             // layers per launch
};

StackLayout stack_layout(const moe_shape* s, int n_layers) {
    StackLayout L{};
    const size_t d = (size_t)s->d_model, f = (size_t)s->d_ff, E = (size_t)s->n_experts, k = (size_t)s->top_k;
    L.lc = n_layers < STACK_LAYERS_PER_LAUNCH ? n_layers : STACK_LAYERS_PER_LAUNCH;
    const size_t lc = L.lc < 1 ? 1 : (size_t)L.lc;
    // h between layers: one 128-byte line per 8-row block
    const size_t lg_b = up(E * 4), xn_b = up(d * 2), a_b = up(k * f * 4), h_b = up((d + 7) / 8 * 128);
    L.sh_lg = (int64_t)(lg_b / 4);
    L.sh_xn = (int64_t)(xn_b / 2);
    L.sh_a = (int64_t)(a_b / 4);
    L.sh_h = (int64_t)(h_b / 4);
    size_t o = 0;
    L.bar = o; o = up(o + (size_t)dec_stack_bar_ints() * 4);
    L.logits = o; o += lc * lg_b;
    L.xn = o; o += lc * xn_b;
    L.a = o; o += lc * a_b;
    L.hbuf = o; o += (lc - 1) * h_b;
    L.total = up(o);
    return L;
}

int g_stack_spin_limit = 1 << 20;

// The shapes whose decode stack runs as dec_logits (single pass), dec_w13 and dec_w2c1 with
// MXFP4 weights, one token and no shared expert.
int check_stack_persistent(const moe_shape* s) {
    int rc = check_shape(s);
    if (rc != MOE_OK) return rc;
    if (s->T != 1 || s->act_dtype != MOE_BF16 || s->weight_dtype != MOE_MXFP4 || s->n_shared != 0 || !use_decode(s) ||
        !dec_stack_supported(s->d_model, s->d_ff, s->n_experts, s->top_k))
        return MOE_ERR_UNSUPPORTED;
    return MOE_OK;
}
}  // namespace

namespace moe {
void prof_events(int cls, hipEvent_t* start, hipEvent_t* stop) {
    if (cls == g_prof_kernel) {
        *start = g_prof_start;
        *stop = g_prof_stop;
    }
}
}  // namespace moe

extern "C" {

size_t moe_workspace_size(const moe_shape* s) {
    if (check_shape(s) != MOE_OK) return 0;
    return layout(s).total;
}

const char* moe_status_string(int status) {
    switch (status) {
        case MOE_OK: return "ok";
        case MOE_ERR_INVALID_ARG: return "invalid argument";
        case MOE_ERR_UNSUPPORTED: return "unsupported configuration";
        case MOE_ERR_WORKSPACE: return "workspace too small";
        case MOE_ERR_HIP: return "HIP error";
        case MOE_ERR_SCRATCH_LIMIT: return "shape needs more scratch than moe_layer_forward_noalloc holds (64 MiB)";
        default: return "unknown status";
    }
}

int moe_route(const moe_shape* s, const void* x, const void* w_router, const float* b_router, const float* logits_in,
              int32_t* topk_idx, float* topk_w, float* logits_out, void* ws, size_t ws_bytes, void* stream) {
    int rc = check_shape(s);
    if (rc != MOE_OK) return rc;
    if (s->T == 0) return MOE_OK;
    if (!ptr_ok(topk_idx) || !ptr_ok(topk_w)) return MOE_ERR_INVALID_ARG;
    if (logits_out && !aligned16(logits_out)) return MOE_ERR_INVALID_ARG;
    if (logits_in) {
        if (!aligned16(logits_in)) return MOE_ERR_INVALID_ARG;
    } else {
        if (!ptr_ok(x) || !ptr_ok(w_router)) return MOE_ERR_INVALID_ARG;
        if (b_router && !aligned16(b_router)) return MOE_ERR_INVALID_ARG;
    }
    const Layout L = layout(s);
    if (!ws || !aligned16(ws) || ws_bytes < L.total) return MOE_ERR_WORKSPACE;
    hipStream_t st = (hipStream_t)stream;
    const int T = s->T, E = s->n_experts;
    const float* logits = logits_in;
    RouterPartials rp{};  // the MFMA router's K-split partials are added up by the top-k kernel
    if (!logits_in) {
        float* dst = logits_out ? logits_out : at<float>(ws, L.logits);
        if (use_gemm(s) && T > DECODE_MAX_T)
            MOE_TRY(launch_route_logits_mfma(x, w_router, b_router, dst, T, s->d_model, E, at<float>(ws, L.y),
                                             L.ysh - L.y, st, &rp));
        else
            MOE_TRY(launch_route_logits(s->act_dtype, x, w_router, b_router, dst, T, s->d_model, E, st));
        logits = dst;
    } else if (logits_out && logits_out != logits_in) {
        MOE_TRY(hipMemcpyAsync(logits_out, logits_in, (size_t)T * E * 4, hipMemcpyDeviceToDevice, st));
    }
    MOE_TRY(launch_route_topk(logits, T, E, s->top_k, (s->flags & MOE_F_NO_RENORM) != 0, topk_idx, topk_w, nullptr,
                              st, rp.part ? &rp : nullptr));
    return MOE_OK;
}

int moe_permute(const moe_shape* s, const int32_t* topk_idx, int32_t* counts, int32_t* offsets, int32_t* perm,
                int32_t* inv_perm, void* ws, size_t ws_bytes, void* stream) {
    int rc = check_shape(s);
    if (rc != MOE_OK) return rc;
    if (s->T == 0) return MOE_OK;
    if (!ptr_ok(topk_idx) || !ptr_ok(counts) || !ptr_ok(offsets) || !ptr_ok(perm) || !ptr_ok(inv_perm))
        return MOE_ERR_INVALID_ARG;
    const Layout L = layout(s);
    if (!ws || !aligned16(ws) || ws_bytes < L.total) return MOE_ERR_WORKSPACE;
    MOE_TRY(launch_permute(topk_idx, s->T * s->top_k, s->n_experts, GEMM_BM, counts, offsets, perm, inv_perm,
                           at<int32_t>(ws, L.act_list), at<int32_t>(ws, L.tile_off), at<int32_t>(ws, L.meta),
                           at<int32_t>(ws, L.blk), (hipStream_t)stream));
    return MOE_OK;
}

int moe_grouped_ffn(const moe_shape* s, const void* x, const int32_t* perm, const int32_t* offsets,
                    const moe_weights* w, void* y_sorted, void* y_shared, void* ws, size_t ws_bytes, void* stream) {
    int rc = check_shape(s);
    if (rc != MOE_OK) return rc;
    if (s->T == 0) return MOE_OK;
    if ((rc = check_weights(s, w)) != MOE_OK) return rc;
    if (!ptr_ok(x) || !ptr_ok(perm) || !ptr_ok(offsets) || !ptr_ok(y_sorted)) return MOE_ERR_INVALID_ARG;
    if (s->n_shared ? !ptr_ok(y_shared) : y_shared != nullptr) return MOE_ERR_INVALID_ARG;
    const Layout L = layout(s);
    if (!ws || !aligned16(ws) || ws_bytes < L.total) return MOE_ERR_WORKSPACE;
    hipStream_t st = (hipStream_t)stream;
    int32_t* act_list = at<int32_t>(ws, L.act_list);
    int32_t* tile_off = at<int32_t>(ws, L.tile_off);
    int32_t* meta = at<int32_t>(ws, L.meta);
    MOE_TRY(launch_active_from_offsets(offsets, s->n_experts, GEMM_BM, act_list, tile_off, meta, st));
    return run_ffn(s, x, perm, offsets, act_list, tile_off, meta, w, ws, L, y_sorted, y_shared, false, nullptr, st);
}

// The two contractions of the MX prefill path as separate calls (MXFP4 weights, bf16 act, the
// MFMA GEMM's shape constraints).
static int mx_stage_check(const moe_shape* s, const moe_weights* w) {
    int rc = check_shape(s);
    if (rc != MOE_OK) return rc;
    if (s->weight_dtype != MOE_MXFP4 || !gemm_shape_ok(s)) return MOE_ERR_UNSUPPORTED;
    if (s->T == 0) return MOE_OK;
    return check_weights(s, w);
}

int moe_mx_gate_up(const moe_shape* s, const void* x, const int32_t* perm, const int32_t* offsets,
                   const moe_weights* w, uint8_t* a_codes, uint8_t* a_scales, void* ws, size_t ws_bytes,
                   void* stream) {
    int rc = mx_stage_check(s, w);
    if (rc != MOE_OK || s->T == 0) return rc;
    if (!ptr_ok(x) || !ptr_ok(perm) || !ptr_ok(offsets) || !ptr_ok(a_codes) || !ptr_ok(a_scales))
        return MOE_ERR_INVALID_ARG;
    const Layout L = layout(s);
    if (!ws || !aligned16(ws) || ws_bytes < L.total) return MOE_ERR_WORKSPACE;
    hipStream_t st = (hipStream_t)stream;
    const int64_t T = s->T, d = s->d_model;
    uint8_t* xq = at<uint8_t>(ws, L.y);
    MOE_TRY(launch_mx_quant_rows(MOE_BF16, x, xq, xq + T * d, T, d, st));
    MOE_TRY(launch_mxgemm_w13(xq, xq + T * d, perm, offsets, w->w13, w->w13_scale, w->s13, w->s13_scale, a_codes,
                              a_scales, s->T, s->d_model, s->d_ff, s->n_shared ? s->shared_d_ff : 0, s->top_k,
                              s->n_experts, s->n_shared, nullptr, st));
    return MOE_OK;
}

int moe_mx_down(const moe_shape* s, const uint8_t* a_codes, const uint8_t* a_scales, const int32_t* offsets,
                const moe_weights* w, void* y_sorted, void* y_shared, void* stream) {
    int rc = mx_stage_check(s, w);
    if (rc != MOE_OK || s->T == 0) return rc;
    if (!ptr_ok(a_codes) || !ptr_ok(a_scales) || !ptr_ok(offsets) || !ptr_ok(y_sorted)) return MOE_ERR_INVALID_ARG;
    if (s->n_shared ? !ptr_ok(y_shared) : y_shared != nullptr) return MOE_ERR_INVALID_ARG;
    MOE_TRY(launch_mxgemm_w2(a_codes, a_scales, offsets, w->w2, w->w2_scale, w->s2, w->s2_scale, y_sorted, y_shared,
                             false, s->T, s->d_model, s->d_ff, s->n_shared ? s->shared_d_ff : 0, s->top_k,
                             s->n_experts, s->n_shared, nullptr, (hipStream_t)stream));
    return MOE_OK;
}

int moe_combine(const moe_shape* s, const void* y_sorted, const int32_t* inv_perm, const float* topk_w,
                const void* y_shared, void* out, void* stream) {
    int rc = check_shape(s);
    if (rc != MOE_OK) return rc;
    if (s->T == 0) return MOE_OK;
    if (!ptr_ok(y_sorted) || !ptr_ok(inv_perm) || !ptr_ok(topk_w) || !ptr_ok(out)) return MOE_ERR_INVALID_ARG;
    if (y_shared && !aligned16(y_shared)) return MOE_ERR_INVALID_ARG;
    const int dt = s->act_dtype == MOE_BF16 ? 1 : 0;
    MOE_TRY(launch_combine(dt, dt, y_sorted, inv_perm, topk_w, y_shared, out, s->T, s->d_model, s->top_k,
                           (s->flags & MOE_F_ACCUMULATE) != 0, nullptr, nullptr, s->n_experts, (hipStream_t)stream));
    return MOE_OK;
}

// Argument checks of the layer calls (everything but the workspace).
static int check_layer_args(const moe_shape* s, const void* x, const void* w_router, const float* b_router,
                            const moe_weights* w, const uint8_t* expert_mask, bool masked, void* out,
                            int32_t* topk_idx_out) {
    int rc = check_shape(s);
    if (rc != MOE_OK) return rc;
    if (masked && !ptr_ok(expert_mask)) return MOE_ERR_INVALID_ARG;
    if (s->T == 0) return MOE_OK;
    if ((rc = check_weights(s, w)) != MOE_OK) return rc;
    if (!ptr_ok(x) || !ptr_ok(w_router) || !ptr_ok(out)) return MOE_ERR_INVALID_ARG;
    if ((b_router && !aligned16(b_router)) || (topk_idx_out && !aligned16(topk_idx_out))) return MOE_ERR_INVALID_ARG;
    return MOE_OK;
}

static int layer_entry(const moe_shape* s, const void* x, const void* w_router, const float* b_router,
                       const moe_weights* w, const uint8_t* expert_mask, bool masked, void* out,
                       int32_t* topk_idx_out, void* ws, size_t ws_bytes, void* stream) {
    const int rc = check_layer_args(s, x, w_router, b_router, w, expert_mask, masked, out, topk_idx_out);
    if (rc != MOE_OK || s->T == 0) return rc;
    const Layout L = layout(s);
    if (!ws || !aligned16(ws) || ws_bytes < L.total) return MOE_ERR_WORKSPACE;
    return run_layer(s, x, w_router, b_router, w, out, s->act_dtype, (s->flags & MOE_F_ACCUMULATE) != 0,
                     topk_idx_out, ws, L, masked ? expert_mask : nullptr, (hipStream_t)stream);
}

int moe_layer_forward(const moe_shape* s, const void* x, const void* w_router, const float* b_router,
                      const moe_weights* w, void* out, int32_t* topk_idx_out, void* ws, size_t ws_bytes,
                      void* stream) {
    return layer_entry(s, x, w_router, b_router, w, nullptr, false, out, topk_idx_out, ws, ws_bytes, stream);
}

int moe_layer_forward_noalloc(const moe_shape* s, const void* x, const void* w_router, const float* b_router,
                              const moe_weights* w, void* out, int32_t* topk_idx_out, void* stream) {
    const int rc = check_layer_args(s, x, w_router, b_router, w, nullptr, false, out, topk_idx_out);
    if (rc != MOE_OK || s->T == 0) return rc;
    if (layout(s).total > MOE_NOALLOC_SCRATCH_BYTES) return MOE_ERR_SCRATCH_LIMIT;
    void* ws = nullptr;
    if (scratch_ptr(&ws) != hipSuccess) return MOE_ERR_HIP;
    return layer_entry(s, x, w_router, b_router, w, nullptr, false, out, topk_idx_out, ws, MOE_NOALLOC_SCRATCH_BYTES,
                       stream);
}

int moe_layer_forward_masked(const moe_shape* s, const void* x, const void* w_router, const float* b_router,
                             const moe_weights* w, const uint8_t* expert_mask, void* out, int32_t* topk_idx_out,
                             void* ws, size_t ws_bytes, void* stream) {
    return layer_entry(s, x, w_router, b_router, w, expert_mask, true, out, topk_idx_out, ws, ws_bytes, stream);
}

// Layer l's [T, k] block of the stack's optional selection output.
static int32_t* layer_idx(int32_t* base, int l, const moe_shape* s) {
    return base ? base + (int64_t)l * s->T * s->top_k : nullptr;
}

int moe_stack_forward(const moe_shape* s, int32_t n_layers, float* h, const void* const* w_router,
                      const float* const* b_router, const moe_weights* w, int32_t* topk_idx_out, void* ws,
                      size_t ws_bytes, void* stream) {
    int rc = check_shape(s);
    if (rc != MOE_OK) return rc;
    if (n_layers < 0 || !w_router || !w) return MOE_ERR_INVALID_ARG;
    if (s->T == 0 || n_layers == 0) return MOE_OK;
    if (!ptr_ok(h) || (topk_idx_out && !aligned16(topk_idx_out))) return MOE_ERR_INVALID_ARG;
    for (int l = 0; l < n_layers; ++l) {
        if ((rc = check_weights(s, &w[l])) != MOE_OK) return rc;
        if (!ptr_ok(w_router[l])) return MOE_ERR_INVALID_ARG;
        if (b_router && b_router[l] && !aligned16(b_router[l])) return MOE_ERR_INVALID_ARG;
    }
    const Layout L = layout(s);
    if (!ws || !aligned16(ws) || ws_bytes < L.total) return MOE_ERR_WORKSPACE;
    hipStream_t st = (hipStream_t)stream;
    void* xn = at<void>(ws, L.xn);
    if (use_decode(s)) {
        // decode: the logits kernel normalises h itself and leaves x for the FFN kernels
        for (int l = 0; l < n_layers; ++l) {
            rc = run_decode(s, h, w_router[l], b_router ? b_router[l] : nullptr, &w[l], h, MOE_F32, true,
                            layer_idx(topk_idx_out, l, s), true, ws, L, nullptr, st);
            if (rc != MOE_OK) return rc;
        }
        return MOE_OK;
    }
    for (int l = 0; l < n_layers; ++l) {
        MOE_TRY(launch_rmsnorm(s->act_dtype == MOE_BF16 ? 1 : 0, h, xn, s->T, s->d_model, 1e-6f, st));
        rc = run_layer(s, xn, w_router[l], b_router ? b_router[l] : nullptr, &w[l], h, MOE_F32, true,
                       layer_idx(topk_idx_out, l, s), ws, L, nullptr, st);
        if (rc != MOE_OK) return rc;
    }
    return MOE_OK;
}


size_t moe_stack_persistent_workspace_size(const moe_shape* s, int32_t n_layers) {
    if (n_layers < 1 || check_stack_persistent(s) != MOE_OK) return 0;
    return stack_layout(s, n_layers).total;
}

int moe_stack_forward_persistent(const moe_shape* s, int32_t n_layers, float* h, const void* const* w_router,
                                 const float* const* b_router, const moe_weights* w, int32_t* topk_idx_out, void* ws,
                                 size_t ws_bytes, void* stream) {
    int rc = check_shape(s);
    if (rc != MOE_OK) return rc;
    if (n_layers < 0 || !w_router || !w) return MOE_ERR_INVALID_ARG;
    if (s->T == 0 || n_layers == 0) return MOE_OK;
    if ((rc = check_stack_persistent(s)) != MOE_OK) return rc;
    if (!ptr_ok(h) || (topk_idx_out && !aligned16(topk_idx_out))) return MOE_ERR_INVALID_ARG;
    for (int l = 0; l < n_layers; ++l) {
        if ((rc = check_weights(s, &w[l])) != MOE_OK) return rc;
        if (!ptr_ok(w_router[l])) return MOE_ERR_INVALID_ARG;
        if (b_router && b_router[l] && !aligned16(b_router[l])) return MOE_ERR_INVALID_ARG;
    }
    const StackLayout L = stack_layout(s, n_layers);
    if (!ws || !aligned16(ws) || ws_bytes < L.total) return MOE_ERR_WORKSPACE;
    hipStream_t st = (hipStream_t)stream;
    StackLayerPtrs lp[STACK_LAYERS_PER_LAUNCH];
    for (int l0 = 0; l0 < n_layers; l0 += L.lc) {
        const int n = n_layers - l0 < L.lc ? n_layers - l0 : L.lc;
        for (int j = 0; j < n; ++j) {
            const moe_weights& wl = w[l0 + j];
            lp[j] = StackLayerPtrs{w_router[l0 + j], b_router ? b_router[l0 + j] : nullptr, wl.w13, wl.w13_scale, wl.w2,
                                   wl.w2_scale};
        }
        const hipError_t e = launch_dec_stack(
            lp, n, h, at<float>(ws, L.hbuf), at<float>(ws, L.logits), at<uint16_t>(ws, L.xn), at<float>(ws, L.a),
            topk_idx_out ? topk_idx_out + (int64_t)l0 * s->top_k : nullptr, at<int>(ws, L.bar), L.sh_h, L.sh_lg,
            L.sh_xn, L.sh_a, s->d_model, s->d_ff, s->n_experts, s->top_k, (s->flags & MOE_F_NO_RENORM) != 0,
            g_stack_spin_limit, l0 == 0, st);
        if (e != hipSuccess) return MOE_ERR_HIP;
    }
    return MOE_OK;
}

int moe_stack_persistent_status(const void* ws, int32_t* status, void* stream) {
    if (!ws || !aligned16(ws) || !status) return MOE_ERR_INVALID_ARG;
    hipStream_t st = (hipStream_t)stream;
    int32_t v = 0;
    const char* p = reinterpret_cast<const char*>(ws) + (size_t)dec_stack_err_index() * 4;
    if (hipMemcpyAsync(&v, p, sizeof v, hipMemcpyDeviceToHost, st) != hipSuccess) return MOE_ERR_HIP;
    if (hipStreamSynchronize(st) != hipSuccess) return MOE_ERR_HIP;
    *status = v;
    return MOE_OK;
}

int moe_stack_persistent_set_spin_limit(int32_t spins) {
    if (spins < 0) return MOE_ERR_INVALID_ARG;
    g_stack_spin_limit = spins;
    return MOE_OK;
}

int moe_profile_kernel(int kernel, void* ev_start, void* ev_stop) {
    if (kernel < -1 || kernel > MOE_KERNEL_FFN_DOWN) return MOE_ERR_INVALID_ARG;
    if (kernel >= 0 && (!ev_start || !ev_stop)) return MOE_ERR_INVALID_ARG;
    g_prof_kernel = kernel;
    g_prof_start = (hipEvent_t)ev_start;
    g_prof_stop = (hipEvent_t)ev_stop;
    return MOE_OK;
}

int moe_mxfp4_dequant(const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t K, float* out, void* stream) {
    if (rows < 0 || K < 0 || K % 32 != 0) return MOE_ERR_INVALID_ARG;
    if (rows == 0 || K == 0) return MOE_OK;
    if (!ptr_ok(codes) || !scales || !ptr_ok(out)) return MOE_ERR_INVALID_ARG;
    MOE_TRY(launch_mxfp4_dequant(codes, scales, out, rows, K, (hipStream_t)stream));
    return MOE_OK;
}

int moe_nvfp4_dequant(const uint8_t* codes, const uint8_t* scales, float gscale, int64_t rows, int64_t K, float* out,
                      void* stream) {
    if (rows < 0 || K < 0 || K % 32) return MOE_ERR_INVALID_ARG;
    if (rows == 0 || K == 0) return MOE_OK;
    if (!ptr_ok(codes) || !scales || ((uintptr_t)scales & 1) || !ptr_ok(out)) return MOE_ERR_INVALID_ARG;
    MOE_TRY(launch_nvfp4_dequant(codes, scales, gscale, out, rows, K, (hipStream_t)stream));
    return MOE_OK;
}

int moe_mxfp8_quantize(const void* x, int32_t x_dtype, int64_t rows, int64_t K, uint8_t* codes, uint8_t* scales,
                       void* stream) {
    if (rows < 0 || K < 0 || K % 32 || (x_dtype != MOE_F32 && x_dtype != MOE_BF16)) return MOE_ERR_INVALID_ARG;
    if (rows == 0 || K == 0) return MOE_OK;
    if (!ptr_ok(x) || !ptr_ok(codes) || !scales) return MOE_ERR_INVALID_ARG;
    MOE_TRY(launch_mx_quant_rows(x_dtype, x, codes, scales, rows, K, (hipStream_t)stream));
    return MOE_OK;
}

}  // extern "C"
