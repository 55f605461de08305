/*
 * moe.h -- C-ABI of the MI355X (gfx950) routed mixture-of-experts layer.
 *
 * The layer is the sparse hot path the FreeToken pages describe: every token
 * activates k of E routed experts per layer (DeepSeek-V4-Flash: 6 of 256 in
 * each of 43 layers; dothoosh.com FreeToken article, "FreeToken architecture
 * and the sparsity puzzle"; aihot.vn FreeToken article, "The gap it
 * targets"), optionally beside one always-on shared expert (8 of 128 routed
 * plus 1 shared; dothoosh.com TurboFieldfare article, "Background: Gemma 4
 * 26B A4B"), with BF16 or MXFP4 expert weights (dothoosh.com FreeToken
 * article, "Benchmarks and real performance"), and the partial sums of the
 * experts merge exactly (same article, mechanism 1, the q* policy).  The
 * pages give no formulas; this library computes the plain dropless top-k
 * reading:
 *   logits  l[t,e] = x[t] . W_r[e] + b[e]                        (fp32)
 *   select  the k largest l[t,.], equal logits -> lower expert index,
 *           NaN below every number, +0 == -0; topk_idx in that order
 *   gates   g = softmax over the k selected logits (MOE_F_NO_RENORM: the
 *           full softmax over all E, read at the selected experts)
 *   expert  y_e(x) = W2_e (silu(Wg_e x) * (Wu_e x))   (SwiGLU)
 *   out[t]  = sum over the token's experts, ascending expert index, of
 *             g * y_e(x[t]), + shared(x[t]) when n_shared = 1
 *
 * Conventions for every entry point:
 *  - `shape`, `weights` and arrays of pointers are HOST memory; every other
 *    pointer is DEVICE memory owned by the caller, 16-byte aligned.
 *  - Calls validate all arguments on the host first; on any failure they
 *    return a negative moe_status and enqueue nothing.  On success they
 *    enqueue kernels on `stream` (a hipStream_t; NULL = the null stream) and
 *    return without synchronising.  HIP launch errors come back as
 *    MOE_ERR_HIP; faults inside kernels surface at the caller's next
 *    synchronisation.
 *  - The library allocates no device memory: scratch space comes from the
 *    caller's workspace `ws` of at least moe_workspace_size(shape) bytes.
 *    Calls that share a workspace must not overlap in time.
 *  - T = 0 is a valid empty batch: MOE_OK, nothing enqueued.
 *  - Results are deterministic run to run (fixed summation orders, no
 *    floating-point atomics).
 *
 * Tensor layouts (row-major, last index contiguous):
 *   x, out        [T, d_model]          act dtype (f32 or bf16)
 *   w_router      [E, d_model]          act dtype;  b_router [E] f32 (may be NULL = 0)
 *   w13           [E, 2*d_ff, d_model]  rows 0..d_ff-1 gate, d_ff..2*d_ff-1 up
 *   w2            [E, d_model, d_ff]
 *   s13, s2       shared expert, same layout with E = 1 and shared_d_ff
 *   MXFP4 weights: codes [.., N, K/2] uint8, element 2i in the LOW nibble of
 *     byte i, E2M1 per the OCP Microscaling v1.0 specification; scales
 *     [.., N, K/32] uint8 E8M0 (2^(s-127); 0xFF = NaN), one per 32
 *     consecutive elements of a row.
 *   NVFP4 weights (the 4-bit build named in the aihot.vn FreeToken article,
 *     "Flags", and the dothoosh.com FreeToken article, "Editorial"; the pages
 *     give no layout, so this library takes NVIDIA's published one): codes as
 *     for MXFP4; scales [.., N, K/16] uint8 OCP FP8 E4M3 (no infinities;
 *     0x7F/0xFF = NaN), one per 16 consecutive elements; one fp32 scale per
 *     tensor (moe_weights.*_gscale).  Element value = E2M1 * E4M3 * gscale.
 *     d_model, d_ff and shared_d_ff must be multiples of 32 for both 4-bit
 *     formats.  NVFP4 weights take the grouped-GEMV kernels at every T.
 *   topk_idx [T, k] int32, topk_w [T, k] f32, logits [T, E] f32
 *   counts [E], offsets [E+1], perm [T*k], inv_perm [T*k] int32
 *   y_sorted [T*k, d_model], y_shared [T, d_model]  act dtype
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MOE_OK = 0,
    MOE_ERR_INVALID_ARG = -1,  /* NULL/misaligned pointer, k not in [1,E], negative sizes, ... */
    MOE_ERR_UNSUPPORTED = -2,  /* valid but not implemented: dtype pair, E > 1024, k > 64, ... */
    MOE_ERR_WORKSPACE = -3,    /* ws_bytes < moe_workspace_size(shape) */
    MOE_ERR_HIP = -4,          /* a HIP launch reported an error */
    MOE_ERR_SCRATCH_LIMIT = -5 /* moe_layer_forward_noalloc: the shape needs more scratch than it holds */
} moe_status;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1, MOE_MXFP4 = 2, MOE_NVFP4 = 3 } moe_dtype;

enum {
    MOE_F_NO_RENORM = 1u << 0,   /* gates = full-softmax probabilities at the selected experts */
    MOE_F_ACCUMULATE = 1u << 1,  /* out += layer(x) instead of out = layer(x) */
    MOE_F_FORCE_GEMV = 1u << 3,  /* use the decode (grouped GEMV) kernels at any T */
    MOE_F_FORCE_GEMM = 1u << 4,  /* use the prefill (grouped MFMA GEMM) kernels at any T */
    /* MXFP4 weights only (else MOE_ERR_UNSUPPORTED): where the grouped MFMA GEMM kernels run
       (T > 32, or MOE_F_FORCE_GEMM), run them on the fp8 x fp4 scaled matrix cores, with x and
       the SwiGLU output a quantised to MXFP8 (OCP Microscaling Formats v1.0: E4M3 elements,
       one E8M0 scale floor(log2 max|v|) - 8 per 32 consecutive elements along K, round to
       nearest even, magnitudes above 448 clamped to 448) before each contraction.  This is an
       approximation of the layer (a few percent relative error); the decode kernels (T <= 32)
       ignore the flag and stay exact. */
    MOE_F_MX_GEMM = 1u << 5
};

/* Limits of this implementation (MOE_ERR_UNSUPPORTED beyond them). */
#define MOE_MAX_EXPERTS 1024
#define MOE_MAX_TOPK 64

typedef struct {
    int32_t T;            /* tokens in the batch */
    int32_t d_model;
    int32_t d_ff;         /* routed expert hidden size */
    int32_t n_experts;    /* E, routed experts */
    int32_t top_k;        /* k */
    int32_t n_shared;     /* 0 or 1 always-on shared expert (weight 1, no gate) */
    int32_t shared_d_ff;
    int32_t act_dtype;    /* moe_dtype: MOE_F32 or MOE_BF16 */
    int32_t weight_dtype; /* moe_dtype: MOE_F32 (with f32 act); MOE_BF16, MOE_MXFP4 or MOE_NVFP4 (bf16 act) */
    uint32_t flags;       /* MOE_F_* */
} moe_shape;

typedef struct {
    const void* w13;           /* [E, 2f, d] (MXFP4/NVFP4: codes [E, 2f, d/2]) */
    const void* w2;            /* [E, d, f]  (MXFP4/NVFP4: codes [E, d, f/2]) */
    const uint8_t* w13_scale;  /* MXFP4: [E, 2f, d/32]; NVFP4: [E, 2f, d/16]; else unused */
    const uint8_t* w2_scale;   /* MXFP4: [E, d, f/32];  NVFP4: [E, d, f/16];  else unused */
    const void* s13;           /* shared expert (n_shared = 1), else NULL */
    const void* s2;
    const uint8_t* s13_scale;
    const uint8_t* s2_scale;
    float w13_gscale, w2_gscale, s13_gscale, s2_gscale; /* NVFP4 only: per-tensor fp32 scales */
} moe_weights;

/* Bytes of device workspace the calls below need for this shape (0 on an invalid shape).
   The contents of a workspace need no initialisation: every call writes each region it
   reads before reading it. */
size_t moe_workspace_size(const moe_shape* shape);

/* Static description of a status code. */
const char* moe_status_string(int status);

/* Router: logits -> top-k selection -> gates.  Each token activates k of the E routed
   experts of the layer and the choice changes from token to token (dothoosh.com FreeToken
   article, "FreeToken architecture and the sparsity puzzle": 6 of 256 experts per layer;
   aihot.vn FreeToken article, "The gap it targets").  The pages give no gating formula; the
   plain top-k softmax reading is computed: the k largest logits (ties -> lower expert index,
   NaN below every number, +0 == -0), gates = softmax over those k (MOE_F_NO_RENORM: the full
   softmax read at them).
   logits_in: NULL -> logits are computed from x, w_router, b_router; else a [T,E] f32
   array used as the logits (x, w_router, b_router ignored).  logits_out (nullable)
   receives the logits used.  topk_idx [T,k] in descending-logit order, topk_w [T,k].
   Errors: INVALID_ARG for a bad shape or a NULL/misaligned required pointer, WORKSPACE for
   a short workspace; nothing is enqueued then. */
int moe_route(const moe_shape* shape, const void* x, const void* w_router, const float* b_router,
              const float* logits_in, int32_t* topk_idx, float* topk_w, float* logits_out,
              void* ws, size_t ws_bytes, void* stream);

/* Grouping of tokens by expert.  A prefill batch sends thousands of tokens to nearly every
   expert at once (dothoosh.com FreeToken article, "FreeToken architecture and the sparsity
   puzzle", the first failure mode of per-token expert caching), so the pairs are grouped per
   expert before the expert FFNs run as one grouped GEMM: a stable counting sort of the flat
   pairs p = t*k + j by expert id.  counts[e] [E], offsets = exclusive prefix sum [E+1],
   perm [T*k] = pairs in ascending (expert, p) order, inv_perm[perm[i]] = i (all int32,
   device).  Every topk_idx entry must lie in [0, E) (not checked on the device).  Errors as
   moe_route. */
int moe_permute(const moe_shape* shape, const int32_t* topk_idx, int32_t* counts, int32_t* offsets,
                int32_t* perm, int32_t* inv_perm, void* ws, size_t ws_bytes, void* stream);

/* Expert SwiGLU FFNs on the grouped pairs.  Only the selected experts compute, each over the
   tokens routed to it (dothoosh.com FreeToken article, "FreeToken architecture and the
   sparsity puzzle": 13B of 284B parameters active per token), with BF16 or 4-bit expert
   weights (same article, "Benchmarks and real performance": MXFP4), beside the always-on
   shared expert when n_shared = 1 (dothoosh.com TurboFieldfare article, "Background: Gemma 4
   26B A4B": 8 of 128 routed + 1 shared).  y_sorted[i] = y_e(x[perm[i] / k]) for the expert e
   whose segment [offsets[e], offsets[e+1]) holds slot i, y_e(v) = W2_e (silu(Wg_e v) *
   (Wu_e v)); y_shared[t] = shared(x[t]) (NULL if n_shared = 0).  perm/offsets as produced by
   moe_permute (a slot outside every segment is left unwritten).  T <= 32 runs the grouped
   GEMV kernels, larger T the grouped MFMA GEMM (MOE_F_FORCE_* override).  Errors as
   moe_route, plus INVALID_ARG for missing weight or scale pointers. */
int moe_grouped_ffn(const moe_shape* shape, const void* x, const int32_t* perm, const int32_t* offsets,
                    const moe_weights* weights, void* y_sorted, void* y_shared,
                    void* ws, size_t ws_bytes, void* stream);

/* Gate-weighted combine.  The experts' partial results add up exactly to the layer's output
   (dothoosh.com FreeToken article, "FreeToken architecture and the sparsity puzzle",
   mechanism 1: the GPU's and the CPU's partial sums merge with no estimate; ai4bro.com
   FreeToken article, "Key points").  out[t] = sum over j in ascending expert order
   (= ascending inv_perm[t*k+j]) of topk_w[t,j] * y_sorted[inv_perm[t*k+j]],
   + y_shared[t] (nullable), accumulated in fp32 and rounded once to the act dtype; with
   MOE_F_ACCUMULATE added to out.  Uses no workspace.  Errors as moe_route. */
int moe_combine(const moe_shape* shape, const void* y_sorted, const int32_t* inv_perm, const float* topk_w,
                const void* y_shared, void* out, void* stream);

/* Whole layer (router to combine), fusing where it pays (at decode the combine is
   fused into the down projection).  topk_idx_out (nullable) receives [T,k]. */
int moe_layer_forward(const moe_shape* shape, const void* x, const void* w_router, const float* b_router,
                      const moe_weights* weights, void* out, int32_t* topk_idx_out,
                      void* ws, size_t ws_bytes, void* stream);

/* moe_layer_forward for callers that cannot allocate device memory (code under HIP graph
   capture, tight serving loops, harnesses that forbid allocation): the same kernels and
   results, with the workspace taken from a scratch area the library holds in device memory
   instead of from the caller.  The scratch area is MOE_NOALLOC_SCRATCH_BYTES (64 MiB) per GPU,
   set up on the first call on each device (its address is looked up, nothing is allocated)
   and kept until the process ends.  Shapes whose moe_workspace_size exceeds it (prefill
   batches of more than a few hundred tokens at the benchmark shapes) return
   MOE_ERR_SCRATCH_LIMIT with nothing enqueued; use moe_layer_forward with a caller workspace
   for those.  No kernel needs the scratch area zeroed, and every call rewrites what it reads.
   All calls on one GPU share its scratch area, so calls that overlap in time on one GPU (two
   streams, two threads) race and must be serialised by the caller.  The call itself performs
   no allocation (no hipMalloc, no hipFree, no allocating library routine).  Other arguments
   and errors as moe_layer_forward. */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int moe_layer_forward_noalloc(const moe_shape* shape, const void* x, const void* w_router, const float* b_router,
                              const moe_weights* weights, void* out, int32_t* topk_idx_out, void* stream);

/* Partial layer (the exact merge of partial expert sums; FreeToken/dothoosh, "Architecture and
   the sparsity puzzle", mechanism 1: the GPU's and the CPU's partial results add up to the
   whole): moe_layer_forward with the combine restricted to the experts whose byte in
   expert_mask is nonzero.  expert_mask: DEVICE, E + 1 bytes (routed experts 0..E-1, then the
   shared expert), 16-byte aligned.  Routing (selection and gates) is over all E experts as in
   the full layer; the FFNs of masked-out experts are not computed.  With MOE_F_ACCUMULATE,
   calls over disjoint masks whose union is every expert sum to the full layer (up to fp32
   rounding of the additions).  Errors as moe_layer_forward; a NULL mask is INVALID_ARG. */
int moe_layer_forward_masked(const moe_shape* shape, const void* x, const void* w_router, const float* b_router,
                             const moe_weights* weights, const uint8_t* expert_mask, void* out,
                             int32_t* topk_idx_out, void* ws, size_t ws_bytes, void* stream);

/* Residual stack of n_layers MoE layers on the fp32 residual stream
   h [T, d_model] (DeepSeek-V4-Flash: 43 layers, each routing 6 of 256 experts afresh;
   dothoosh.com FreeToken article, "FreeToken architecture and the sparsity puzzle"): for
   each layer l, x = act(h / sqrt(mean(h^2) + 1e-6)) rounded to the act dtype, then
   h += layer_l(x) in fp32.  w_router, b_router and weights are HOST arrays of n_layers
   entries (each holding device pointers); b_router may be NULL.  Routing is recomputed in
   every layer; topk_idx_out (nullable, DEVICE [n_layers, T, k] int32) receives each layer's
   selection.  Errors as moe_layer_forward. */
int moe_stack_forward(const moe_shape* shape, int32_t n_layers, float* h, const void* const* w_router,
                      const float* const* b_router, const moe_weights* weights, int32_t* topk_idx_out,
                      void* ws, size_t ws_bytes, void* stream);

/* moe_stack_forward for one token as ONE persistent launch per 48 layers (the 43-layer decode
   of DeepSeek-V4-Flash, 6 of 256 experts per layer; dothoosh.com FreeToken article, "FreeToken
   architecture and the sparsity puzzle"): the same three steps per layer and the same results
   bit for bit, with grid-wide barriers between them instead of kernel boundaries.  Supported:
   T = 1, bf16 activations, MXFP4 weights, no shared expert, d_model <= 4096 and d_ff <= 2048
   (multiples of 32); else MOE_ERR_UNSUPPORTED with nothing enqueued.  The launch is cooperative
   (all workgroups resident); a barrier wait that runs out of polls (moe_stack_persistent_set_spin_limit,
   default 2^20, about a second) makes every workgroup leave, the call's results are then
   undefined and moe_stack_persistent_status reports 1.  ws: at least
   moe_stack_persistent_workspace_size(shape, n_layers) bytes (0 = unsupported shape), no
   initialisation needed.  Other arguments and errors as moe_stack_forward. */
size_t moe_stack_persistent_workspace_size(const moe_shape* shape, int32_t n_layers);
int moe_stack_forward_persistent(const moe_shape* shape, int32_t n_layers, float* h, const void* const* w_router,
                                 const float* const* b_router, const moe_weights* weights, int32_t* topk_idx_out,
                                 void* ws, size_t ws_bytes, void* stream);
/* Synchronises `stream`, then *status = 0 (the last moe_stack_forward_persistent on ws ran to
   the end) or 1 (a barrier wait ran out).  INVALID_ARG for a NULL or misaligned ws or NULL
   status; HIP for a failed copy. */
int moe_stack_persistent_status(const void* ws, int32_t* status, void* stream);
/* Polls of one barrier wait before moe_stack_forward_persistent gives up (>= 0; 0 gives up at
   the first wait that has to poll).  Process-wide; for tests of the time-out path. */
int moe_stack_persistent_set_spin_limit(int32_t spins);

/* MXFP4 -> f32 dequantisation on its own: out[r*K + j] =
   (-1)^b3 * M[code & 7] * 2^(s - 127) with M = {0, .5, 1, 1.5, 2, 3, 4, 6},
   NaN for s = 0xFF; codes [rows, K/2], scales [rows, K/32]; K % 32 == 0. */
int moe_mxfp4_dequant(const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t K, float* out,
                      void* stream);

/* NVFP4 -> f32 dequantisation: out[r*K + j] = E2M1(code) * E4M3(scales[r*(K/16) + j/16])
   * gscale, rounded once to f32 (NaN for a NaN scale); codes [rows, K/2], scales
   [rows, K/16]; K % 32 == 0.  MOE_ERR_INVALID_ARG otherwise. */
int moe_nvfp4_dequant(const uint8_t* codes, const uint8_t* scales, float gscale, int64_t rows, int64_t K,
                      float* out, void* stream);

/* Rows -> MXFP8, the activation quantisation of MOE_F_MX_GEMM on its own (OCP Microscaling
   Formats v1.0): for each 32-element block of a row, scale byte = max(biased exponent of the
   block's largest magnitude - 8, 0) (E8M0: floor(log2 max|v|) - 8), codes = E4M3(v / 2^(s-127))
   rounded to nearest even with magnitudes above 448 clamped to 448; a block holding an infinity
   or NaN gets scale 0xFF and NaN codes 0x7F.  x [rows, K] f32 or bf16 (x_dtype MOE_F32 /
   MOE_BF16), codes [rows, K], scales [rows, K/32]; K % 32 == 0. */
int moe_mxfp8_quantize(const void* x, int32_t x_dtype, int64_t rows, int64_t K, uint8_t* codes, uint8_t* scales,
                       void* stream);

/* The two contractions of the MOE_F_MX_GEMM path as separate calls (MXFP4 weights, bf16
   activations, d_model, d_ff and shared_d_ff multiples of 128; else MOE_ERR_UNSUPPORTED).
   moe_mx_gate_up: x quantised to MXFP8 (as moe_mxfp8_quantize), then for every sorted slot i
   (perm/offsets as from moe_permute) and the shared expert, a = silu(Wg x) * (Wu x) on the fp8 x
   fp4 matrix cores, quantised to MXFP8 per 32 consecutive elements: a_codes [T*k*f + T*f_s]
   bytes (slot rows of f, then the shared rows of f_s), a_scales [(T*k*f + T*f_s)/32].  Uses the
   workspace.  moe_mx_down: y_sorted [T*k, d] and y_shared [T, d] (bf16) from those codes and
   scales. */
int moe_mx_gate_up(const moe_shape* shape, const void* x, const int32_t* perm, const int32_t* offsets,
                   const moe_weights* weights, uint8_t* a_codes, uint8_t* a_scales, void* ws, size_t ws_bytes,
                   void* stream);
int moe_mx_down(const moe_shape* shape, const uint8_t* a_codes, const uint8_t* a_scales, const int32_t* offsets,
                const moe_weights* weights, void* y_sorted, void* y_shared, void* stream);

/* Timing aid for benchmarks: while set, every launch of the given kernel class carries
   ev_start / ev_stop on its own dispatch (hipExtLaunchKernel), so the events hold that
   kernel's start and end timestamps; with several such launches in one call (the stack),
   the last one's remain.
   kernel: MOE_KERNEL_FFN_UP (gate/up projection + SwiGLU, the largest byte/flop share),
   MOE_KERNEL_FFN_DOWN (down projection), or -1 to switch the hook off (events ignored).
   ev_start/ev_stop are hipEvent_t handles owned by the caller.  The setting is
   process-wide and not synchronised: set it only while no other thread calls the library. */
enum { MOE_KERNEL_FFN_UP = 0, MOE_KERNEL_FFN_DOWN = 1 };
int moe_profile_kernel(int kernel, void* ev_start, void* ev_stop);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H */
