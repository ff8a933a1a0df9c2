/*
 * moe.h -- C ABI of libmoe: the forward pass of one Hunyuan-style
 * mixture-of-experts layer on an AMD Instinct MI355X (gfx950).
 *
 * The layer (Hy3 on CANN NPU guide, section 1 and section 8.5; Hy4-preview
 * tutorial, section 1; HunyuanImage-3.0 multi-stream article, source
 * walkthrough parts 1-3):
 *
 *   s      = sigmoid(x W_r^T + b)                         gating scores
 *   idx    = the top-k experts of each token by s          (ties: lower index;
 *                                                           a NaN s counts as 0)
 *   w      = rho * s[idx] / sum(s[idx])                    route_norm, scaling
 *   y_e    = W_d,e ( silu(W_g,e x) * (W_u,e x) )           SwiGLU expert FFN
 *   out    = sum_j w_j y_idx_j(x)  +  FFN_shared(x)        combine + shared
 *
 * computed as Gating -> InitRouting (permutation) -> grouped GEMM ->
 * FinalizeRouting (weighted combine) -> add of the always-on shared expert,
 * which runs on a second stream joined by an event where that pays (see
 * moe_layer_forward).
 *
 * Conventions for every call:
 *  - Pointers are DEVICE pointers unless marked "host".  The caller owns all
 *    memory; the library never allocates device memory after moe_ctx_create
 *    (which creates two events) and never frees caller memory.
 *  - Activations, outputs, workspaces, router weights and packed expert
 *    weights are read or written with 16-byte vector accesses and must start
 *    16-byte aligned (any allocation is); a misaligned one returns
 *    MOE_ERR_INVALID_ARG.  The sources of moe_mx_quantize, moe_fp8_quantize
 *    and moe_pack_experts and moe_permute's topk_idx may be unaligned.
 *  - Streams are hipStream_t handles passed as void* (NULL = the null stream).
 *    Calls enqueue work on the given stream and return without synchronising;
 *    results are ready when that stream reaches the point of the call.
 *  - Arguments are validated before anything is enqueued.  A failed validation
 *    returns MOE_ERR_INVALID_ARG / MOE_ERR_UNSUPPORTED / MOE_ERR_WORKSPACE and
 *    enqueues nothing.  T == 0 returns MOE_OK and enqueues nothing; T * top_k
 *    above 2^31 - 1 (the int32 pair indices) returns MOE_ERR_UNSUPPORTED.  A HIP
 *    launch error returns MOE_ERR_DEVICE (text in moe_ctx_last_error).  Faults
 *    inside kernels surface at the caller's next synchronisation, as with any
 *    HIP library.  No call aborts or throws.
 *  - Outputs are bit-identical from run to run for identical inputs (no
 *    floating-point atomics; fixed reduction orders).
 *  - A moe_ctx may be used by one host thread at a time.
 *
 * Shape limits: 1 <= E <= 1024, 1 <= k <= min(E, 16); H a multiple of 256;
 * I and I_s multiples of 128 (256 for MX-fp8 and MXFP4); I_s = 0 means no
 * shared expert.
 */
#ifndef MOE_H_
#define MOE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_API __attribute__((visibility("default")))

typedef enum moe_status {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1, /* null pointer, bad size, bad enum            */
  MOE_ERR_UNSUPPORTED = 2, /* valid but not implemented (dtype combination) */
  MOE_ERR_WORKSPACE = 3,   /* workspace smaller than moe_workspace_bytes() */
  MOE_ERR_DEVICE = 4       /* a HIP call failed                            */
} moe_status;

typedef enum moe_dtype {
  MOE_F32 = 0,   /* IEEE binary32                                           */
  MOE_BF16 = 1,  /* bfloat16, round-to-nearest-even on every store          */
  MOE_MXFP8 = 2, /* OCP MX: E4M3 (FN) elements, one E8M0 scale per 32       */
  MOE_MXFP4 = 3, /* OCP MX: E2M1 elements (two per byte, low nibble first),
                    one E8M0 scale per 32; expert weights only (W4A8)      */
  MOE_FP8 = 4    /* E4M3 (FN) with one static fp32 scale per tensor        */
} moe_dtype;

/* Layer description (host struct).  Field names follow HYV3Config (Hy3 guide,
 * section 1).  Supported dtype combinations (act, expert, out):
 *   (F32, F32, F32)     all-fp32 layer
 *   (BF16, BF16, BF16)  bf16 activations and experts, fp32 accumulation
 *   (BF16, MXFP8, BF16) MX-fp8 experts; activations x and the SwiGLU output
 *                       are quantised to MX-fp8 on the fly (32-element blocks
 *                       along the reduction axis); bf16 output
 *   (BF16, MXFP4, BF16) W4A8, the hybrid recipe of the Hy3 guide, section 8.2:
 *                       routed experts MXFP4 (scale X = floor(log2 max|v|) - 2,
 *                       E2M1 round-to-nearest-even, saturating at 6), the
 *                       shared expert MX-fp8 (W8A8), activations MX-fp8 as
 *                       above; bf16 output
 *   (BF16, FP8, BF16)   static per-tensor FP8 W8A8 (the FP8 checkpoints of the
 *                       Hy3 guide, section 2, and the Hy4 tutorial's w8a8
 *                       weights): every expert weight matrix has one fp32
 *                       scale max|w| / 448 (computed by moe_pack_experts);
 *                       x and h are quantised with the fixed activation
 *                       scales fp8_x_scale / fp8_h_scale / fp8_sh_h_scale;
 *                       codes are E4M3 of fp32(v / scale), round to nearest
 *                       even, saturating; products are scaled by weight scale
 *                       x activation scale after fp32 accumulation
 * The router always runs in fp32 on the unquantised x. */
typedef struct moe_desc {
  int32_t hidden;                /* H                                        */
  int32_t num_experts;           /* E routed experts                         */
  int32_t top_k;                 /* k (num_experts_per_tok)                  */
  int32_t inter;                 /* I, routed expert intermediate size       */
  int32_t shared_inter;          /* I_s, 0 = no shared expert                */
  float router_scaling_factor;   /* rho, multiplies the routed weights only  */
  int32_t route_norm;            /* 1: divide selected scores by their sum   */
  int32_t act_dtype;             /* moe_dtype of x                           */
  int32_t expert_dtype;          /* moe_dtype of the packed expert weights   */
  int32_t out_dtype;             /* moe_dtype of y, shared output and out    */
  /* static activation scales (> 0), read only when expert_dtype == MOE_FP8:
   * x (routed and shared experts), the routed SwiGLU output h, and the
   * shared expert's h */
  float fp8_x_scale, fp8_h_scale, fp8_sh_h_scale;
} moe_desc;

/* Device pointers to the layer's weights (host struct). */
typedef struct moe_weights {
  const float *router_w;           /* [E,H] fp32, row-major                 */
  const float *router_bias;        /* [E] fp32 logit bias, or NULL          */
  const void *gate_up;             /* routed gate+up, packed (moe_pack_experts) */
  const void *down;                /* routed down, packed                   */
  const uint8_t *gate_up_scale;    /* MX: packed E8M0 scales; FP8: fp32 per-tensor
                                      scales [E][2] (gate, up), down [E]; else NULL */
  const uint8_t *down_scale;
  const void *sh_gate_up;          /* shared expert, packed with shared = 1 */
  const void *sh_down;
  const uint8_t *sh_gate_up_scale;
  const uint8_t *sh_down_scale;
} moe_weights;

typedef struct moe_ctx moe_ctx;

/* Create a context on HIP device `device`.  `side_stream` (borrowed, never
 * destroyed by the library) is where moe_layer_forward runs the shared
 * expert; NULL runs it on the caller's stream.  The context owns two HIP
 * events (the input-ready and shared-done events of the HunyuanImage-3.0
 * article, source walkthrough part 3).  Returns MOE_ERR_DEVICE if the device
 * is not a gfx950 GPU. */
MOE_API moe_status moe_ctx_create(int device, void *side_stream, moe_ctx **out /* host */);
MOE_API moe_status moe_ctx_destroy(moe_ctx *ctx);

/* Static text for a status code; never NULL. */
MOE_API const char *moe_status_string(moe_status s);
/* Text of the last HIP error seen by calls on ctx ("" if none). */
MOE_API const char *moe_ctx_last_error(const moe_ctx *ctx);

/* Workspace sizes in bytes for a call with T tokens.
 * which: MOE_WS_ROUTE, MOE_WS_PERMUTE, MOE_WS_GROUPED_FFN (routed, shared=0),
 * MOE_WS_SHARED_FFN (shared=1), MOE_WS_LAYER.  0 on invalid arguments. */
enum { MOE_WS_ROUTE = 0, MOE_WS_PERMUTE = 1, MOE_WS_GROUPED_FFN = 2, MOE_WS_SHARED_FFN = 3,
       MOE_WS_LAYER = 4 };
MOE_API size_t moe_workspace_bytes(const moe_desc *desc /* host */, int32_t T, int which);

/* Packed weight sizes in bytes.  shared: 0 routed experts, 1 shared expert.
 * which: MOE_PACK_GATE_UP, MOE_PACK_DOWN, MOE_PACK_GATE_UP_SCALE,
 * MOE_PACK_DOWN_SCALE (scales are 0 bytes unless expert_dtype is MX-fp8,
 * MXFP4 or FP8; the shared expert of an MXFP4 layer is packed as MX-fp8;
 * FP8 scales are fp32, 2 per expert for gate/up and 1 for down). */
enum { MOE_PACK_GATE_UP = 0, MOE_PACK_DOWN = 1, MOE_PACK_GATE_UP_SCALE = 2,
       MOE_PACK_DOWN_SCALE = 3 };
MOE_API size_t moe_packed_bytes(const moe_desc *desc /* host */, int shared, int which);

/* Pack expert weights into the kernels' layout (the FusedMoEGMM weight of
 * the HunyuanImage-3.0 article, part 1, built from per-expert [out,in]
 * matrices).  Inputs, row-major, src_dtype MOE_F32 or MOE_BF16:
 *   gate [E,I,H], up [E,I,H], down [E,H,I]   (shared: E = 1, I = I_s)
 * Outputs in desc->expert_dtype (MX-fp8 for the shared expert of an MXFP4
 * layer): gate_up_out, down_out, and for MX formats the scale arrays
 * (quantised here: OCP MX rule, blocks of 32 along the reduction axis).
 * Sizes from moe_packed_bytes.  Layout: 4 KiB blocks of 16 output rows x 256
 * bytes of K (MXFP4: 2 KiB blocks of 16 rows x 256 K elements), ordered
 * [expert][row block][K chunk]; gate and up row blocks alternate (gate
 * block j, then up block j). */
MOE_API moe_status moe_pack_experts(const moe_desc *desc /* host */, int shared, int src_dtype,
                            const void *gate, const void *up, const void *down,
                            void *gate_up_out, void *down_out, uint8_t *gate_up_scale_out,
                            uint8_t *down_scale_out, void *stream);

/* MX-fp8 quantisation of a row-major [rows, cols] matrix along its rows
 * (cols a multiple of 32): q [rows, cols] E4M3 codes, scale [rows, cols/32]
 * E8M0 bytes.  src_dtype MOE_F32 or MOE_BF16.  OCP MX v1.0 rule: X =
 * floor(log2 max|v|) - 8 clamped to [-127, 127] (zero blocks: -127), codes
 * = E4M3 round-to-nearest-even of v / 2^X saturated to +-448. */
MOE_API moe_status moe_mx_quantize(const void *src, int src_dtype, int64_t rows, int64_t cols,
                           uint8_t *q, uint8_t *scale, void *stream);

/* Static per-tensor FP8 quantisation of n elements (n a multiple of 8):
 * q[i] = E4M3 (FN) of fp32(src[i] / scale), round to nearest even,
 * saturating to +-448.  src_dtype MOE_F32 or MOE_BF16; scale > 0 (host). */
MOE_API moe_status moe_fp8_quantize(const void *src, int src_dtype, int64_t n, float scale,
                            uint8_t *q, void *stream);

/* Gating (Hy3 guide, section 1 and section 8.5 "Gating"; HunyuanImage-3.0
 * article part 3: the gate yields expert_index and topk_weight).
 *   x [T,H] (desc->act_dtype), router_w [E,H] fp32, router_bias [E] or NULL
 *   -> topk_idx [T,k] int32, experts of each token best first,
 *      topk_w   [T,k] fp32, rho * s / sum(selected s) (route_norm = 1).
 * ws: moe_workspace_bytes(desc, T, MOE_WS_ROUTE) bytes (fp32 logits). */
MOE_API moe_status moe_route(moe_ctx *ctx, const moe_desc *desc /* host */, const void *x, int32_t T,
                     const float *router_w, const float *router_bias, int32_t *topk_idx,
                     float *topk_w, void *ws, size_t ws_bytes, void *stream);

/* InitRouting (Hy3 guide, section 8.1 "MoE EP" and section 8.5): group the
 * T*k (token, slot) pairs by expert.  Pair f = t*k + j.
 *   topk_idx [T,k] int32: every entry in [0, E), distinct within a token
 *   -> expert_counts [E], expert_offsets [E+1] (exclusive prefix, last = T*k),
 *      sorted_src [T*k]: row r -> pair f, rows of one expert in ascending f,
 *      dest [T*k]:       pair f -> row r.
 * Entries outside [0, E) or repeated within a token give an unspecified (but
 * in-bounds) permutation.  ws: moe_workspace_bytes(.., MOE_WS_PERMUTE). */
MOE_API moe_status moe_permute(moe_ctx *ctx, const moe_desc *desc /* host */, const int32_t *topk_idx,
                       int32_t T, int32_t *expert_counts, int32_t *expert_offsets,
                       int32_t *sorted_src, int32_t *dest, void *ws, size_t ws_bytes,
                       void *stream);

/* Grouped expert GEMM (Hy3 guide, sections 8.1 and 8.5 "grouped GMM";
 * HunyuanImage-3.0 article part 1, FusedMoEGMM(num_experts, hidden_size,
 * intermediate_size)): for every row r of expert e (rows [offsets[e],
 * offsets[e+1]) ), with token t = sorted_src[r] / k,
 *   y[r] = W_d,e ( silu(W_g,e x[t]) * (W_u,e x[t]) ).
 * shared = 1 runs the shared expert instead: sorted_src and expert_offsets
 * are ignored (may be NULL), rows are the T tokens, y is [T,H].
 *   x [T,H] (act_dtype), y [T*k,H] or [T,H] (out_dtype).
 * ws: moe_workspace_bytes(.., MOE_WS_GROUPED_FFN or MOE_WS_SHARED_FFN). */
MOE_API moe_status moe_grouped_ffn(moe_ctx *ctx, const moe_desc *desc /* host */,
                           const moe_weights *w /* host */, int shared, const void *x, int32_t T,
                           const int32_t *sorted_src, const int32_t *expert_offsets, void *y,
                           void *ws, size_t ws_bytes, void *stream);

/* FinalizeRouting + shared add (Hy3 guide, section 8.5; HunyuanImage-3.0
 * article part 3, output = shared-MLP output + combined output):
 *   out[t] = (sum_{j<k} topk_w[t,j] * y[dest[t*k+j]]) + shared_out[t]
 * summed in fp32 in slot order, shared_out added last (NULL: none).
 *   y [T*k,H], shared_out [T,H], out [T,H], all in out_dtype. */
MOE_API moe_status moe_combine(moe_ctx *ctx, const moe_desc *desc /* host */, const void *y,
                       const int32_t *dest, const float *topk_w, const void *shared_out, int32_t T,
                       void *out, void *stream);

/* The whole layer on `stream` (Hy3 guide, section 8.5 two-stream schedule):
 * (8-bit and MXFP4 experts: quantise x;) gating, permutation and the routed
 * gate/up GEMM on `stream`, then the input-ready event; the side stream
 * waits on it and runs the shared expert beside the routed down GEMM, then
 * records the shared-done event, which `stream` waits on before the
 * combine.  The side stream is used where the overlap was measured to pay:
 * not for a shared expert under 1 MiB of weights (launch-bound layers), and
 * not at 256 or more rows per routed expert (T * k >= 256 * E, where every
 * GEMM is bound by the matrix cores); there the shared expert runs on
 * `stream` in the same place -- for f32 / bf16 experts with I_s equal to I
 * (and fewer than 1024 experts) as one more segment of the routed grouped
 * GEMMs, whose last partial round of tiles it fills; the result is the same
 * bit for bit.  On return `stream` has been made to wait for
 * the side stream, so work queued on `stream` afterwards sees the finished
 * layer.
 *   x [T,H] (act_dtype), out [T,H] (out_dtype).
 * ws: moe_workspace_bytes(desc, T, MOE_WS_LAYER) bytes; its layout is
 * internal, except that moe_layer_ws_topk() locates the routing result. */
MOE_API moe_status moe_layer_forward(moe_ctx *ctx, const moe_desc *desc /* host */,
                             const moe_weights *w /* host */, const void *x, int32_t T, void *out,
                             void *ws, size_t ws_bytes, void *stream);

/* Per-stage timing of moe_layer_forward.  With profiling enabled the call
 * records a pair of timing events around each stage on the stream the stage
 * runs on; moe_ctx_stage_ms then waits for the last call's events and writes
 * each stage's duration in milliseconds (0 for stages that did not run):
 *   MOE_STAGE_ROUTE, MOE_STAGE_MX_QUANT, MOE_STAGE_PERMUTE,
 *   MOE_STAGE_GATE_UP (routed gate/up GEMM + SwiGLU, one kernel),
 *   MOE_STAGE_DOWN (routed down GEMM, one kernel),
 *   MOE_STAGE_SHARED_GATE_UP, MOE_STAGE_SHARED_DOWN, MOE_STAGE_COMBINE.
 * Enabling creates the events (the only allocation after moe_ctx_create);
 * the timing adds an event record between kernels, so leave it off when the
 * layer's own latency is what is measured. */
enum { MOE_STAGE_ROUTE = 0, MOE_STAGE_MX_QUANT = 1, MOE_STAGE_PERMUTE = 2, MOE_STAGE_GATE_UP = 3,
       MOE_STAGE_DOWN = 4, MOE_STAGE_SHARED_GATE_UP = 5, MOE_STAGE_SHARED_DOWN = 6,
       MOE_STAGE_COMBINE = 7, MOE_NUM_STAGES = 8 };
MOE_API moe_status moe_ctx_set_profiling(moe_ctx *ctx, int enable);
MOE_API moe_status moe_ctx_stage_ms(moe_ctx *ctx, float *ms /* host, MOE_NUM_STAGES */);

/* Byte offsets, inside a moe_layer_forward workspace for T tokens, of the
 * topk_idx [T,k] int32 and topk_w [T,k] fp32 arrays the call wrote. */
MOE_API moe_status moe_layer_ws_topk(const moe_desc *desc /* host */, int32_t T,
                             size_t *idx_offset /* host */, size_t *w_offset /* host */);

/* moe_layer_forward with no caller workspace and no allocation, for callers
 * that cannot call hipMalloc: code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation.  The workspace is a static device
 * array of MOE_NOALLOC_SCRATCH_BYTES (64 MiB) inside the library, one copy
 * per GPU, held until the process ends; moe_ctx_create looks up its address
 * on the context's device.  Arguments and results are those of
 * moe_layer_forward.  If moe_workspace_bytes(desc, T, MOE_WS_LAYER) exceeds
 * the array the call returns MOE_ERR_WORKSPACE (text in moe_ctx_last_error)
 * and enqueues nothing; for the Hy3 shape in bf16 (H = 4096, E = 192, k = 8,
 * I = I_s = 1536) that admits up to T = 548 tokens (64 tokens use 11.5 MiB).  Every call on one GPU
 * shares the array and leaves its contents behind: calls that can overlap on
 * one GPU (other streams or contexts without ordering between them) race and
 * give undefined results.  Nothing in the array needs to start at zero. */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
MOE_API moe_status moe_layer_forward_noalloc(moe_ctx *ctx, const moe_desc *desc /* host */,
                                     const moe_weights *w /* host */, const void *x, int32_t T,
                                     void *out, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H_ */
