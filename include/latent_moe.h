/*
 * latent_moe.h -- C ABI of the latent-MoE layer forward for MI355X (gfx950).
 *
 * The layer (web page "SGLang and Miles Add Day-0 Support for Muse Spark
 * Open", section "MoE with Pooler, Unpooler and Per-Expert Normalization";
 * vLLM Day-0 post on Muse Spark Open, section on the latent MoE) maps each
 * token x_t (model width H, already normed) to out_t (width H):
 *
 *   l_t  = Wr x_t + b                          router on the full width, FP32
 *   S_t  = top-k of l_t (ties -> lowest index), slot j = j-th largest
 *   w_tj = softmax over the k selected logits
 *   u_t  = RMSNorm(Wp x_t) * gamma_p           pooler H -> P, pre-expert norm
 *   o_tj = Wd_e (silu(Wg_e u_t) * (Wu_e u_t))   SwiGLU expert e = S_t[j]
 *   y_t  = sum_j w_tj * RMSNorm(o_tj) * gamma_e  per-expert norm, FP32 sum
 *   out_t = Wun y_t                            unpooler P -> H
 *
 * RMSNorm(v) = v / sqrt(mean(v^2) + eps).  The per-expert norm is applied to
 * each selected expert's output before its routing weight (same section;
 * "The Fused Post-per-expert Norm"), and the weighted sum is FP32 (section
 * "Trainable Muse Spark Open Backend").
 *
 * Conventions for every entry point:
 *   - All tensor pointers are DEVICE pointers on the device that was current
 *     when the handle was created; tensors are dense, row-major, in the
 *     [out_features, in_features] convention of the linear maps above.
 *   - Every pointer must be 16-byte aligned; H and P must be multiples of
 *     64, I a multiple of 128, 1 <= E <= 1024 (else INVALID_ARG). Layers with
 *     BF16 activations, whatever the expert format, are built for H, P and I
 *     multiples of 512 (other valid sizes: UNSUPPORTED).
 *   - Calls return 0 (LMOE_OK) or a negative error code; no exception or
 *     abort crosses the ABI. latent_moe_last_error() then holds a message for
 *     the calling thread. All argument checks run on the host before any GPU
 *     work is enqueued, so a failed call has launched nothing.
 */
#ifndef LATENT_MOE_H
#define LATENT_MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LMOE_OK 0
#define LMOE_ERR_INVALID_ARG (-1)     /* null pointer, bad dimension, misalignment */
#define LMOE_ERR_UNSUPPORTED (-2)     /* a dtype combination not implemented */
#define LMOE_ERR_OOM (-3)             /* device allocation failed in create */
#define LMOE_ERR_HIP (-4)             /* any HIP runtime error, including "no device" */
#define LMOE_ERR_TOO_MANY_TOKENS (-5) /* T > max_tokens of the handle */
#define LMOE_ERR_CORRUPT (-6)         /* debug mode only: workspace guard words overwritten */

/* Element formats. */
#define LMOE_F32 0   /* IEEE binary32 */
#define LMOE_BF16 1  /* bfloat16 (upper half of binary32), stored as 16-bit words */
#define LMOE_MXFP4 2 /* OCP MX FP4: E2M1 elements, two per byte (element 2i in the
                        low nibble), plus one E8M0 scale byte per 32 consecutive
                        elements along the input (K) axis */
#define LMOE_MXFP8 3 /* OCP MX FP8: E4M3 elements, one per byte, plus one E8M0
                        scale byte per 32 consecutive elements along K */

typedef struct latent_moe latent_moe_t;

typedef struct {
  int64_t hidden;       /* H: model width (8192 for the published model) */
  int64_t pooled;       /* P: expert width after the pooler (4096) */
  int64_t experts;      /* E: routed experts per layer (256) */
  int64_t intermediate; /* I: SwiGLU intermediate width per expert */
  int32_t top_k;        /* k: experts per token, 1 <= k <= min(E, 32) */
  float eps;            /* RMSNorm epsilon for both norms, finite, >= 0 */
  int32_t act_dtype;    /* x, pooler and unpooler: LMOE_F32 or LMOE_BF16.
                           LMOE_BF16: the pooler multiplies BF16 x by BF16 Wp;
                           the expert and unpooler GEMMs then run on FP16
                           operands: u, the SwiGLU output a and y are rounded
                           to FP16 (nearest even), each stored times a power
                           of two chosen at create that keeps a bound on it
                           within 2^15 (u, y: sqrt(P) max|gamma|; a, per
                           expert and 32 columns: ||Wg_i|| ||Wu_i|| P
                           max|gamma_p|^2), 1 for ordinary weights and gammas,
                           so none of them saturates; the down weights carry
                           a's power of two. The
                           weights are used as FP16 copies made at create,
                           each weight row times a power of two 2^s that puts
                           its largest magnitude in [2^14, 2^15), undone in
                           FP32 after the product. Every BF16 weight within
                           2^31 of its row's largest is exact in that copy.
                           FP16 carries three more significand bits than BF16
                           at the same matrix rate; products accumulate in
                           FP32 */
  int32_t expert_dtype; /* gate/up/down: LMOE_F32, LMOE_BF16 or LMOE_MXFP4.
                           LMOE_F32 requires act_dtype LMOE_F32 and vice versa;
                           LMOE_MXFP4 runs with BF16 activations: each element
                           is decoded in registers to FP16, times its row's
                           2^s (code value x 2^(scale-127+s), exact for every
                           block whose scale is within 2^35 of the row's
                           largest), and the products accumulate in FP32 as
                           for BF16 experts */
  int64_t max_tokens;   /* upper bound on T per forward; sizes the workspace */
  int32_t input_norm;   /* 0: x is the normed token. 1: x is the pre-norm
                           residual r; the layer first forms
                           x = r / sqrt(mean(r^2) + eps) * input_gamma in FP32
                           (sandwich pre-norm: vLLM Day-0 post, sections on the
                           sandwich norm and on the FP32 router input; lmsys
                           post, "Fuse normalization and remove routing
                           conversions"). The router then reads that FP32
                           value and the pooler its act_dtype rounding (BF16
                           nearest-even, or the FP32 value). */
  int32_t expert_act;   /* 0: the expert GEMMs read u and a in FP16 (above).
                           LMOE_MXFP8: they read them as MX FP8 (E4M3, one E8M0
                           scale per 32 along K), quantised with nearest-even
                           rounding and saturation at 448, on the scaled matrix
                           cores against MXFP4 weights ("fp8 x fp4" MMA kind,
                           lmsys post, "NVFP4 as a third MMA kind"; the
                           pre-expert norm is applied by the quantiser, section
                           "Fuse normalization and remove routing conversions").
                           LMOE_MXFP4: MX FP4 (E2M1, two per byte, one E8M0
                           scale per 32 along K), nearest-even rounding,
                           saturation at 6 ("mxfp4 x mxfp4" MMA kind, same
                           section). Both need expert_dtype LMOE_MXFP4 and
                           act_dtype LMOE_BF16 and change the numerics. */
} latent_moe_config;

/* Layer weights (device pointers, on the device current at create). They are
 * BORROWED FOR THE DURATION OF latent_moe_create ONLY: create copies every
 * tensor the forward reads into library-owned device memory and synchronises
 * its stream before returning, so the caller may free or overwrite them as
 * soon as create returns. FP32 layers keep the copies as given; BF16 layers
 * keep the pooler in BF16, the unpooler and the three expert matrices in a
 * matrix-core tiled layout (blocks of 32 rows x 64 columns ordered as the
 * MFMA B fragments; MXFP4 codes and scales likewise, the scale bytes of four
 * k-tiles side by side), and the router as its exact three-piece BF16 split.
 * An MXFP4 scale byte 0xFF (NaN in E8M0) makes its 32 elements NaN.
 *   router       [E, H]   F32
 *   router_bias  [E]      F32, or NULL for no bias (added to the logits)
 *   pooler       [P, H]   act_dtype
 *   pool_gamma   [P]      F32
 *   w_gate, w_up [E, I, P] expert_dtype (MXFP4: [E, I, P/2] bytes)
 *   w_down       [E, P, I] expert_dtype (MXFP4: [E, P, I/2] bytes)
 *   s_gate, s_up [E, I, P/32], s_down [E, P, I/32]  E8M0 bytes (MXFP4 only,
 *                 else ignored)
 *   expert_gamma [E, P]   F32, one gamma row per expert
 *   unpooler     [H, P]   act_dtype
 *   input_gamma  [H]      F32, the boundary norm's gamma (input_norm only)   */
typedef struct {
  const float* router;
  const float* router_bias;
  const void* pooler;
  const float* pool_gamma;
  const void* w_gate;
  const void* w_up;
  const void* w_down;
  const uint8_t* s_gate;
  const uint8_t* s_up;
  const uint8_t* s_down;
  const float* expert_gamma;
  const void* unpooler;
  const float* input_gamma; /* [H] F32 when cfg.input_norm, else ignored */
} latent_moe_weights;

/* Create a handle on the current device. Validates cfg and w on the host,
 * allocates the workspace for cfg->max_tokens tokens (never reallocated
 * later) and one buffer for the weight copies (about the size of the given
 * weights), runs the copy and repack kernels on `stream` (a hipStream_t; NULL
 * = the null stream), creates the handle's routing stream (default priority)
 * and synchronises `stream` (not the device) before returning. Nothing of `w`
 * is referenced after create returns.
 * Errors: INVALID_ARG, UNSUPPORTED, OOM, HIP. On error *out is set to NULL and
 * everything create allocated is released.
 * Test hooks (environment, read at create): LATENT_MOE_FAULT=alloc (or
 * alloc:N) makes the first (N-th) device allocation of create fail with OOM;
 * LATENT_MOE_DEBUG=poison fills the workspace with 0xFF bytes at create and
 * before every forward (a stage that reads a value not written earlier in the
 * same forward then sees NaN) and puts guard words after it, checked by
 * destroy (LMOE_ERR_CORRUPT). */
int latent_moe_create(latent_moe_t** out, const latent_moe_config* cfg, const latent_moe_weights* w,
                      void* stream);

/* Bytes of device workspace a handle with this config allocates (besides its
 * copies of the weights). Errors as for create's validation. */
int latent_moe_workspace_bytes(const latent_moe_config* cfg, size_t* bytes);

/* Run the layer on T tokens, asynchronously on `stream` (a hipStream_t; NULL =
 * the null stream).
 *   x            [T, H] act_dtype, read-only
 *   out          [T, H] F32, written
 *   topk_ids     [T, k] int32 or NULL: selected experts in slot order
 *                (logit descending, index ascending on ties)
 *   topk_weights [T, k] F32 or NULL: routing weights in the same order
 * Caller-owned buffers must stay valid until the stream passes this call.
 * T = 0 succeeds and enqueues nothing. One forward in flight per handle: the
 * workspace is shared, so overlapping forwards of one handle on different
 * streams race. The forward never allocates or synchronises the host.
 * The pooler steps (pooler GEMM and the pre-expert norm) run on a stream the
 * handle owns, forked from `stream` by an event and joined back into it
 * before the expert GEMMs, so they overlap routing (router, top-k, grouping),
 * which runs on `stream`; all work still completes in `stream`'s order
 * (stage profiling, latent_moe_set_profiling, runs everything on `stream`).
 * Errors: INVALID_ARG (null handle/x/out, misaligned pointer, T < 0),
 * TOO_MANY_TOKENS, HIP (launch failure). */
int latent_moe_forward(latent_moe_t* h, const void* x, int64_t T, float* out, int32_t* topk_ids,
                       float* topk_weights, void* stream);

/* For callers that cannot allocate device memory (code under stream capture,
 * tight serving loops, harnesses that forbid hipMalloc): the FP32 layer's
 * forward without a handle. It takes the config and the weights as create
 * does and x, out, topk_ids, topk_weights and stream as forward does, reads
 * the weights in place (they must stay valid and unchanged until the stream
 * passes this call), and keeps its whole workspace in a static device array
 * of LMOE_STATIC_SCRATCH_BYTES (16 MiB) that the library holds on each device
 * it runs on until the process ends; it calls no allocating routine. Every
 * call on one device shares that device's array, which keeps the last call's
 * contents: calls that overlap on one device (different streams or threads)
 * race. cfg->max_tokens is ignored; T is limited by the array (the tiny
 * layer, H 256, P 128, I 128, E 8, k 2, fits about 4900 tokens).
 * Errors: INVALID_ARG and UNSUPPORTED as for create's validation (BF16
 * layers are UNSUPPORTED: they run on weight copies made by create);
 * TOO_MANY_TOKENS when the workspace for T tokens exceeds the array; HIP. */
#define LMOE_STATIC_SCRATCH_BYTES (16u << 20)
int latent_moe_forward_static(const latent_moe_config* cfg, const latent_moe_weights* w, const void* x,
                              int64_t T, float* out, int32_t* topk_ids, float* topk_weights, void* stream);

/* Views of the last forward's intermediates, for inspection and per-stage
 * tests. Pointers are into the handle's workspace (device memory), valid
 * until the next forward or destroy; rows beyond the last forward's T (or
 * its T*k routed pairs) hold stale data. Layouts:
 *   logits   [T, E] F32 router logits (bias included)
 *   ids      [T, k] int32, weights [T, k] F32 (as exported by forward)
 *   counts   [E] int32 routed pairs per expert; offsets [E+1] int32 exclusive
 *            prefix of counts
 *   perm_token [T*k] int32: token of each routed pair, grouped by expert
 *            (stable in (t, j) order within an expert)
 *   pair_row [T*k] int32: for pair (t, j) at index t*k+j, its row in the
 *            grouped order
 *   pooled   [T, P] F32: gamma_p * (Wp x_t), before the row scale
 *   row_scale [T] F32: 1/sqrt(mean((Wp x_t)^2) + eps)
 *   act      [T*k, I] (F32 if expert_dtype is F32, else FP16): SwiGLU
 *            output, grouped order
 *   expert_out [T*k, P]: grouped order; FP32 layers: o (before the
 *            per-expert norm) in F32; BF16 layers: gamma_e * o (the expert's
 *            norm gamma applied, the norm's 1/rms not) in FP16 times
 *            expert_out_down[e]
 *   combined y [T, P]: F32 in FP32 layers, FP16 in BF16 layers          */
typedef struct {
  const float* logits;
  const int32_t* ids;
  const float* weights;
  const int32_t* counts;
  const int32_t* offsets;
  const int32_t* perm_token;
  const int32_t* pair_row;
  const void* pooled;
  const float* row_scale;
  const void* act;
  const void* expert_out;
  const void* combined;
  const uint8_t* expert_in;        /* the expert GEMMs' input u as they read it:
                                      MX expert inputs: codes, [T, P] E4M3 bytes
                                      (MXFP8) or [T, P/2] packed E2M1 (MXFP4);
                                      other BF16 layers: [T, P] FP16 (row_scale
                                      times pooled, rounded); FP32 layers: NULL */
  const uint8_t* expert_in_scales; /* MX expert inputs: u scales [T, P/32] E8M0,
                                      else NULL */
  const uint8_t* act_scales;       /* MX expert inputs: act scales [T*k, I/32] E8M0
                                      (act then holds the codes, [T*k, I] E4M3 or
                                      [T*k, I/2] packed E2M1), else NULL */
  const void* x_norm;   /* boundary norm output (input_norm only, else NULL): FP32 layers
                           [T, H] F32; BF16 layers its exact three-piece BF16 split
                           [T, 3H] (pieces p1 | p2 | p3 side by side, p1 + p2 + p3 =
                           the FP32 value, p1 = its BF16 rounding, the pooler's input) */
  float expert_in_scale; /* the FP16 expert_in holds u times this power of two, and */
  float combined_scale;  /* the FP16 combined holds y times this one: 1 unless
                            sqrt(P) max|gamma| exceeds 2^15 (then the largest power of
                            two that keeps u, y below 2^15 in magnitude); 1 for F32 */
  const float* act_down; /* BF16 layers without MX expert inputs: [E, I/32] F32, the
                            FP16 act of a pair routed to expert e holds a times
                            act_down[e][i/32], a power of two (1 unless the
                            Cauchy-Schwarz bound |a_i| <= ||Wg_i|| ||Wu_i|| P
                            max|gamma_p|^2 exceeds 2^15); else NULL */
  const float* expert_out_down; /* BF16 layers: [E] F32, expert_out holds FP16 gamma_e * o
                            times expert_out_down[e] for a pair routed to expert e, a
                            power of two keeping ||Wd_p|| ||u||^2 sqrt(sum_i (||Wg_i||
                            ||Wu_i||)^2) max|gamma_e| within 2^15; FP32 layers: NULL
                            (expert_out is F32 o) */
} latent_moe_views;

int latent_moe_debug_views(const latent_moe_t* h, latent_moe_views* v);

/* Stage timing, for measurement. With profiling enabled, each forward records
 * one HIP event on its stream before the first stage and after each of the
 * LMOE_NUM_STAGES stages (events are created here, never in forward):
 *   0 boundary norm        1 router GEMM        2 top-k/softmax
 *   3 grouping by expert   4 pooler GEMM        5 pooled row scale
 *   6 gate/up GEMM+SwiGLU  7 down GEMM          8 combine
 *   9 unpooler GEMM
 * (stage 0 is empty unless cfg.input_norm). latent_moe_stage_times waits for
 * the last recorded event and writes the elapsed milliseconds of each stage
 * of the last forward into ms[0..9].
 * Errors: INVALID_ARG (NULL handle/ms, n < LMOE_NUM_STAGES, no profiled
 * forward yet), HIP. */
#define LMOE_NUM_STAGES 10
int latent_moe_set_profiling(latent_moe_t* h, int enable);
int latent_moe_stage_times(latent_moe_t* h, float* ms, int n);

/* Wait for the handle's work (device synchronisation), free its workspace,
 * weight copies, routing stream and the handle. NULL returns INVALID_ARG.
 * CORRUPT (debug mode only): guard words after the workspace were overwritten
 * (the handle is freed all the same). Using a handle after destroy is
 * undefined. */
int latent_moe_destroy(latent_moe_t* h);

/* Message for the last failed call on this thread ("" if none). The string is
 * owned by the library and valid until the thread's next call. */
const char* latent_moe_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* LATENT_MOE_H */
