/*
 * moe.h -- C ABI of the routed mixture-of-experts MLP forward for MI355X
 * (gfx950, CDNA4).  Plain pointers and sizes only; every buffer is device
 * memory unless a comment says "host".
 *
 * The layer (one token t of T, hidden size H, E routed experts, top-k):
 *   [ScMoE] xr = bf16(RMSNorm_pre(x_prev))            else xr = x
 *   l  = fp32(xr @ W_r^T)                             router GEMM, fp32
 *   s  = sigmoid(l);  s' = s + b                      b steers selection only
 *   ids = the k largest s' over all E (ties -> lower id), ascending
 *   w  = rsf * s[ids]                                 unbiased, scaled
 *   permute the T*k (token, slot) pairs by expert id (stable)
 *   per expert e: h = bf16(silu(min(g, L)) * clamp(u, -L, L)),
 *                 [g, u] = x_row @ W_gu[e]^T,  y = h @ W_d[e]^T (fp32)
 *   shared:       the same FFN on x (ScMoE: x_cur), width I_s, unscaled
 *   z  = sum_j w[t,j] * y[t,j] + ys[t]                one combine, fp32
 *   out = bf16(z)           [ScMoE] out = bf16(RMSNorm_post(z))
 *   [finish] out = bf16(bf16(out * c0) + bf16(residual * c1))   (optional)
 *
 * Sources (web pages; cited by title and section):
 *   "Module glm5next_mlp" (metrale_model_arch docs): section "Numerics the
 *     kernels rely on" (asymmetric SwiGLU clamp with a required limit;
 *     selection-only correction bias; routed_scaling_factor on routed
 *     weights only; top-k over the full expert count), section "One
 *     all-reduce for both EP and TP" (shared output and routed slots summed
 *     in one combine), Modules forward / forward_prefill_gemm (dense SwiGLU
 *     FFN reused as the shared expert; one grouped launch per projection),
 *     Constants KERNEL_MAX_TOP_K (k <= 16) and MOE_MODULE (token sort /
 *     permute / unpermute).
 *   "bridge.models.beam.modeling_beam" (NeMo Megatron-Bridge API docs):
 *     beam_router_gating_linear, _BeamRouterGatingLinear, BeamTopKRouter
 *     (router logits inp @ weight^T in fp32 with fp32 router weights).
 *   "mstar.model.components.distributed.mlp": ParallelGatedMLP (gate and up
 *     fused in one weight, gate first).
 *   "core.models.hybrid.shortcut_block" (Megatron-Core API docs): module
 *     doc and ShortcutMoEBlock (ScMoE: the preceding layer's normalised
 *     representation is routed, the shared expert runs on the current one,
 *     the merged sum is normalised again, _postprocess finishes the
 *     residual/BDA).
 *   "bridge.models.beam.modeling_beam": _beam_bda, scaled_residual_add and
 *     depth_scaled_residual_coefs (post-sublayer norm, then a residual add
 *     with two scalar coefficients in the residual's dtype).
 *
 * Conventions shared by every entry point:
 *   - bf16 values are passed as uint16_t bit patterns (moe_bf16).
 *   - Weights are [out, in] with the input dimension contiguous (the layout
 *     of x @ W^T).  w_gate_up[e] holds the I gate rows, then the I up rows.
 *   - Every call only enqueues work on `stream` and returns; it never
 *     synchronises, allocates or frees device memory, and keeps no pointer
 *     after it returns.  The caller owns all buffers and keeps them alive
 *     until the stream has run the work.
 *   - Arguments are validated on the host before anything is enqueued; on
 *     any error nothing is enqueued and no output is touched.  The detail of
 *     the last error of the calling thread is in moe_last_error().
 *   - Results are deterministic: identical inputs give identical bits (no
 *     floating-point atomics anywhere).
 *   - Device pointers must be 16-byte aligned; H, I and I_shared must be
 *     multiples of 8.  T == 0 is a successful no-op.
 *   - Functions are reentrant.  Library state: the per-thread error text,
 *     and, per thread and device, one extra stream with two events that
 *     moe_forward creates on its first call that needs them (see there) and
 *     keeps until the process ends.
 */
#ifndef MOE_H_
#define MOE_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef uint16_t moe_bf16;

#define MOE_MAX_TOP_K 16      /* "Module glm5next_mlp", Constants, KERNEL_MAX_TOP_K */
#define MOE_MAX_EXPERTS 1024  /* implementation bound of the top-k and permute kernels */

typedef enum moe_status {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1, /* violates the layer's definition (k < 1, k > 16,
                              k > E, E < 1, H or I < 1, I_shared < 0, T < 0,
                              limit not finite or <= 0, rsf not finite,
                              ScMoE with eps <= 0 or no x_shared, a NULL
                              required pointer) */
  MOE_ERR_UNSUPPORTED = 2, /* valid but outside the kernels: H, I or I_shared
                              not a multiple of 8, a pointer not 16-byte
                              aligned, E > 1024, T*k >= 2^31, ScMoE with
                              H > 8192 */
  MOE_ERR_WORKSPACE = 3,   /* ws_bytes smaller than the size asked for */
  MOE_ERR_DEVICE = 4       /* a launch failed (hipGetLastError); faults inside
                              kernels surface at the caller's synchronisation */
} moe_status;

/* Shape and constants of one layer call. */
typedef struct moe_params {
  int64_t T;                   /* tokens (rows of x)                              */
  int32_t H;                   /* hidden size                                     */
  int32_t E;                   /* routed experts (the full count, never a share)  */
  int32_t k;                   /* experts per token, 1 <= k <= min(E, 16)         */
  int32_t I;                   /* routed expert intermediate width                */
  int32_t I_shared;            /* shared expert width; 0 = no shared expert       */
  float routed_scaling_factor; /* multiplies the routed weights only; finite      */
  float swiglu_limit;          /* L: required, finite, > 0 (no default exists)    */
  int32_t scmoe;               /* 1 = ScMoE pairing: RMSNorm before routing and   */
                               /*     on the merged output; 0 = plain layer       */
  float norm_eps;              /* RMSNorm epsilon (ScMoE), > 0                    */
  int32_t w4;                  /* 1 = W4A16 routed experts (moe_weights' *_q and  */
                               /*     *_scale arrays); 0 = bf16                   */
} moe_params;

/* Device weights of one layer (all caller-owned, read-only). */
typedef struct moe_weights {
  const float* w_router;       /* [E, H] fp32                                     */
  const float* corr_bias;      /* [E] fp32 selection-only bias; NULL = zeros      */
  const moe_bf16* w_gate_up;   /* [E, 2I, H] bf16: gate rows [0,I), up [I,2I)     */
  const moe_bf16* w_down;      /* [E, H, I] bf16                                  */
  const moe_bf16* ws_gate_up;  /* [2I_s, H] bf16; unused when I_shared == 0       */
  const moe_bf16* ws_down;     /* [H, I_s] bf16; unused when I_shared == 0        */
  const float* gamma_pre;      /* [H] fp32 ScMoE pre-norm gain; NULL = ones       */
  const float* gamma_post;     /* [H] fp32 ScMoE post-norm gain; NULL = ones      */
  /* W4A16 routed experts (the W4A16 expert GEMM named by "Module
   * glm5next_mlp", Modules forward_prefill_gemm and Constants
   * MOE_GROUPED_MODULE / W4A16_GEMV_MODULE, with the two scale levels of the
   * NVFP4 routed experts its module doc names; the layout is this
   * library's): with moe_params.w4 = 1, the routed experts use these arrays
   * and w_gate_up / w_down are ignored.  A weight is
   *   (u - 8) * e4m3(scale) * tensor_scale,
   * u a 4-bit code, packed along K in 4-byte words of 8 columns (byte j of
   * a word: column j in the low nibble, column j + 4 in the high nibble);
   * scale one OCP FP8 E4M3 byte per row and group of 128 columns, stored
   * group-major; tensor_scale one fp32 value per expert and projection.
   * H and I must be multiples of 128; the shared expert stays bf16.  Every
   * code and scale byte is accepted (an E4M3 NaN scale, 0x7F or 0xFF, makes
   * its weights NaN).  (u - 8) * e4m3(scale) is exact in bf16, and the
   * tensor scale multiplies the fp32 GEMM sums, so on every path the
   * results equal the exactly dequantised layer up to fp32 summation order.
   * Decode-sized batches (T*k <= 64*E) stream the codes and unpack them in
   * registers; prefill-sized ones (T*k >= 512*E) stage the codes and scales
   * in LDS and unpack them there, a stage ahead of the MFMAs, inside the
   * grouped GEMM; batches in between (or a tile variant forced through
   * MOE_GEMM_VARIANT) first expand the layer's experts into the workspace
   * as bf16 (exactly; the workspace then holds E * 3 * I * H bf16 more) and
   * run the bf16 grouped GEMMs. */
  const uint8_t* w_gate_up_q;       /* [E, 2I, H/2] codes; NULL = bf16 experts    */
  const uint8_t* w_gate_up_scale;   /* [E, H/128, 2I] E4M3                        */
  const uint8_t* w_down_q;          /* [E, H, I/2] codes                          */
  const uint8_t* w_down_scale;      /* [E, I/128, H] E4M3                         */
  const float* w_gate_up_tscale;    /* [E] fp32 tensor scales; NULL = ones        */
  const float* w_down_tscale;       /* [E] fp32 tensor scales; NULL = ones        */
  /* Optional tile-blocked copies of the bf16 experts, written once by
   * moe_pack_experts (NULL = not given), each pair both or neither: the
   * routed pair (bf16 routed experts only, not with W4A16) and the shared
   * expert's (moe_pack_experts with E = 1 and I = I_shared).  With bf16
   * routed experts and I_shared > 0 the two pairs come together (the tiles
   * run both in one launch); with W4A16 routed experts the shared pair
   * alone may be given.
   * Prefill-sized batches (the 256-row tiles) then read each 32-column K
   * stage of a 256-row weight tile as one contiguous 16 KB block instead of
   * 256 pieces of 64 bytes, in fewer and larger requests to the caches; the
   * results are the same bits.  The row-major weights stay required (the
   * other batch sizes read them). */
  const moe_bf16* w_gate_up_packed;
  const moe_bf16* w_down_packed;
  const moe_bf16* ws_gate_up_packed;
  const moe_bf16* ws_down_packed;
} moe_weights;

/* Finish of the layer, fused into its combine (moe_forward_finish,
 * moe_combine_finish): the residual add after the layer output,
 *   out = bf16(bf16(o * out_scale) + bf16(residual * residual_scale)),
 * each product and the sum computed in fp32 and rounded to bf16 (the add in
 * the residual's dtype), o the layer output as moe_forward writes it: after
 * the post-norm, which post_norm = 1 also applies to a plain layer (a
 * sandwich norm on the MLP output: RMSNorm(z) * gamma_post, eps =
 * norm_eps).  out_scale = residual_scale = 1 is the ScMoE block's
 * residual/bias-dropout-add at inference (the layer has no output bias and
 * dropout is the identity); other values are Beam's depth-scaled residual
 * add, whose two coefficients the caller computes (their squares sum to one
 * there; the library does not require it).
 * Sources: "bridge.models.beam.modeling_beam", _beam_bda,
 * scaled_residual_add, depth_scaled_residual_coefs,
 * BeamTransformerLayerSubmodules.post_mlp_layernorm;
 * "core.models.hybrid.shortcut_block", ShortcutMoEBlock._postprocess. */
typedef struct moe_finish {
  const moe_bf16* residual;  /* [T, H] bf16, required; may be the out buffer   */
                             /* itself (the add is then in place)             */
  float out_scale;           /* c0, finite                                    */
  float residual_scale;      /* c1, finite                                    */
  int32_t post_norm;         /* 1 = RMSNorm_post also without ScMoE (needs     */
                             /* norm_eps > 0, H <= 8192); 0 = ScMoE's only    */
} moe_finish;

/* Step boundaries of moe_forward at which caller-created HIP events can be
 * recorded on `stream` (for timing a step on the stream it runs on).
 * events[MOE_EV_BEGIN] is recorded before the first kernel, events[s] right
 * after step s; a step the layer does not run records at the same point as
 * the one before it.  For batches of at most 4096 (token, slot) pairs and
 * T*E <= 16384 the top-k and the permutation are one launch: MOE_EV_ROUTER
 * then follows both and MOE_EV_PERMUTE is recorded at the same point. */
enum {
  MOE_EV_BEGIN = 0,
  MOE_EV_PRENORM = 1,  /* ScMoE pre-norm                                    */
  MOE_EV_ROUTER = 2,   /* router logits + top-k                             */
  MOE_EV_PERMUTE = 3,  /* permutation + grouped-GEMM tile schedule (and, for */
                       /* W4A16 experts expanded in the workspace, the wait */
                       /* for the gate_up weights' dequantisation)          */
  MOE_EV_GATE_UP = 4,  /* grouped gate_up + SwiGLU (routed and shared)      */
  MOE_EV_DOWN = 5,     /* grouped down projection (routed and shared)       */
  MOE_EV_COMBINE = 6,  /* weighted combine (+ ScMoE post-norm)              */
  MOE_EV_COUNT = 7
};

/* Optional observation points of moe_forward.  A non-NULL output pointer
 * receives that step's result (and is used in place of the workspace
 * slot); a non-NULL event is recorded at its step boundary; NULL members
 * are skipped. */
typedef struct moe_probes {
  int32_t* topk_ids;           /* [T, k]                                          */
  float* topk_w;               /* [T, k]                                          */
  int32_t* expert_offsets;     /* [E + 1]                                         */
  int32_t* sorted_token;       /* [T * k]                                         */
  int32_t* inv_pos;            /* [T * k]                                         */
  moe_bf16* xr;                /* [T, H] ScMoE routed input after the pre-norm    */
  float* logits;               /* [T, E] fp32 router logits                       */
  moe_bf16* h;                 /* [T * k, I] routed SwiGLU outputs (permuted rows) */
  float* y;                    /* [T * k, H] routed down outputs (permuted rows)  */
  moe_bf16* h_shared;          /* [T, I_shared] shared expert's SwiGLU outputs    */
  float* y_shared;             /* [T, H] shared expert's output                   */
  hipEvent_t events[MOE_EV_COUNT];
} moe_probes;

/* Bytes of workspace that moe_forward (and, for the same params, each of
 * moe_router_topk and moe_permute) needs.  Host-only, pure function of
 * *p; validates *p like moe_forward. */
moe_status moe_workspace_size(const moe_params* p, size_t* bytes);

/* Router: l = fp32(x @ W_r^T), s = sigmoid(l), s' = s + corr_bias, the k
 * largest s' over all E experts (equal s' -> lower id first, NaN below every
 * number), emitted in ascending id order with weight rsf * s (the bias never
 * enters a weight).
 *   x         [T, H] bf16 (for ScMoE: the already normalised routed input)
 *   w_router  [E, H] fp32;  corr_bias [E] fp32 or NULL
 *   topk_ids  [T, k] int32 out;  topk_w [T, k] fp32 out
 *   ws        >= moe_workspace_size(p) bytes of scratch; on return its first
 *             T*E floats hold the fp32 logits [T, E] (once the stream has
 *             run the work)
 * Uses p->T, H, E, k, routed_scaling_factor.
 * Sources: "Module glm5next_mlp", "Numerics the kernels rely on" and
 * KERNEL_MAX_TOP_K; "bridge.models.beam.modeling_beam",
 * beam_router_gating_linear. */
moe_status moe_router_topk(const moe_params* p, const moe_bf16* x, const float* w_router,
                           const float* corr_bias, int32_t* topk_ids, float* topk_w,
                           void* ws, size_t ws_bytes, hipStream_t stream);

/* Permute: stable counting sort of the T*k pairs (t, j), keyed by
 * topk_ids[t, j] (each in [0, E)).
 *   expert_offsets [E+1] out: offsets[0] = 0, offsets[E] = T*k, segment e is
 *                  rows [offsets[e], offsets[e+1])
 *   sorted_token   [T*k] out: token of each permuted row (ascending inside a
 *                  segment)
 *   inv_pos        [T*k] out: permuted row of pair t*k + j
 *   x, x_perm      optional gather: with both non-NULL, x_perm[r] =
 *                  x[sorted_token[r]] ([T, H] bf16 in, [T*k, H] bf16 out);
 *                  with both NULL nothing is gathered (moe_forward never
 *                  gathers: its gate_up GEMM reads x through sorted_token);
 *                  x_perm without x is MOE_ERR_INVALID_ARG
 * Bit-exact and deterministic.  Ids outside [0, E) are undefined behaviour
 * (they are not checked on the device).
 * Source: "Module glm5next_mlp", Constants, MOE_MODULE (token sort / permute
 * / unpermute). */
moe_status moe_permute(const moe_params* p, const int32_t* topk_ids, const moe_bf16* x,
                       int32_t* expert_offsets, int32_t* sorted_token, int32_t* inv_pos,
                       moe_bf16* x_perm, void* ws, size_t ws_bytes, hipStream_t stream);

/* Bytes of workspace moe_grouped_swiglu_gemm needs (host-only, pure). */
moe_status moe_grouped_gemm_workspace_size(int32_t n_groups, int64_t M_total, int32_t H,
                                           int32_t I, size_t* bytes);

/* Grouped SwiGLU FFN, one launch per projection for all groups.  For each
 * group g and each row r in [group_offsets[g], group_offsets[g+1]):
 *   a_r = a[row_index ? row_index[r] : r]                     (bf16, length H)
 *   g_r = a_r @ W_gu[g][0:I]^T,  u_r = a_r @ W_gu[g][I:2I]^T   (fp32 accumulate)
 *   h[r] = bf16(silu(min(g_r, L)) * clamp(u_r, -L, L))       [M_total, I] bf16
 *   y[r] = h[r] @ W_d[g]^T                                    [M_total, H] fp32
 *   n_groups       >= 1
 *   M_total        rows; group_offsets[n_groups] must equal it (device data:
 *                  group_offsets[0] = 0, non-decreasing)
 *   a              [rows_a, H] bf16; row_index [M_total] int32 or NULL
 *   group_offsets  [n_groups + 1] int32 (device)
 *   w_gate_up      [n_groups, 2I, H] bf16;  w_down [n_groups, H, I] bf16
 *   h, y           outputs as above
 * Source: "Module glm5next_mlp", Modules forward_prefill_gemm (one grouped
 * launch per projection) and "Numerics the kernels rely on" (the clamp);
 * "mstar.model.components.distributed.mlp", ParallelGatedMLP (fused
 * gate/up weight). */
moe_status moe_grouped_swiglu_gemm(int32_t n_groups, int64_t M_total, int32_t H, int32_t I,
                                   float swiglu_limit, const moe_bf16* a,
                                   const int32_t* row_index, const int32_t* group_offsets,
                                   const moe_bf16* w_gate_up, const moe_bf16* w_down,
                                   moe_bf16* h, float* y, void* ws, size_t ws_bytes,
                                   hipStream_t stream);

/* Combine: z[t] = sum_{j<k} topk_w[t,j] * y_perm[inv_pos[t*k+j]] + y_shared[t]
 * (fp32, j ascending), then out = bf16(z), or with p->scmoe
 * out = bf16(z * gamma_post / sqrt(mean(z^2) + eps)).
 *   y_perm [T*k, H] fp32; topk_w [T, k] fp32; inv_pos [T*k] int32
 *   y_shared [T, H] fp32 or NULL (no shared term);  gamma_post [H] or NULL
 *   out [T, H] bf16
 * Sources: "Module glm5next_mlp", "One all-reduce for both EP and TP";
 * "core.models.hybrid.shortcut_block", ShortcutMoEBlock._postprocess. */
moe_status moe_combine(const moe_params* p, const float* y_perm, const float* topk_w,
                       const int32_t* inv_pos, const float* y_shared, const float* gamma_post,
                       moe_bf16* out, hipStream_t stream);

/* moe_combine followed by the finish *fin (required), in the same kernel:
 * the post-norm when p->scmoe or fin->post_norm, then the residual add
 * (moe_finish).  out may be fin->residual (in place). */
moe_status moe_combine_finish(const moe_params* p, const float* y_perm, const float* topk_w,
                              const int32_t* inv_pos, const float* y_shared,
                              const float* gamma_post, const moe_finish* fin, moe_bf16* out,
                              hipStream_t stream);

/* The whole layer.
 *   x_routed  [T, H] bf16: the layer input (ScMoE: the preceding layer's
 *             hidden, normalised here before routing and the experts)
 *   x_shared  [T, H] bf16: the shared expert's input; NULL = x_routed in the
 *             plain layer; required with ScMoE (the current layer's hidden)
 *   w         weights;  out [T, H] bf16;  probes NULL or optional outputs
 *   ws        >= moe_workspace_size(p) bytes
 * With a few rows per expert (T*k <= 64*E: the expert GEMMs stream weights)
 * and a shared expert, the shared expert's two GEMMs run on the calling
 * thread's second stream for the current device: forked from `stream` at
 * the start (event record + wait), on 3/4 of the CUs beside the routing
 * kernels, and joined back into `stream` before the combine.  Work is still
 * ordered after everything enqueued on `stream` before the call and before
 * everything enqueued after it, and graph capture on `stream` captures both
 * branches; make the first such call outside a capture (it creates the
 * stream and events).
 * Sources: all of the above; "Module glm5next_mlp", Modules forward. */
moe_status moe_forward(const moe_params* p, const moe_bf16* x_routed, const moe_bf16* x_shared,
                       const moe_weights* w, moe_bf16* out, const moe_probes* probes, void* ws,
                       size_t ws_bytes, hipStream_t stream);

/* moe_forward with the finish *fin (required) fused into its combine (see
 * moe_finish); out may be fin->residual (in place).  Everything else as in
 * moe_forward. */
moe_status moe_forward_finish(const moe_params* p, const moe_bf16* x_routed,
                              const moe_bf16* x_shared, const moe_weights* w,
                              const moe_finish* fin, moe_bf16* out, const moe_probes* probes,
                              void* ws, size_t ws_bytes, hipStream_t stream);

/* Bytes of the fixed device scratch of moe_forward_noalloc (64 MiB). */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/* moe_forward without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc).  The layer's intermediates live
 * in a fixed scratch array of MOE_NOALLOC_SCRATCH_BYTES inside the library,
 * one copy per device, held from the library's first use on that device
 * until the process ends; its device address is looked up once per device
 * (the first call on it).  The call allocates and frees nothing and creates
 * no stream: every kernel runs on `stream` (the shared expert shares the
 * routed experts' grouped launches instead of running beside the routing
 * kernels).  Results equal moe_forward's for the same inputs.
 *   Returns MOE_ERR_WORKSPACE, enqueuing nothing, when
 *   moe_workspace_size(p) > MOE_NOALLOC_SCRATCH_BYTES (decode-sized
 *   batches fit: T = 32, H = 4096, E = 64, k = 8, I = 1408, I_shared =
 *   2816 needs 5.5 MiB, T = 256 of the same layer 44 MiB).
 *   Every call on one device uses that device's one scratch array, which
 *   keeps the previous call's contents (nothing in it needs to start at
 *   zero): calls whose work can overlap on one device -- on different
 *   streams, or from several threads -- race and corrupt each other's
 *   results.  Order them on one stream.
 * Other arguments, validation and errors as in moe_forward. */
moe_status moe_forward_noalloc(const moe_params* p, const moe_bf16* x_routed,
                               const moe_bf16* x_shared, const moe_weights* w, moe_bf16* out,
                               const moe_probes* probes, hipStream_t stream);

/* Bytes of workspace moe_router_backward needs for p->T, H, E (host-only,
 * pure; 0 is possible). */
moe_status moe_router_backward_workspace_size(const moe_params* p, size_t* bytes);

/* Backward of the router GEMM l = x @ W_r^T (+ b), fp32 (training path):
 * for the upstream gradient dL [T, E] (fp32),
 *   grad_x = bf16(fp32(dL @ W_r))    [T, H] bf16 out, or NULL to skip
 *   grad_w = fp32(dL^T @ x)          [E, H] fp32 out, or NULL to skip
 *   grad_b = fp32(sum_t dL[t, :])    [E] fp32 out, or NULL to skip
 * both GEMMs in fp32 with every product exact (results equal fp32 GEMMs up
 * to summation order, deterministic); grad_x comes back in the saved
 * input's dtype.  dL element (t, e) is read at grad_logits[t * g_row_stride
 * + e * g_col_stride] (strides in elements, >= 0): an expanded gradient
 * such as that of logits.sum() (both strides 0) is used as it is, without
 * a contiguous copy.  x [T, H] bf16 (the saved router input), w_router
 * [E, H] fp32; ws >= moe_router_backward_workspace_size(p) bytes.  With
 * T == 0, grad_w and grad_b are zero-filled.  Uses p->T, H, E.
 * Source: "bridge.models.beam.modeling_beam", _BeamRouterGatingLinear
 * (forward/backward of the fp32 gating GEMM with fp32 weights, bf16 saved
 * activations, stride-0 gradients). */
moe_status moe_router_backward(const moe_params* p, const float* grad_logits,
                               int64_t g_row_stride, int64_t g_col_stride, const moe_bf16* x,
                               const float* w_router, moe_bf16* grad_x, float* grad_w,
                               float* grad_b, void* ws, size_t ws_bytes, hipStream_t stream);

/* W4A16 weights -> bf16, for callers whose weights stay fixed across calls:
 * expand them once, then run the bf16 forward (moe_forward with w4 = 0)
 * instead of expanding on every prefill-sized call.  q: [n_groups, rows,
 * K/2] codes, scale: [n_groups, K/128, rows] E4M3 bytes, both in the W4A16
 * layout of moe_weights; tscale: [n_groups] fp32 tensor scales or NULL
 * (= 1); out: [n_groups, rows, K] bf16,
 *   out[g][r][c] = bf16((u - 8) * e4m3(scale) * tscale[g]),
 * rounded to nearest, ties to even -- exact when tscale is NULL or a power
 * of two ((u - 8) * e4m3(scale) is always a bf16 value); a zero weight is
 * +0.  K must be a multiple of 128 and n_groups * rows < 2^31; q, scale and
 * out 16-byte aligned, tscale 4-byte aligned (the caller owns all of them;
 * out must not overlap the inputs).  n_groups, rows or K == 0 is a
 * successful no-op.  Source: the grouped W4A16 expert GEMM of "Module
 * glm5next_mlp" (its weights are dequantised to the 16-bit MMA operand
 * type; the layout is this library's). */
moe_status moe_w4_dequantize(const uint8_t* q, const uint8_t* scale, const float* tscale,
                             int32_t n_groups, int64_t rows, int32_t K, moe_bf16* out,
                             hipStream_t stream);

/* Tile-blocked copies of bf16 experts for moe_weights' *_packed fields: a
 * one-time preparation of the weights, like loading them, not a step of the
 * layer (the layout is this library's: the loads of its 256-row tiles, not
 * a format of the pages).  p is checked as in every call; only its E, H
 * and I shape the copies.
 * gate_up_packed: for expert e, column tile b (output columns [128 b,
 *   128 b + 128), b < ceil(I/128)) and K stage s (columns [32 s, 32 s + 32)
 *   of H, s < H/32), one block of 256 rows x 32 values, each row's 32
 *   values contiguous: rows 0..127 the gate rows 128 b + r of w_gate_up[e],
 *   rows 128..255 the up rows I + 128 b + r; rows past I are zeros.  Blocks
 *   in the order (e, b, s).
 * down_packed: for expert e, row tile b (rows [256 b, 256 b + 256) of
 *   w_down[e], b < ceil(H/256)) and K stage s (s < I/32), the 256 x 32
 *   block of those rows; rows past H are zeros.  Blocks in the order
 *   (e, b, s).
 * moe_packed_experts_size gives the element counts (E * ceil(I/128) * 256
 * * H and E * ceil(H/256) * 256 * I bf16).  The shared expert's copies are
 * the same with E = 1 and I = I_shared (ws_gate_up, ws_down as w_gate_up,
 * w_down).  H and I must be multiples of 32 (else MOE_ERR_UNSUPPORTED);
 * pointers device and 16-byte aligned (NULL: MOE_ERR_INVALID_ARG,
 * misaligned: MOE_ERR_UNSUPPORTED); the outputs must not overlap the
 * inputs.  Asynchronous on stream. */
moe_status moe_packed_experts_size(const moe_params* p, int64_t* gate_up_elems,
                                   int64_t* down_elems);
moe_status moe_pack_experts(const moe_params* p, const moe_bf16* w_gate_up, const moe_bf16* w_down,
                            moe_bf16* gate_up_packed, moe_bf16* down_packed, hipStream_t stream);

/* Diagnostics, not on the layer's path: what the current device delivers,
 * for reporting the layer's rates against measured peaks beside the
 * published ones.
 * moe_probe_mfma_bf16: `workgroups` workgroups of four wavefronts, each
 *   running `iters` rounds of four independent 32x32x16 bf16 MFMAs on
 *   varied non-zero operands (workgroups, iters >= 1); sink [workgroups *
 *   256] fp32 device scratch the kernel writes (16-byte aligned);
 *   *flops (host) receives the floating-point operations enqueued.
 * moe_probe_hbm_read: reads `bytes` of src once (each of `workgroups`
 *   workgroups of 256 threads streams one contiguous block, 16 KB per step
 *   in non-temporal 16-byte loads; bytes a positive multiple of 16, src
 *   16-byte aligned); sink [workgroups * 256] uint32 device scratch the
 *   kernel writes.
 * Time them with events on `stream`. */
moe_status moe_probe_mfma_bf16(int32_t workgroups, int32_t iters, float* sink, double* flops,
                               hipStream_t stream);
moe_status moe_probe_hbm_read(const void* src, int64_t bytes, int32_t workgroups,
                              uint32_t* sink, hipStream_t stream);

/* Static text naming a status code. */
const char* moe_status_string(moe_status s);

/* Detail of the last error returned to the calling thread ("" if none).
 * The pointer stays valid until the thread's next library call. */
const char* moe_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H_ */
