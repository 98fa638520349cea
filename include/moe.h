/*
 * moe.h -- C ABI of the MI355X (gfx950) sparse Mixture-of-Experts layer
 * forward pass: router -> gating -> dispatch -> expert FFNs -> combine.
 *
 * Pages cited (titles as published):
 *   [devtips]  devtips.kr, "MoE (Mixture of Experts) 아키텍처 완전 정복:
 *              Mixtral부터 DeepSeek-MoE까지 구현 원리와 실전 최적화 기법"
 *   [garden]   ricepunchb.github.io obsidian garden, "Mixture of Experts (MoE)"
 *   [yj-zh]    youngju.dev, "Mixture of Experts（MoE）架构深度解析：从 Switch
 *              Transformer 到 Mixtral 的演进与高效扩展策略"
 *   [yj-ja]    youngju.dev, "Sparse Mixture of Experts（MoE）アーキテクチャ深層分析：
 *              設計原理からDeepSeek-V3・Qwen3まで"
 *   [lecture]  study-site lecture-03, "Mixture of Experts"
 *
 * General rules for every entry point
 *   - Pointers named "device" point to GPU memory that the caller allocated
 *     and owns; the library allocates no memory and keeps none of them.
 *     Vector-loaded buffers (x, weights, x_perm, y_perm, y, workspace) must
 *     be 16-byte aligned.
 *   - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL = the
 *     default stream).  The library never synchronises the host with the
 *     device, except in moe_timing_read().
 *   - Argument and shape checks run on the host before any launch and
 *     return MOE_ERR_INVALID_ARG / MOE_ERR_UNSUPPORTED / MOE_ERR_WORKSPACE
 *     with nothing enqueued.  A failed launch returns MOE_ERR_HIP.  Device
 *     faults surface at the caller's next synchronisation.  moe_last_error()
 *     returns a message for the last non-OK status of the calling thread.
 *   - Results are deterministic: the same inputs give the same bits.
 *   - Inputs must be finite; NaN logits give unspecified routing.
 *   - Layouts are row-major; weights follow nn.Linear ([out][in]), stacked
 *     over experts.  dtype MOE_BF16 means bfloat16 storage with float32
 *     accumulation; MOE_F32 is float32 throughout.
 *   - Supported shapes (else MOE_ERR_UNSUPPORTED): d_model, d_ff and
 *     d_ff_shared multiples of 64 (bf16) or 16 (f32) and at most 2^21;
 *     num_shared * d_ff_shared at most 2^21 and the shared down projection
 *     (num_shared * d_model * d_ff_shared elements) under 2^31 bytes;
 *     num_experts <= 1024, and <= 256 for the fused router and the router
 *     losses; expert-choice capacity <= 4096; T * k < 2^31.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum moe_status {
    MOE_OK = 0,
    MOE_ERR_INVALID_ARG = 1,
    MOE_ERR_UNSUPPORTED = 2,
    MOE_ERR_WORKSPACE = 3,
    MOE_ERR_HIP = 4
} moe_status;

/* Gating.  Selection always ranks experts (or, for expert choice, tokens)
 * by their float32 logit, larger first; equal logits rank the lower index
 * first; -0.0 equals +0.0.
 *   MOE_GATE_TOPK_SOFTMAX  top-k of the logits, then softmax over the k
 *       kept logits ([devtips] MoELayer; [yj-zh] GatingNetwork,
 *       MixtralMoELayer).  Softmax over all experts, top-k, renormalise
 *       ([yj-ja] TopKGating) is the same function.
 *   MOE_GATE_SOFTMAX_TOPK  softmax over all E logits, kept unrenormalised
 *       for the top-k experts ([yj-ja] gating formula).
 *   MOE_GATE_SWITCH        top-1; gate = largest softmax probability; with
 *       capacity dropping ([yj-zh] SwitchRouter).  top_k must be 1.
 *   MOE_GATE_EXPERT_CHOICE each expert takes its C best tokens; scores are
 *       a softmax over the token axis ([yj-zh] ExpertChoiceRouter; [yj-ja]
 *       ExpertChoiceGating).  top_k is ignored. */
typedef enum moe_gating {
    MOE_GATE_TOPK_SOFTMAX = 0,
    MOE_GATE_SOFTMAX_TOPK = 1,
    MOE_GATE_SWITCH = 2,
    MOE_GATE_EXPERT_CHOICE = 3
} moe_gating;

/* Expert FFN.
 *   MOE_ACT_RELU      y = W2 relu(W1 u + b1) + b2   ([devtips] MoELayer experts)
 *   MOE_ACT_GELU_ERF  y = W2 gelu(W1 u + b1) + b2, exact erf GELU ([yj-zh] MoELayer)
 *   MOE_ACT_SWIGLU    y = W2 (silu(W1 u) * (W3 u)) ([yj-zh] SwiGLUExpert w1/w3/w2;
 *                     [yj-ja] SwiGLUExpert w_gate/w_up/w_down; [lecture] SwiGLU row)
 * The optional shared experts are always SwiGLU ([yj-zh] DeepSeekMoELayer).
 * S of them of width Fs run as one SwiGLU expert of width S*Fs: their
 * stacked gate and up rows are the [S*Fs][d] matrices of that expert, and the
 * down projection reads the S [d][Fs] blocks as consecutive slices of its
 * hidden axis, so the S outputs are summed inside one accumulation. */
typedef enum moe_act { MOE_ACT_RELU = 0, MOE_ACT_GELU_ERF = 1, MOE_ACT_SWIGLU = 2 } moe_act;

typedef enum moe_dtype { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype;

typedef struct moe_config {
    int32_t num_tokens;      /* T = batch * sequence (flattened, [yj-zh] MixtralMoELayer) */
    int32_t d_model;         /* d */
    int32_t num_experts;     /* E, routed experts */
    int32_t top_k;           /* k, token choice only */
    int32_t d_ff;            /* F, hidden width of each routed expert */
    int32_t d_ff_shared;     /* hidden width Fs of each always-on shared expert, 0 = none */
    int32_t gating;          /* moe_gating */
    int32_t act;             /* moe_act */
    int32_t dtype;           /* moe_dtype of x, all weights, x_perm, y_perm and y */
    int32_t capacity_group;  /* token choice with capacity: tokens per capacity
                                group (the sequence length; a multiple of 64),
                                0 = all T tokens */
    float capacity_factor;   /* SWITCH (required) and TOPK_SOFTMAX / SOFTMAX_TOPK
                                (optional, 0 = no capacity): per group and expert
                                C = max(min_capacity, int(cf * G * k / E)), G =
                                capacity_group or T ([yj-zh] SwitchRouter; the
                                [devtips] capacity example scales by top_k);
                                assignments are kept in token order, the rest
                                dropped.  EXPERT_CHOICE: C = int(cf * T / E). */
    int32_t min_capacity;    /* floor of the token-choice capacity ([yj-zh]
                                DeepSpeed MoE configuration example); 0 = none */
    int32_t num_shared;      /* S always-on shared SwiGLU experts of width
                                d_ff_shared, whose outputs are summed ([yj-zh]
                                DeepSeekMoELayer num_shared_experts; [devtips]
                                DeepSeekMoE); must be >= 1 when d_ff_shared > 0
                                and is ignored when d_ff_shared == 0 */
} moe_config;

/* Weights (device pointers). */
typedef struct moe_weights {
    const void *w_router;  /* [E][d] dtype */
    const float *b_router; /* [E] float32 or NULL: router bias / fixed logit skew */
    const void *w1;        /* [E][F][d] first linear (ReLU/GELU) or gate projection (SwiGLU) */
    const void *w3;        /* [E][F][d] up projection, SwiGLU only, else NULL */
    const void *w2;        /* [E][d][F] down projection */
    const float *b1;       /* [E][F] float32 or NULL; ReLU/GELU only */
    const float *b2;       /* [E][d] float32 or NULL; ReLU/GELU only */
    const void *ws1;       /* shared experts' gate  [S][Fs][d] dtype, or NULL */
    const void *ws3;       /* shared experts' up    [S][Fs][d] dtype, or NULL */
    const void *ws2;       /* shared experts' down  [S][d][Fs] dtype, or NULL */
} moe_weights;

/* Routing buffers (device pointers), written by moe_route / moe_permute and
 * read by moe_expert_ffn / moe_combine.  A_max = T*k for token choice and
 * E*C for expert choice. */
typedef struct moe_routing {
    float *logits;       /* [T][E] float32; moe_route writes it when non-NULL
                            (required for EXPERT_CHOICE) */
    int32_t *topk_idx;   /* token choice: [T][k] expert of slot j, slot j = rank j;
                            expert choice: [E][C] chosen tokens in rank order */
    float *topk_w;       /* token choice: [T][k] gate weights; expert choice: [E][C] scores */
    int32_t *counts;     /* [E] rows kept per expert */
    int32_t *offsets;    /* [E+1] exclusive prefix sum of counts */
    int32_t *row_token;  /* [A_max] token of each expert-contiguous row; rows of
                            expert e are offsets[e]..offsets[e+1]-1 in ascending
                            token order (expert choice: rank order) */
    int32_t *slot_row;   /* token choice: [T][k] row of slot j or -1 if dropped;
                            expert choice: [T][E] row of (token, expert) or -1 */
} moe_routing;

/* Capacity C of the configuration: int(cf * G / E) evaluated in double,
 * 0 for gatings without capacity. */
moe_status moe_capacity(const moe_config *cfg, int32_t *capacity);

/* Workspace bytes for a stage: MOE_STAGE_FORWARD (moe_forward with routing
 * == NULL, which keeps every routing buffer and intermediate in the
 * workspace), MOE_STAGE_PERMUTE (moe_permute), MOE_STAGE_FFN (moe_expert_ffn),
 * MOE_STAGE_LOSSES (moe_router_losses). */
enum { MOE_STAGE_FORWARD = 0, MOE_STAGE_PERMUTE = 1, MOE_STAGE_FFN = 2, MOE_STAGE_LOSSES = 3 };
moe_status moe_workspace_size(const moe_config *cfg, int32_t stage, size_t *bytes);

/* Router GEMM fused with gating: logits = x W_router^T + b_router (float32
 * accumulation), then the gating of cfg->gating.  Token choice writes
 * topk_idx/topk_w ([T][k]) and logits if non-NULL; expert choice writes
 * logits, then topk_idx/topk_w as [E][C] ([yj-ja] gating formula; [yj-zh]
 * GatingNetwork, SwitchRouter, ExpertChoiceRouter).
 * x: device [T][d] dtype.  E must be <= 256 for token choice; expert choice
 * needs C <= 4096. */
moe_status moe_route(const moe_config *cfg, const void *x, const moe_weights *w,
                     moe_routing *routing, void *stream);

/* Noisy top-k router ([yj-ja] TopKGating, training branch; [garden]
 * "7. 안정화 기법" Noisy Top-k): logits = x W_router^T + b_router +
 * softplus(x W_noise^T) * noise, then the gating of cfg->gating on those
 * logits.  w_noise: device [E][d] dtype; noise: device [T][E] float32, the
 * standard-normal draw supplied by the caller (the library draws nothing).
 * Token choice only; otherwise as moe_route. */
moe_status moe_route_noisy(const moe_config *cfg, const void *x, const moe_weights *w, const void *w_noise,
                           const float *noise, moe_routing *routing, void *stream);

/* Router side outputs of token-choice gating ([yj-ja]
 * compute_load_balancing_loss and router_z_loss; [yj-zh] load_balancing_loss):
 *   out[0] = E * sum_e f_e * P_e  (load-balancing loss, before any weight),
 *   out[1] = mean over tokens of logsumexp(logits_t)^2  (router z-loss),
 *   out[2 + e] = P_e = mean over tokens of softmax(logits_t)_e,
 * with f_e = (assignments to e in topk_idx) / (T * k), counted before any
 * capacity drop.  logits: device [T][E] float32; topk_idx: device [T][k];
 * out: device float [2 + E].  Deterministic fixed-order reductions.
 * ws: MOE_STAGE_LOSSES bytes.  E <= 256; not defined for expert choice. */
moe_status moe_router_losses(const moe_config *cfg, const float *logits, const int32_t *topk_idx, float *out,
                             void *ws, size_t ws_bytes, void *stream);

/* The gating step alone on caller-provided float32 logits [T][E] (device):
 * the same selection and weights moe_route applies after its router GEMM.
 * routing->logits is ignored. */
moe_status moe_route_from_logits(const moe_config *cfg, const float *logits,
                                 moe_routing *routing, void *stream);

/* Counts, capacity and permutation, then the gather of token rows into
 * expert-contiguous x_perm [A_max][d] (rows >= offsets[E] are not written).
 * Reads topk_idx; writes counts, offsets, row_token, slot_row.  SWITCH keeps,
 * per capacity group and expert, the first C tokens in sequence order and
 * drops the rest ([yj-zh] SwitchRouter).  ws: MOE_STAGE_PERMUTE bytes. */
moe_status moe_permute(const moe_config *cfg, const void *x, moe_routing *routing,
                       void *x_perm, void *ws, size_t ws_bytes, void *stream);

/* moe_permute for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * no workspace argument.  The scratch space moe_permute takes from `ws`
 * (per-chunk expert counts, prefixes and bases, per-assignment ranks) comes
 * from a fixed array in the library's own device memory instead, of
 * MOE_PERMUTE_NOALLOC_SCRATCH_BYTES per GPU, allocated when the library's
 * code is loaded on that GPU and held until the process ends.  Calls no
 * hipMalloc/hipFree and records no timing events.  A configuration whose
 * MOE_STAGE_PERMUTE workspace exceeds that size returns MOE_ERR_UNSUPPORTED
 * before any launch (8 MiB holds, e.g., T = 65536 tokens with k = 8 of
 * E = 256 experts).  Every call on one GPU shares that GPU's array: calls
 * that overlap on one GPU (on different streams, or from host threads that
 * do not order them) race and give undefined results.  Each call writes
 * every scratch entry it reads, so nothing carries over from the previous
 * call.  `stream` must belong to the current device.  Arguments, results
 * and errors otherwise as moe_permute. */
#define MOE_PERMUTE_NOALLOC_SCRATCH_BYTES (8u << 20)
moe_status moe_permute_noalloc(const moe_config *cfg, const void *x, moe_routing *routing, void *x_perm,
                               void *stream);

/* Expert FFNs as grouped GEMMs over the expert-contiguous rows: y_perm [A_max][d]
 * (dtype) for rows < offsets[E]; y_shared [T][d] (dtype) = the sum of the
 * shared experts of x when cfg->d_ff_shared > 0 (x: device [T][d], else may be NULL).  Only the
 * rows routed to an expert are computed for it ([lecture] "Token Routing":
 * unselected experts do no work).  ws: MOE_STAGE_FFN bytes (holds the hidden
 * activations). */
moe_status moe_expert_ffn(const moe_config *cfg, const void *x_perm, const void *x,
                          const moe_routing *routing, const moe_weights *w, void *y_perm,
                          void *y_shared, void *ws, size_t ws_bytes, void *stream);

/* Gate-weighted combine y[t] = sum_slots w * y_perm[row] (+ y_shared[t]),
 * float32 accumulation in slot order (expert choice: expert order), output
 * in dtype; tokens with no kept slot get 0 (+ shared) ([yj-ja] gating
 * formula y = sum_i G(x)_i E_i(x); [garden] "4. 기본 구조" weighted sum). */
moe_status moe_combine(const moe_config *cfg, const void *y_perm, const void *y_shared,
                       const moe_routing *routing, void *y, void *stream);

/* The whole layer: route -> permute -> expert_ffn -> combine, no host
 * synchronisation.  routing may be NULL (all routing buffers in ws) or a
 * caller-owned set that receives the routing.  ws: MOE_STAGE_FORWARD bytes.
 * With float32 data, or bf16 data and T*d*2 < 2^31, the first expert GEMM
 * reads the routed rows of x through routing.row_token instead of a gathered
 * x_perm (same values, same result). */
moe_status moe_forward(const moe_config *cfg, const void *x, const moe_weights *w, void *y,
                       moe_routing *routing, void *ws, size_t ws_bytes, void *stream);

/* Message for the calling thread's last non-OK status ("" if none). */
const char *moe_last_error(void);

/* Per-kernel timing with hipEvents recorded on the launching stream around
 * every kernel the library launches (off by default).  moe_timing_read
 * synchronises on the recorded events and returns the summed duration and
 * launch count of kernel kind `kind` since the last reset; kinds are listed
 * by moe_kernel_name (NULL past the last). */
moe_status moe_timing_enable(int32_t on);
moe_status moe_timing_reset(void);
moe_status moe_timing_read(int32_t kind, double *total_ms, int64_t *launches);
const char *moe_kernel_name(int32_t kind);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
