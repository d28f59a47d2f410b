/*
 * moe.h -- C ABI of libmoe.so: the Kimi-K2 routed mixture-of-experts FFN layer
 * (sigmoid scoring, correction-bias top-k, renormalised and scaled weights,
 * SwiGLU experts plus a shared expert) as hand-written HIP kernels for gfx950.
 *
 * Conventions (all entry points)
 * ------------------------------
 *  - Every tensor pointer is a DEVICE pointer owned by the caller, row-major,
 *    16-byte aligned.  The library never allocates, frees or synchronises;
 *    every call only enqueues kernels on `stream` (a hipStream_t passed as
 *    void*, NULL = the null stream) and returns.
 *  - Scratch memory is a caller-owned device workspace of at least
 *    moe_workspace_size(cfg, num_tokens) bytes (256-byte aligned).  Calls that
 *    share a workspace must be ordered (same stream).  No entry point uses
 *    hipMemset, so a caller may capture a whole call in a HIP graph.
 *  - Arguments are validated on the host before anything is launched; a bad
 *    argument returns an error code and launches nothing.  num_tokens == 0 is
 *    a no-op that returns MOE_OK.  moe_last_error() gives a message for the
 *    last failure on the calling thread.
 *  - Launch failures (hipGetLastError after a launch) return MOE_ERR_HIP.
 *  - num_tokens is at most 65536.
 *
 * Shapes: T = num_tokens, H = hidden_size, F = moe_intermediate_size,
 * E = n_routed_experts, k = num_experts_per_tok, Fs = n_shared_experts * F.
 * Field names follow the model config tables ("Kimi K2 Base" / "Kimi K2 0905"
 * raw config fields).  Linear weights are [out][in] without bias ("Kimi K2 .
 * Down projection": "[out, in]", no bias parameter).
 */
#ifndef MOE_H_
#define MOE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 1

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1, /* null pointer, bad size, misaligned pointer */
  MOE_ERR_UNSUPPORTED = 2, /* valid but not implemented (dtype, scoring)    */
  MOE_ERR_WORKSPACE = 3,   /* ws_bytes < moe_workspace_size(cfg, T)        */
  MOE_ERR_HIP = 4          /* a HIP launch failed                          */
} moe_status_t;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1, MOE_FP8_E4M3 = 2 } moe_dtype_t;

/* scoring_func / topk_method values (raw config fields: scoring_func sigmoid,
 * topk_method noaux_tc are the only ones accepted). */
enum { MOE_SCORING_SIGMOID = 0 };
enum { MOE_TOPK_NOAUX_TC = 0 };

typedef struct {
  int32_t hidden_size;           /* H; multiple of 128                          */
  int32_t moe_intermediate_size; /* F; multiple of 128                          */
  int32_t n_routed_experts;      /* E; 1..1023                                  */
  int32_t num_experts_per_tok;   /* k; 1..32, and <= E where routing reads it    */
  int32_t n_shared_experts;      /* 0..8; shared width Fs = n_shared * F         */
  int32_t n_group;               /* >= 1, divides E, <= 64                       */
  int32_t topk_group;            /* 1..n_group; k <= topk_group * E / n_group    */
  int32_t norm_topk_prob;        /* 1: renormalise the k weights to sum 1        */
  float routed_scaling_factor;   /* 2.827 for K2                                 */
  int32_t scoring_func;          /* MOE_SCORING_SIGMOID                          */
  int32_t topk_method;           /* MOE_TOPK_NOAUX_TC                            */
  int32_t act_dtype;             /* x, router weight, y, out: MOE_F32 / MOE_BF16 */
  int32_t weight_dtype;          /* expert weights: MOE_F32 / MOE_BF16 / MOE_FP8_E4M3 */
  int32_t weight_block_size[2];  /* {128,128} for MOE_FP8_E4M3, else {0,0}       */
} moe_config_t;
/* Accepted dtype pairs (act, weight): (F32, F32), (BF16, BF16), (BF16, FP8_E4M3). */

typedef struct {
  /* routed experts, [E][F][H], [E][F][H], [E][H][F] of weight_dtype */
  const void *w_gate, *w_up, *w_down;
  /* FP8 only: fp32 block scales [E][F/128][H/128], same, [E][H/128][F/128] */
  const float *s_gate, *s_up, *s_down;
  /* shared expert: [Fs][H], [Fs][H], [H][Fs]; NULL when n_shared_experts == 0 */
  const void *sh_gate, *sh_up, *sh_down;
  /* FP8 only: [Fs/128][H/128], same, [H/128][Fs/128] */
  const float *sh_s_gate, *sh_s_up, *sh_s_down;
} moe_weights_t;

/* Bytes of workspace every entry point below needs for T tokens (the maximum
 * over the entry points, so one workspace serves all of them); 0 for an
 * invalid configuration or a token count outside 0..65536. */
size_t moe_workspace_size(const moe_config_t* cfg, int64_t num_tokens);

/* Router ("Kimi K2 Base"/"Kimi K2 0905" raw config fields: scoring_func
 * sigmoid, topk_method noaux_tc, n_group, topk_group, num_experts_per_tok,
 * norm_topk_prob, routed_scaling_factor).
 *   s = sigmoid(x W_r^T); sel = s + router_bias (selection only);
 *   if n_group > 1 only the topk_group groups (contiguous, E/n_group experts)
 *   with the largest sum-of-two-best sel stay eligible;
 *   topk_ids = the k largest sel (ties: lower id), written ascending;
 *   topk_weights = s[ids] / sum(s[ids]) (if norm_topk_prob) * routed_scaling_factor.
 * Every token gets k distinct ids in [0, E), whatever its values: a NaN sel
 * (from NaN or infinite inputs) orders as -inf, and experts that are not
 * eligible (groups not kept) are taken, lowest id first, only when fewer than
 * k eligible experts with a finite sel remain.
 * x [T][H] act_dtype; router_w [E][H] act_dtype; router_bias [E] fp32;
 * topk_ids [T][k] int32; topk_weights [T][k] fp32. */
moe_status_t moe_route(const moe_config_t* cfg, const void* x, const void* router_w,
                       const float* router_bias, int64_t num_tokens, int32_t* topk_ids,
                       float* topk_weights, void* ws, size_t ws_bytes, void* stream);

/* Grouping of the T*k (token, slot) pairs by expert: the stable sort of the
 * pairs by expert id, in flat order t*k + j inside a segment.
 *   expert_offsets [E+1]: segment of expert e is [offsets[e], offsets[e+1]),
 *     offsets[E] = the number of grouped pairs (T*k when every id is valid);
 *   sorted_token_ids [T*k]: token of each grouped row, ascending inside a
 *     segment; entries from offsets[E] on are left untouched;
 *   inv_perm [T*k]: inv_perm[t*k+j] = grouped row of (t, j), or -1;
 *   x_perm [T*k][H]: x[sorted_token_ids[p]]; act_dtype, or for FP8 weights the
 *     e4m3 codes (1 byte each) of the dynamically quantised row, with
 *   x_perm_scales [T*k][H/128] fp32 (FP8 only, else may be NULL): per token and
 *     128 channels s = amax/448 (1 if all zero), code = e4m3(RNE, saturating)(x/s)
 *     ("Kimi K2 . Down projection", quantization_config: activation_scheme dynamic).
 * x_perm may be NULL (then only the index arrays are produced); its rows
 * from offsets[E] on are left untouched.
 * topk_ids may hold any int32 values.  moe_route writes k distinct ids in
 * [0, E) per token; other callers may not:
 *   - a pair whose id lies outside [0, E) (for instance an expert another
 *     expert-parallel rank holds) is not grouped: it is not counted, takes no
 *     row, and its inv_perm entry is -1;
 *   - a token may name one expert in several slots: each such pair is a row
 *     of its own, in slot order. */
moe_status_t moe_permute(const moe_config_t* cfg, const void* x, const int32_t* topk_ids,
                         int64_t num_tokens, int32_t* expert_offsets, int32_t* sorted_token_ids,
                         int32_t* inv_perm, void* x_perm, float* x_perm_scales, void* ws,
                         size_t ws_bytes, void* stream);

/* Expert FFNs ("Kimi K2 . Down projection": down_proj(act_fn(gate_proj(x)) *
 * up_proj(x)), act_fn silu): for every grouped row p of expert e,
 *   y_perm[p] = W_down[e] (silu(W_gate[e] a_p) * (W_up[e] a_p)), a_p = x_perm[p];
 * and for every token t the shared expert y_shared[t] = the same form on x[t]
 * with the shared weights.  FP8: a_p is the dequantised x_perm row; the shared
 * expert quantises x the same way; the SwiGLU output is quantised again per row
 * and 128 channels before the down projection; weights are code * block scale.
 * x [T][H] act_dtype; x_perm/x_perm_scales as produced by moe_permute;
 * expert_offsets [E+1]; y_perm [T*k][H] act_dtype; y_shared [T][H] act_dtype
 * (ignored when n_shared_experts == 0).
 * Only the rows [0, offsets[E]) of x_perm / y_perm are used; rows after it
 * are left untouched.  Each segment is clamped into [0, T*k] on the device,
 * so no offsets array makes the kernels leave the buffers.
 * Expert parallelism ("Behind Kimi-K2's Config" section 2.1: at EP=128 a
 * DeepSeek-V3 rank holds 2 routed + 1 shared expert per layer, so K2's 384
 * give 3 + 1): one rank's share is
 * this call with E = its local expert count, x_perm = the rows dispatched to
 * it grouped by local expert, x / T = its own tokens for the shared expert,
 * and k any row capacity per token with T*k >= offsets[E].  This entry point
 * therefore does not apply the routing constraints (k <= E, n_group,
 * topk_group); k is 1..32. */
moe_status_t moe_expert_ffn(const moe_config_t* cfg, const moe_weights_t* w, const void* x,
                            const void* x_perm, const float* x_perm_scales,
                            const int32_t* expert_offsets, int64_t num_tokens, void* y_perm,
                            void* y_shared, void* ws, size_t ws_bytes, void* stream);

/* Weighted combine with the shared-expert add:
 *   out[t] = y_shared[t] + sum_{j<k} topk_weights[t][j] * y_perm[inv_perm[t*k+j]],
 * accumulated in fp32 in slot order, rounded once to act_dtype (nearest even).
 * A slot whose inv_perm entry lies outside [0, T*k) (a pair moe_permute did
 * not group: -1) contributes nothing.
 * y_shared may be NULL when n_shared_experts == 0.  out [T][H] act_dtype. */
moe_status_t moe_combine(const moe_config_t* cfg, const void* y_perm, const void* y_shared,
                         const float* topk_weights, const int32_t* inv_perm, int64_t num_tokens,
                         void* out, void* stream);

/* The whole layer: route -> group -> expert FFNs (rows gathered on the fly,
 * nothing materialised per row beyond the SwiGLU output) -> combine.
 * out [T][H] act_dtype.  topk_ids_out [T][k] int32 and topk_weights_out
 * [T][k] fp32 are optional (NULL: kept in the workspace). */
moe_status_t moe_layer_forward(const moe_config_t* cfg, const moe_weights_t* w, const void* x,
                               const void* router_w, const float* router_bias, int64_t num_tokens,
                               void* out, int32_t* topk_ids_out, float* topk_weights_out,
                               void* ws, size_t ws_bytes, void* stream);

/* moe_layer_forward for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same computation and results, bit for bit, with the
 * workspace taken from a fixed array of MOE_STATIC_SCRATCH_BYTES that the
 * library holds on each GPU it runs on (from the first call on that device
 * until the process ends).  Calls nothing that allocates.  Rejects, with
 * MOE_ERR_WORKSPACE and launching nothing, a token count whose workspace
 * (moe_workspace_size) exceeds MOE_STATIC_SCRATCH_BYTES (Kimi-K2 bf16:
 * about 330 tokens).  The array is shared by every call on one GPU and keeps
 * the last call's contents: calls that overlap on one GPU (concurrent
 * streams or threads) race; order them on one stream.  The device is the
 * current HIP device of the calling thread. */
#define MOE_STATIC_SCRATCH_BYTES (64ull << 20)
moe_status_t moe_layer_forward_static(const moe_config_t* cfg, const moe_weights_t* w, const void* x,
                                      const void* router_w, const float* router_bias, int64_t num_tokens,
                                      void* out, int32_t* topk_ids_out, float* topk_weights_out, void* stream);

/* The MoE sub-block of a decoder layer: the pre-MoE RMSNorm, the layer, and
 * the residual add ("Kimi K2 Base" architecture table: RMSNorm; raw config
 * fields: rms_norm_eps 1e-06):
 *   u[t]   = act( x[t] / sqrt(mean_h x[t][h]^2 + rms_norm_eps) * norm_weight ),
 *            computed in fp64 and rounded once to act_dtype (nearest even);
 *   out[t] = act( x[t] + shared(u[t]) + sum_j w_tj expert_j(u[t]) ),
 *            accumulated in fp32 in that order, rounded once.
 * Routing and the experts see u exactly as moe_layer_forward sees its x (with
 * fp8 weights the same pass writes u's e4m3 codes).  x [T][H] act_dtype is
 * the residual stream; norm_weight [H] act_dtype; rms_norm_eps in [0, 1).
 * Other arguments as moe_layer_forward; out may not alias x. */
moe_status_t moe_block_forward(const moe_config_t* cfg, const moe_weights_t* w, const void* x,
                               const void* norm_weight, float rms_norm_eps, const void* router_w,
                               const float* router_bias, int64_t num_tokens, void* out,
                               int32_t* topk_ids_out, float* topk_weights_out, void* ws,
                               size_t ws_bytes, void* stream);

/* Where an intermediate of the last call lies in the caller's workspace, for
 * inspecting it afterwards (the layout depends only on cfg and num_tokens):
 * *offset and *bytes of region `region` (MOE_WS_*) for T tokens.  Contents
 * after moe_expert_ffn / moe_layer_forward / moe_block_forward on that
 * workspace ("Kimi K2 . Down projection": h = act_fn(gate_proj(x)) *
 * up_proj(x) is the input of down_proj):
 *   MOE_WS_H            [T*k][F] routed SwiGLU output h, act_dtype (with FP8
 *                       weights: unspecified);
 *   MOE_WS_H_CODES      [T*k][F] e4m3 codes of h (FP8 weights), quantised per
 *                       row and 128 channels as x is (quantization_config:
 *                       activation_scheme dynamic);
 *   MOE_WS_H_SCALES     [T*k][F/128] fp32 scales of those codes;
 *   MOE_WS_H_SHARED, MOE_WS_H_SHARED_CODES, MOE_WS_H_SHARED_SCALES: the same
 *                       for the shared expert, [T][Fs], [T][Fs/128];
 *   MOE_WS_Y, MOE_WS_Y_SHARED: [T*k][H] and [T][H] down outputs, act_dtype
 *                       (moe_layer_forward / moe_block_forward only;
 *                       moe_expert_ffn writes them to its y_perm / y_shared).
 * Rows are the grouped rows of the call's expert_offsets.  Regions that the
 * configuration does not use have 0 bytes.  Returns MOE_ERR_INVALID_ARG for a
 * bad configuration, token count, region or NULL output pointer. */
enum {
  MOE_WS_H = 0,
  MOE_WS_H_CODES = 1,
  MOE_WS_H_SCALES = 2,
  MOE_WS_H_SHARED = 3,
  MOE_WS_H_SHARED_CODES = 4,
  MOE_WS_H_SHARED_SCALES = 5,
  MOE_WS_Y = 6,
  MOE_WS_Y_SHARED = 7,
  MOE_WS_COUNT = 8
};
moe_status_t moe_workspace_region(const moe_config_t* cfg, int64_t num_tokens, int32_t region,
                                  size_t* offset, size_t* bytes);

const char* moe_status_string(moe_status_t status);
/* Message describing the last failure on the calling thread ("" if none). */
const char* moe_last_error(void);
int moe_abi_version(void);

/* Profiling aid.  Arms a one-shot pair of HIP events (hipEvent_t passed as
 * void*) that the next launch of kernel `kernel_id` (MOE_KID_*) made by a
 * library call on the calling thread records around itself, on that call's
 * stream; NULL/NULL disarms.  The arming is per thread.  A launch into a
 * stream that is being captured into a HIP graph records nothing and leaves
 * the events armed. */
enum {
  MOE_KID_ROUTER_LOGITS = 0, /* x W_r^T                                        */
  MOE_KID_ROUTER_TOPK = 1,   /* sigmoid, bias, groups, top-k, weights          */
  MOE_KID_PERMUTE = 2,       /* histogram + scan + stable scatter: 3 kernels,
                                one up to 256 tokens (in the layer it also
                                writes the work list)                          */
  MOE_KID_TILES = 3,         /* work list of the grouped GEMMs (when not
                                written by the grouping kernel)               */
  MOE_KID_GATHER = 4,        /* x_perm rows (moe_permute only)                 */
  MOE_KID_ACT_QUANT = 5,     /* fp8 activation quantisation of x               */
  MOE_KID_GATE_UP = 6,       /* grouped gate/up GEMM + SiLU * up               */
  MOE_KID_DOWN = 7,          /* grouped down GEMM                              */
  MOE_KID_COMBINE = 8,       /* weighted combine + shared add                  */
  MOE_KID_NORM = 9,          /* pre-MoE RMSNorm (moe_block_forward)            */
  MOE_KID_COUNT = 10
};
moe_status_t moe_profile_arm(int32_t kernel_id, void* ev_start, void* ev_stop);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H_ */
