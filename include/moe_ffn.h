/*
 * moe_ffn.h - C ABI of the MI355X (gfx950) token-choice sparse MoE FFN
 * layer forward.
 *
 * The layer (the pages cited below are "Mixture of Experts for LLM
 * Inference" [MoE-LLM], "AI Infrastructure series - Part 12 of 24" [AIS-12],
 * "Chapter 19: Mixture-of-Experts Models" [CH19] and "Mixture of Experts
 * Explained" [MoE-EXP]):
 *
 *   s      = x @ W_router (+ logit_offset)            router logits
 *   select top-k experts per token (softmax: by logit; sigmoid: by
 *          sigmoid(s) + select_bias, the bias used for selection only)
 *   g      = softmax over the k selected logits  |  sigmoid(s_sel)/sum
 *   out[t] = sum_i g[t,i] * FFN_{idx[t,i]}(x[t])  (+ FFN_shared(x[t]))
 *   FFN(x) = W_down (silu(W_gate x) * (W_up x))    (SwiGLU expert)
 *
 * Conventions for every entry point:
 *   - Pointers are DEVICE pointers unless stated otherwise, owned by the
 *     caller.  The library never allocates device memory; scratch space is
 *     the caller's workspace, sized by moe_workspace_bytes().  Activation,
 *     weight, scale and workspace buffers must be 16-byte aligned (every
 *     hipMalloc result is); a misaligned one returns MOE_ERR_INVALID_ARG.
 *     Index and gate arrays (int32 / float32) need only their natural
 *     alignment.
 *   - Calls are asynchronous on `stream`; results are valid once the stream
 *     has synchronised.  No entry point copies device data to the host or
 *     synchronises the stream.
 *   - Arguments are checked on the host before any HIP call; a bad argument
 *     returns an error status and launches nothing.  A failed launch returns
 *     MOE_ERR_HIP; moe_last_error() then gives the HIP message (per thread).
 *   - Row-major layouts; experts are numbered 0..N-1.  Expert ids and token
 *     indices are int32.  Entry points hold no state and may be called from
 *     several host threads.
 *   - Supported types: x/out float32 or bfloat16; expert weights float32
 *     (with float32 activations), bfloat16, OCP FP8 E4M3 with one float32
 *     scale per 128x128 block, or MXFP4 (E2M1 codes, one E8M0 scale byte per
 *     32 consecutive inputs, 2^(byte - 127), byte 255 = NaN; [AIS-12]
 *     "Quantize the experts first": gpt-oss ships its experts in MXFP4) -
 *     the last three with bfloat16
 *     activations.  The router weight, offset and bias are always float32.
 *   - Shape limits (else MOE_ERR_UNSUPPORTED): N <= 512, k <= 64;
 *     n_shared in {0,1}; bfloat16 weights need d_model % 32 == 0 and
 *     d_ff % 32 == 0; FP8 and MXFP4 weights need d_model % 128 == 0 and
 *     d_ff % 128 == 0; bfloat16 activations need d_model % 8 == 0.  bfloat16,
 *     FP8 and MXFP4 experts run through the weight-streaming kernels at
 *     small batches and through the tiled MFMA GEMM once the routed experts
 *     average 64 rows or more (d_model % 256 == 0 and d_ff % 128 == 0; MXFP4
 *     also needs its operands within 32-bit offsets, else it streams).
 *     float32 weights need n_tokens * top_k <= 1048560.  Invalid values
 *     (k < 1, k > N, negative sizes, ...) are MOE_ERR_INVALID_ARG.
 *     n_tokens == 0 is a valid no-op.
 */
#ifndef MOE_FFN_H
#define MOE_FFN_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1,         /* null pointer, bad value              */
  MOE_ERR_UNSUPPORTED = 2,         /* valid but outside the limits above   */
  MOE_ERR_WORKSPACE_TOO_SMALL = 3, /* ws_bytes < moe_workspace_bytes()     */
  MOE_ERR_HIP = 4                  /* a HIP call failed; see last_error    */
} moe_status_t;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1, MOE_FP8_E4M3 = 2, MOE_MXFP4 = 3 } moe_dtype_t;

/* softmax over the top-k logits ([CH19] 19.3.2; [MoE-EXP] "The router, with
 * real numbers"), or sigmoid affinities with a selection-only per-expert
 * bias and renormalised selected affinities ([AIS-12] worked example,
 * DeepSeek-V3 paragraph; [MoE-LLM] "DeepSeek-style bias controller";
 * [CH19] 19.3.4). */
typedef enum { MOE_ROUTE_SOFTMAX_TOPK = 0, MOE_ROUTE_SIGMOID_BIAS = 1 } moe_route_t;

typedef struct {
  int32_t n_tokens;   /* T  >= 0                                          */
  int32_t d_model;    /* d  >= 1                                          */
  int32_t n_experts;  /* N  routed experts                                */
  int32_t top_k;      /* k                                                */
  int32_t d_ff;       /* expert hidden width                              */
  int32_t n_shared;   /* 0 or 1 always-on shared expert ([MoE-LLM]
                         "Shared experts"; [AIS-12] "What is a shared
                         expert?")                                         */
  int32_t route;      /* moe_route_t                                      */
  int32_t act_dtype;  /* MOE_F32 | MOE_BF16 : x, out                       */
  int32_t w_dtype;    /* MOE_F32 | MOE_BF16 | MOE_FP8_E4M3 | MOE_MXFP4 :
                         expert weights                                    */
} moe_shape_t;

/* Device pointers to the layer's parameters.  Expert weights are in the
 * packed layout written by moe_pack_weights().  FP8 scales stay in their
 * natural layout, float32 [E][rows/128][cols/128]; MXFP4 scales (E8M0 bytes,
 * value 2^(byte - 127), one per 32 inputs of a row) are passed packed by
 * moe_pack_weights() with which = 2 or 3. */
typedef struct {
  const float* w_router;     /* [d][N]                                    */
  const float* logit_offset; /* [N] added to the logits, or NULL          */
  const float* select_bias;  /* [N] selection-only bias (sigmoid), or NULL */
  const void* w13;           /* packed gate+up of the N routed experts     */
  const void* w2;            /* packed down of the N routed experts        */
  const void* w13_scale;     /* FP8: f32 [N][2][d_ff/128][d/128] gate, up;
                                MXFP4: packed (which = 2), 16-byte aligned */
  const void* w2_scale;      /* FP8: f32 [N][d/128][d_ff/128];
                                MXFP4: packed (which = 3), 16-byte aligned */
  const void* w13_shared;    /* packed gate+up of the shared expert / NULL */
  const void* w2_shared;     /* packed down of the shared expert / NULL    */
  const void* w13_shared_scale; /* scales of the shared expert / NULL      */
  const void* w2_shared_scale;
} moe_weights_t;

/* Routing results (all device pointers; each may be NULL in
 * moe_layer_forward when the caller does not want it back). */
typedef struct {
  int32_t* topk_idx;   /* [T][k] expert ids, best first                    */
  float* topk_w;       /* [T][k] gates, rows sum to 1                      */
  int32_t* counts;     /* [N] assignments per expert                       */
  int32_t* offsets;    /* [N+1] exclusive prefix sum of counts             */
  int32_t* perm_token; /* [T*k] token of each expert-contiguous row        */
  int32_t* inv_perm;   /* [T][k] row of each (token, slot)                 */
} moe_routing_t;

/* Bytes of one packed buffer for `n_mats` experts: which = 0 -> gate+up
 * (w13), which = 1 -> down (w2); MXFP4 only: which = 2 -> gate+up scales,
 * which = 3 -> down scales.  0 on a bad shape or a which the weight type
 * does not have. */
size_t moe_packed_weight_bytes(const moe_shape_t* s, int which, int n_mats);

/* Repack expert weights from [out][in] row-major into the kernels' layout
 * (run once, not part of the forward).  which = 0: src_a = W_gate
 * [n_mats][d_ff][d], src_b = W_up [n_mats][d_ff][d]; which = 1: src_a =
 * W_down [n_mats][d][d_ff], src_b = NULL.  Elements are of s->w_dtype (FP8:
 * uint8 E4M3 codes; MXFP4: [out][in/2] bytes of two E2M1 codes, input 2j in
 * the low nibble).  MXFP4 scales: which = 2: src_a = [n_mats][2][d_ff][d/32]
 * bytes (gate then up), which = 3: src_a = [n_mats][d][d_ff/32], src_b =
 * NULL; they are regrouped so that the 16 rows of a weight block and four
 * 128-wide K steps are 256 contiguous bytes (rows in order, 16 bytes each,
 * a last partial group padded with zeros) - the streaming kernel then
 * fetches a lane's scales of four steps with one 16-byte load.  Any other
 * weight type returns MOE_ERR_UNSUPPORTED for which 2 and 3.  dst must hold moe_packed_weight_bytes(s, which,
 * n_mats) bytes and must not overlap the sources.  Each expert is a
 * separately addressed block, so an unselected expert's bytes are never
 * read ([MoE-EXP] "Why heads cannot be sparsified the same way"). */
moe_status_t moe_pack_weights(const moe_shape_t* s, int which, int n_mats,
                              const void* src_a, const void* src_b, void* dst,
                              hipStream_t stream);

/* Workspace bytes moe_layer_forward / moe_grouped_ffn / moe_router_topk need
 * for this shape (0 when n_tokens == 0); each of them checks ws_bytes against
 * it.  Returns (size_t)-1 on a bad shape.  Layout (256-byte aligned pieces):
 * router partial logits [S][T][N] f32 (S >= 1 K-splits; with bfloat16 x
 * when N > 8 or T >= 1024 followed, 256-aligned, by the router weight split
 * into three bfloat16 planes, ceil(d/32) * ceil(N/16) * 3 KB), topk idx/w,
 * counts, offsets, perm_token, inv_perm, per-256-token-block expert counts
 * [ceil(T/256)][N] int32, per-16-token-block probability sums
 * [ceil(T/16)][N] f32, a second counts / offsets / perm_token / inv_perm
 * set (capacity-limited routing), an 8 KB tile schedule, H [T*k][d_ff]
 * and H_shared [T][d_ff], Y [T*k][d] and Y_shared [T][d] (H, Y in the
 * activation type).  moe_expert_gate_up / moe_expert_down use only the
 * schedule piece but check ws_bytes against the full size. */
size_t moe_workspace_bytes(const moe_shape_t* s);

/* a1+a2: router logits, selection and gates ([MoE-LLM] "Opening the
 * router"; [CH19] 19.3.2; [AIS-12] worked example).  x: [T][d] act_dtype.
 * Writes topk_idx [T][k] (descending selection score, exact ties to the
 * lower index) and topk_w [T][k].  A NaN selection score (from NaN inputs,
 * weights or offsets) ranks below every other score, -inf included, NaN
 * among themselves by index: every id is in [0, N) and k distinct experts
 * are chosen; a token that has to take a NaN-scored expert gets NaN gates.  Uses w->w_router, w->logit_offset and
 * (sigmoid only) w->select_bias; ws holds the split partial logits (with
 * T <= 64 and N <= 8 logits and selection run in one kernel and ws is not
 * touched). */
moe_status_t moe_router_topk(const moe_shape_t* s, const void* x,
                             const moe_weights_t* w, int32_t* topk_idx,
                             float* topk_w, void* ws, size_t ws_bytes,
                             hipStream_t stream);

/* moe_router_topk with group-limited selection ([MoE-LLM] "Three tricks
 * that tame the all-to-alls": DeepSeek-V3 ranges experts into groups, one
 * per node, and caps how many nodes a token may visit; [AIS-12] "How much
 * traffic is that? A worked example": at most 4 servers).  The experts form
 * n_groups groups of N / n_groups consecutive ids; a group scores as its best
 * expert's selection score (a reading: the pages give no rule), the
 * max_groups best groups are kept (exact ties to the lower group index) and
 * the top-k runs over their experts.  Needs n_groups | N, n_groups <= 64
 * (else MOE_ERR_UNSUPPORTED), 1 <= max_groups <= n_groups and
 * top_k <= max_groups * N / n_groups (else MOE_ERR_INVALID_ARG). */
moe_status_t moe_router_topk_grouped(const moe_shape_t* s, const void* x,
                                     const moe_weights_t* w, int32_t n_groups,
                                     int32_t max_groups, int32_t* topk_idx,
                                     float* topk_w, void* ws, size_t ws_bytes,
                                     hipStream_t stream);

/* a3+a4: per-expert counts, offsets, and the stable expert-contiguous
 * permutation of (token, slot) assignments, ordered by (expert, token, slot)
 * ([CH19] 19.6.3 "Route and pack").  Ids outside [0, N) are not counted and
 * get inv_perm = -1.  If x_perm is not NULL, also gathers x_perm[r] =
 * x[perm_token[r]] ([T*k][d] act_dtype; x is then required).  ws holds
 * per-block counts (moe_workspace_bytes(s) always suffices). */
moe_status_t moe_permute(const moe_shape_t* s, const int32_t* topk_idx,
                         const void* x, moe_routing_t* out, void* x_perm,
                         void* ws, size_t ws_bytes, hipStream_t stream);

/* a3+a4 with a per-expert capacity ([CH19] 19.6.1 "Expert capacity: where
 * do overflow tokens go?"; [AIS-12] "How are experts kept evenly busy?";
 * [MoE-EXP] capacity paragraph): as moe_permute, then each expert keeps only
 * its first `capacity` assignments in token order (then slot order); the
 * rest are dropped and get inv_perm = -1, so moe_combine gives them no
 * contribution (the remaining gates are not renormalised).  counts and
 * offsets describe the kept rows.  The capacity is an integer, normally
 * C = ceil(c * T * k / N) for a capacity factor c; capacity < 0 is
 * MOE_ERR_INVALID_ARG.  x_perm is not offered (moe_grouped_ffn gathers
 * through perm_token).  ws holds the dropless routing. */
moe_status_t moe_permute_capacity(const moe_shape_t* s, const int32_t* topk_idx,
                                  int32_t capacity, moe_routing_t* out, void* ws,
                                  size_t ws_bytes, hipStream_t stream);

/* a5+a6: every routed expert's SwiGLU FFN on its rows, and the shared
 * expert on all T tokens.  Rows of expert e are r in
 * [offsets[e], offsets[e+1]); row r reads x_perm[r] when x_perm is not NULL,
 * else x[perm_token[r]].  Writes y_perm [T*k][d] (row r = FFN_e of its
 * token) and, when n_shared == 1, y_shared [T][d]; both act_dtype.
 * offsets/perm_token are device arrays as written by moe_permute. */
moe_status_t moe_grouped_ffn(const moe_shape_t* s, const void* x,
                             const void* x_perm, const int32_t* perm_token,
                             const int32_t* offsets, const moe_weights_t* w,
                             void* y_perm, void* y_shared, void* ws,
                             size_t ws_bytes, hipStream_t stream);

/* a5 alone: H = silu(X W_gate^T) * (X W_up^T) for every routed expert's rows
 * (the SwiGLU in the GEMM epilogue) and, when n_shared == 1, for all T tokens
 * of the shared expert.  Inputs as in moe_grouped_ffn.  h: [T*k][d_ff],
 * h_shared: [T][d_ff] (act_dtype). */
moe_status_t moe_expert_gate_up(const moe_shape_t* s, const void* x,
                                const void* x_perm, const int32_t* perm_token,
                                const int32_t* offsets, const moe_weights_t* w,
                                void* h, void* h_shared, void* ws,
                                size_t ws_bytes, hipStream_t stream);

/* a6 alone: y = H W_down^T per routed expert's rows (and the shared
 * expert's).  h / h_shared as written by moe_expert_gate_up. */
moe_status_t moe_expert_down(const moe_shape_t* s, const void* h,
                             const void* h_shared, const int32_t* offsets,
                             const moe_weights_t* w, void* y_perm,
                             void* y_shared, void* ws, size_t ws_bytes,
                             hipStream_t stream);

/* a7: out[t] = sum_{i<k} topk_w[t,i] * y_perm[inv_perm[t,i]] (+ y_shared[t])
 * in that fixed order with float32 accumulation and one rounding per output
 * element: deterministic, no atomics ([MoE-LLM] "The MoE change is
 * surprisingly local"; [CH19] 19.3.2).  y_shared may be NULL. */
moe_status_t moe_combine(const moe_shape_t* s, const void* y_perm,
                         const void* y_shared, const int32_t* inv_perm,
                         const float* topk_w, void* out, hipStream_t stream);

/* Load statistics of one routed batch and one step of the selection-bias
 * controller ([CH19] 19.3.3 "Why probability variance alone cannot describe
 * load balancing", 19.3.4; [MoE-LLM] "Classic fix: auxiliary loss",
 * "DeepSeek-style bias controller"; [AIS-12] "How are experts kept evenly
 * busy?").  x: the batch [T][d] act_dtype whose routing produced counts [N]
 * (int32, as written by moe_permute).  The router logits are recomputed
 * from x (w->w_router, w->logit_offset); a token's routing probability p is
 * the softmax of its N logits, or in sigmoid mode sigmoid(s) divided by its
 * sum over all N (the selection bias never enters).  Outputs, each NULL to
 * skip (device float32):
 *   frac[N] = counts[i] / (T*k)                    share f_i
 *   prob[N] = (1/T) * sum_t p[t][i]                 mean probability P_i
 *   aux[1]  = alpha * N * sum_i frac[i] * prob[i]   (Switch used alpha 0.01)
 *   bias[N] += step * sign(T*k - N*counts[i])       in place, float32: +step
 *             below the mean load T*k/N, -step above it, unchanged at it
 *             (the pages' step is 0.001); sigmoid router only, else
 *             MOE_ERR_INVALID_ARG.  The result is the bias for the NEXT
 *             batch; it may be the buffer w->select_bias points to.
 * Sums run in a fixed order (bit-reproducible).  ws: moe_workspace_bytes(s). */
moe_status_t moe_load_stats(const moe_shape_t* s, const void* x, const moe_weights_t* w,
                            const int32_t* counts, float alpha, float step, float* frac,
                            float* prob, float* aux, float* bias, void* ws, size_t ws_bytes,
                            hipStream_t stream);

/* The whole layer forward: router, permute, grouped FFN, combine.  x and
 * out: [T][d] act_dtype (must not overlap).  routing_out may be NULL, and
 * any of its members may be NULL.  ws: moe_workspace_bytes(s) bytes. */
moe_status_t moe_layer_forward(const moe_shape_t* s, const moe_weights_t* w,
                               const void* x, void* out,
                               moe_routing_t* routing_out, void* ws,
                               size_t ws_bytes, hipStream_t stream);

/* moe_layer_forward followed by the load statistics of the batch it routed
 * and one selection-bias step, as moe_load_stats computes them (the same
 * kernels, so the same bits), without recomputing the router logits: the
 * statistics read the logit partials the router left in the workspace and
 * the counts of this call's permute (the logits are recomputed only where
 * logits and selection ran in one kernel: T <= 64 and N <= 8).  The
 * selection uses w->select_bias as it was before the call; `bias` (may be
 * that same buffer) receives the step afterwards, for the next batch.
 * Outputs and errors as moe_layer_forward and moe_load_stats ([CH19] 19.3.3,
 * 19.3.4; [MoE-LLM] "Classic fix: auxiliary loss", "DeepSeek-style bias
 * controller"; [AIS-12] "How are experts kept evenly busy?"). */
moe_status_t moe_layer_forward_stats(const moe_shape_t* s, const moe_weights_t* w,
                                     const void* x, void* out, moe_routing_t* routing_out,
                                     float alpha, float step, float* frac, float* prob,
                                     float* aux, float* bias, void* ws, size_t ws_bytes,
                                     hipStream_t stream);

/* moe_layer_forward with capacity-limited dispatch (see
 * moe_permute_capacity): experts run only on their kept rows and dropped
 * branches contribute nothing.  routing_out, when given, receives the
 * capped routing.  capacity >= T*k is the dropless layer. */
moe_status_t moe_layer_forward_capacity(const moe_shape_t* s, const moe_weights_t* w,
                                        const void* x, void* out, int32_t capacity,
                                        moe_routing_t* routing_out, void* ws,
                                        size_t ws_bytes, hipStream_t stream);

/* moe_layer_forward with group-limited selection (see
 * moe_router_topk_grouped).  n_groups = max_groups gives moe_layer_forward. */
moe_status_t moe_layer_forward_grouped(const moe_shape_t* s, const moe_weights_t* w,
                                       const void* x, void* out, int32_t n_groups,
                                       int32_t max_groups, moe_routing_t* routing_out,
                                       void* ws, size_t ws_bytes, hipStream_t stream);

/* Bytes of the static device scratch behind moe_layer_forward_noalloc. */
#define MOE_NOALLOC_SCRATCH_BYTES (64u << 20)

/* moe_layer_forward for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same kernels and results, with the scratch space taken
 * from a static device array of MOE_NOALLOC_SCRATCH_BYTES (64 MiB) per GPU
 * instead of a caller workspace.  No allocation of any kind.  The shape's
 * moe_workspace_bytes() must not exceed that size (decode batches do: the
 * Mixtral 8x7B shape up to about 900 tokens, the DeepSeek-V3 shape up to 256
 * tokens), else MOE_ERR_UNSUPPORTED before any HIP call.  The array's device
 * address is looked up on the first call on each device (the caller's
 * current device).  All calls on one GPU share its array: calls that
 * overlap in time on one GPU (several streams or host threads) race and
 * must be serialised by the caller. */
moe_status_t moe_layer_forward_noalloc(const moe_shape_t* s, const moe_weights_t* w,
                                       const void* x, void* out,
                                       moe_routing_t* routing_out, hipStream_t stream);

/* Static description of a status code. */
const char* moe_status_string(moe_status_t st);

/* Message of the last MOE_ERR_HIP / argument error on this host thread. */
const char* moe_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* MOE_FFN_H */
