/*
 * libmoe -- forward pass of one Mixture-of-Experts FFN layer on an AMD MI355X
 * (gfx950), and the backward of its routed experts, as hand-written HIP
 * kernels behind a plain C ABI.
 *
 * The layer (PLENA_Compiler PR #69 and PLENA_Simulator PR #97, sections
 * "Group C -- shared experts" / "Part 2 -- Shared experts"):
 *
 *     y = shared(x) + sum_k route_weight_k * routed_expert_k(x)
 *
 * computed by six calls, normally in this order on one stream:
 *
 *     moe_route -> moe_build_scatter -> moe_grouped_swiglu_fc1 -> moe_grouped_fc2
 *               -> moe_gather_combine(accumulate=0) -> moe_shared_expert(accumulate=1)
 *
 * (the shared branch may instead run first, with accumulate=0, and the combine
 * after it with accumulate=1).
 *
 * Conventions for every call:
 *  - Every tensor pointer is a DEVICE pointer to a contiguous row-major buffer
 *    that the caller allocated and owns; the library never allocates, frees,
 *    or synchronises.  Calls enqueue kernels on `stream` (a hipStream_t; NULL
 *    is the default stream) and return; results are valid once the caller
 *    has synchronised that stream.
 *  - `dt` is the element type of x, the weights, the scattered rows and the
 *    SwiGLU activation (MOE_F32 or MOE_BF16).  Logits, route weights, the
 *    per-row expert outputs Y_s and the layer output y are always float32.
 *  - All shape arguments are explicit; there are no global modes.  Arguments
 *    are validated on the host before anything is launched: an invalid call
 *    returns a non-zero status, launches nothing, and moe_last_error() names
 *    the offending argument.
 *  - Sizes: T tokens, H hidden, E routed experts, top_k slots per token,
 *    R = T * top_k scattered rows, I routed intermediate size, I_s shared
 *    intermediate size.
 *  - Limits (MOE_ERR_UNSUPPORTED beyond them): E <= 1024, top_k <= 32,
 *    H, I, I_s multiples of 8, T * top_k < 2^31 / 8.
 */
#ifndef LIBMOE_H
#define LIBMOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum moe_status {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARGUMENT = 1, /* null pointer, size < 1, top_k > E, half-specified shared branch */
  MOE_ERR_UNSUPPORTED = 2,      /* legal but beyond the implemented limits above */
  MOE_ERR_WORKSPACE = 3,        /* workspace missing or smaller than the *_workspace_bytes query */
  MOE_ERR_HIP = 4               /* a HIP runtime call or kernel launch failed */
} moe_status;

/* The *_RANGE_ markers of the enums below name no value a call accepts: they
 * make each enum as wide as int32_t, so that whatever int32_t a caller passes
 * is a representable value that validation then rejects (in C++ an enum
 * holding a value outside its enumerators' range is undefined). */
typedef enum moe_dtype {
  MOE_F32 = 0,
  MOE_BF16 = 1,
  MOE_DTYPE_RANGE_MIN = -0x7fffffff - 1,
  MOE_DTYPE_RANGE_MAX = 0x7fffffff
} moe_dtype;

/* Tile configuration of a grouped-GEMM launch, as moe_grouped_gemm_tile reports it. */
typedef enum moe_tile_config {
  MOE_TILE_F32 = 0,       /* float32 path: one thread per output element */
  MOE_TILE_GENERIC = 1,   /* bf16 with a reduction size not a multiple of 64: register-staged 128 x 128 tiles */
  MOE_TILE_128x128 = 2,   /* pipelined: 128 rows x 128 staged weight columns x 64-deep slices, 4 waves */
  MOE_TILE_256x256 = 3,   /* pipelined: 256 x 256 x 64, 8 waves (groups of >= 512 rows on average) */
  MOE_TILE_128x256 = 4,   /* pipelined: 128 x 256 x 32, 8 waves, two workgroups per CU (193..511 rows) */
  MOE_TILE_32x128 = 5,    /* pipelined: 32 x 128 x 64 with split-K waves (groups of <= 32 rows on average) */
  MOE_TILE_128x512 = 6,   /* pipelined: 128 x 512 x 32, 3-stage ring, 8 waves (weight-streaming groups, <= 192 rows) */
  MOE_TILE_32x64 = 7      /* pipelined: 32 x 64 x 64 with split-K waves, two workgroups per CU (fc2 at decode sizes whose
                             32 x 128 tiles would leave CUs idle) */
} moe_tile_config;

/* Stage of a call, in the stage vocabulary of the PLENA pages (PLENA_Compiler
 * PR #69, sections "Group B" and "Group E": router_topk, expert_route_weight,
 * accumulator_init, residual_setup, gather, scatter_combine, expert_projection,
 * expert_bias, shared_expert_projection / _activation / _gate, other).  Every
 * call below opens a roctx range with this name for the duration of the call
 * (seen by `rocprofv3 --marker-trace`); '+' joins the stages of a call that
 * serves several, and backward calls carry the prefix "backward:".  `call` is
 * the function name; `gated` selects the label of the calls whose stages
 * depend on w_gate being given.  Returns "other" for unknown names; the string
 * is static. */
const char* moe_call_stage(const char* call, int32_t gated);

/* Storage of an expert weight W that maps K inputs to N outputs (the layer
 * computes x @ W with W a K x N matrix in the pages' notation):
 *   MOE_W_KN: row-major [K, N], N contiguous (the pages' x @ W form);
 *   MOE_W_NK: row-major [N, K], K contiguous (the layout of a torch.nn.Linear
 *             weight; both MFMA operands are then K-contiguous, so weight
 *             tiles are read from LDS like activation tiles).
 * The values are the same matrix either way; results are identical up to
 * the fp32 accumulation order within a tile. */
typedef enum moe_weight_layout {
  MOE_W_KN = 0,
  MOE_W_NK = 1,
  MOE_W_RANGE_MIN = -0x7fffffff - 1,
  MOE_W_RANGE_MAX = 0x7fffffff
} moe_weight_layout;

/* Name of a status code ("MOE_OK", ...).  Never NULL. */
const char* moe_status_name(int status);

/* Message for the last non-OK status returned on the calling thread
 * (thread-local; "" if none).  Names the offending argument. */
const char* moe_last_error(void);

/* Library version as MAJOR*10000 + MINOR*100 + PATCH. */
int moe_version(void);

/*
 * moe_route -- router GEMM and top-k softmax.
 *
 * Source: PLENA_Compiler PR #69 section "Group E" (the router GEMM) and
 * PLENA_Simulator PR #97 section "C_SET_TOPK_REG" (topk_softmax, generic in
 * the expert count and k; k must be positive).
 *
 *   logits[t, e]   = sum_h x[t, h] * w_router[h, e]  (+ logit_bias[e])      fp32
 *   topk_ids[t, :] = the top_k experts with the largest logits, in slot order:
 *                    descending logit, ties to the lower expert index; NaN
 *                    logits rank below every number
 *   topk_weights   = softmax over the top_k selected logits (sums to 1)
 *
 * x [T, H] (dt), w_router [H, E] (dt), logit_bias [E] fp32 or NULL for none,
 * topk_ids [T, top_k] int32 out, topk_weights [T, top_k] fp32 out,
 * logits [T, E] fp32 out (required): the logits exactly as top-k saw them.
 * workspace: device scratch of at least moe_route_workspace_bytes(dt, T, H, E)
 * bytes (it receives partial sums over slices of H and, for an odd E, a copy
 * of the router weight with a zero column appended; may be NULL when that size
 * is 0), contents undefined on entry and exit.
 */
moe_status moe_route(moe_dtype dt, const void* x, const void* w_router, const float* logit_bias,
                     int32_t T, int32_t H, int32_t E, int32_t top_k,
                     int32_t* topk_ids, float* topk_weights, float* logits,
                     void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes moe_route needs for (dt, T, H, E). */
size_t moe_route_workspace_bytes(moe_dtype dt, int32_t T, int32_t H, int32_t E);

/* Workspace bytes moe_build_scatter needs for (T, top_k, E). */
size_t moe_build_scatter_workspace_bytes(int32_t T, int32_t top_k, int32_t E);

/*
 * moe_build_scatter -- expert-grouped row layout and the scattered rows.
 *
 * Source: VeOmni docs "Fused MoE Kernel Notes", sections "Scatter/gather
 * layout" (tokens [T, H] expand to [T*top_k, H] rows grouped by expert;
 * scatter_index maps (token, slot) to its row) and "Duplicate top-k routes"
 * (several slots of one token may name one expert, so a group can exceed T).
 *
 * Pairs p = t*top_k + j are laid out by a stable counting sort: group e holds
 * rows [expert_offsets[e], expert_offsets[e+1]) in increasing p.
 *
 * topk_ids [T, top_k] int32 in (from moe_route or fed in; duplicates allowed);
 * x [T, H] (dt) in.  Outputs: scatter_index [T, top_k] int32 (row of pair
 * (t, j), or -1 when its expert id is outside [0, E)); row_token [R] int32
 * (token of each row; -1 for rows past expert_offsets[E]); expert_offsets
 * [E+1] int32; status_words [2] int32 = {largest group size, number of
 * out-of-range expert ids} -- a non-zero second word means the routes were
 * invalid and those pairs were dropped; x_scattered [R, H] (dt):
 * x_scattered[r] = x[row_token[r]] for r < expert_offsets[E], other rows
 * untouched.  x_scattered may be NULL: the rows are then not copied, and the
 * *_gather fc1 calls below read them from x through row_token on load (the
 * same values, without writing and re-reading R*H elements).  The same holds
 * for moe_route_and_scatter.  workspace: device scratch of at least
 * moe_build_scatter_workspace_bytes(T, top_k, E) bytes, contents undefined
 * on entry and exit.
 */
moe_status moe_build_scatter(moe_dtype dt, const void* x, const int32_t* topk_ids,
                             int32_t T, int32_t H, int32_t E, int32_t top_k,
                             int32_t* scatter_index, int32_t* row_token, int32_t* expert_offsets,
                             int32_t* status_words, void* x_scattered,
                             void* workspace, size_t workspace_bytes, void* stream);

/*
 * moe_route_and_scatter -- moe_route followed by moe_build_scatter on its
 * topk_ids, in one call.
 *
 * Sources: those of moe_route and moe_build_scatter above.  Every output is
 * the one the two calls produce (same bits), so the same arguments carry the
 * same meaning, layout and ownership; logits is required as in moe_route.
 * For few tokens (bf16, T <= 16, E a multiple of 8) the top-k and the whole
 * scatter build, including the row copy when the rows are few, run in one
 * workgroup after the router product, which saves kernel launches at decode;
 * otherwise the call runs the two calls' kernels back to back.
 * workspace: device scratch of at least
 * moe_route_and_scatter_workspace_bytes(dt, T, H, E, top_k) bytes, contents
 * undefined on entry and exit.  Errors: those of both calls.
 */
moe_status moe_route_and_scatter(moe_dtype dt, const void* x, const void* w_router, const float* logit_bias,
                                 int32_t T, int32_t H, int32_t E, int32_t top_k,
                                 int32_t* topk_ids, float* topk_weights, float* logits,
                                 int32_t* scatter_index, int32_t* row_token, int32_t* expert_offsets,
                                 int32_t* status_words, void* x_scattered,
                                 void* workspace, size_t workspace_bytes, void* stream);

/*
 * moe_grouped_gemm_tile -- which tile configuration (moe_tile_config) the routed
 * experts' launch of a grouped-GEMM call takes for these sizes on the current
 * device.  Host-only: launches nothing, reads the device's CU count.
 *
 * Source: VeOmni docs "Fused MoE Kernel Notes", section "Backward grouped-GEMM
 * launch bound" (the launch is shaped from the sizes; the tile walk itself comes
 * from expert_offsets on the device); PLENA_Simulator PR #97, section "Tests"
 * (a test asserts which encoding a policy took, not only its result).
 * call: 0 = fc1 (moe_grouped_swiglu_fc1 and its _gather / _and_shared variants),
 * 1 = fc2.  R, H, E, I as in those calls; T and I_s > 0 ask about the
 * *_and_shared call (routed and shared experts may then share one launch),
 * I_s = 0 about the plain call.  Returns -1 for invalid arguments.
 */
int32_t moe_grouped_gemm_tile(moe_dtype dt, int32_t call, int32_t R, int32_t H, int32_t E, int32_t I, int32_t T,
                              int32_t I_s);

/* Workspace bytes moe_route_and_scatter needs for (dt, T, H, E, top_k); 0 for invalid sizes. */
size_t moe_route_and_scatter_workspace_bytes(moe_dtype dt, int32_t T, int32_t H, int32_t E, int32_t top_k);

/*
 * moe_route_and_scatter_noalloc -- moe_route_and_scatter without a workspace
 * argument and without any allocation, for callers that cannot allocate device
 * memory during the call: code being captured into a HIP graph, tight decode
 * or serving loops, and harnesses that forbid hipMalloc.
 *
 * Same arguments (minus workspace), outputs (same bits), layouts, ownership and
 * errors as moe_route_and_scatter.  The scratch the kernels need lives in a
 * device array of the library, moe_route_and_scatter_noalloc_max_bytes() bytes
 * (64 MiB) on every GPU the library runs on, allocated when the library's code
 * loads on that GPU and held until the process ends; the call itself allocates
 * nothing.  Sizes whose moe_route_and_scatter_workspace_bytes exceeds that
 * return MOE_ERR_UNSUPPORTED before anything is launched.  Nothing in the
 * scratch needs to start at zero.  Every call on one GPU shares that GPU's
 * array: two calls that may run at the same time on one GPU (on different
 * streams, or from different threads without ordering) race and must not be
 * issued.
 */
moe_status moe_route_and_scatter_noalloc(moe_dtype dt, const void* x, const void* w_router, const float* logit_bias,
                                         int32_t T, int32_t H, int32_t E, int32_t top_k,
                                         int32_t* topk_ids, float* topk_weights, float* logits,
                                         int32_t* scatter_index, int32_t* row_token, int32_t* expert_offsets,
                                         int32_t* status_words, void* x_scattered, void* stream);

/* Bytes of device scratch moe_route_and_scatter_noalloc holds per GPU (its size limit). */
size_t moe_route_and_scatter_noalloc_max_bytes(void);

/*
 * moe_grouped_swiglu_fc1 -- per-expert gate/up projection and SwiGLU.
 *
 * Source: VeOmni docs "Fused MoE Kernel Notes", section "Backward grouped-GEMM
 * launch bound" (a same-N/K grouped GEMM whose launch must cover the largest
 * group, never just the token count); PLENA_Compiler PR #69 section "Group C"
 * and PLENA_Simulator PR #97 section "Tests" (SwiGLU = silu(gate) * up).
 *
 * For every expert e and row r of its group:
 *   g = x_scattered[r] @ w1[e][:, 0:I],  u = x_scattered[r] @ w1[e][:, I:2I]
 *   act[r] = silu(g) * u,  silu(g) = g / (1 + exp(-g))   (fp32, stored as dt;
 *            bf16 is round-to-nearest-even)
 * The tile walk is derived on the device from expert_offsets, so every row of
 * every group is computed whatever the group sizes are (a group may hold up to
 * R rows); empty experts read no weights.
 *
 * x_scattered [R, H] (dt), expert_offsets [E+1] int32 (device),
 * w1 (dt): wl = MOE_W_KN: [E, H, 2I] (per expert [H, 2I], gate columns
 * first); wl = MOE_W_NK: [E, 2I, H] (per expert [2I, H], gate rows first),
 * act [R, I] (dt) out; rows past expert_offsets[E] are not written.
 */
moe_status moe_grouped_swiglu_fc1(moe_dtype dt, moe_weight_layout wl, const void* x_scattered,
                                  const int32_t* expert_offsets, const void* w1, int32_t R, int32_t H,
                                  int32_t E, int32_t I, void* act, void* stream);

/*
 * moe_grouped_fc2 -- per-expert down projection.
 *
 * Source: VeOmni docs "Fused MoE Kernel Notes", sections "Scatter/gather
 * layout" and "Backward grouped-GEMM launch bound".
 *
 *   y_rows[r] = act[r] @ w2[e]   for r in group e, accumulated and stored fp32
 *
 * act [R, I] (dt), expert_offsets [E+1] int32, w2 (dt): [E, I, H] for
 * MOE_W_KN, [E, H, I] for MOE_W_NK, y_rows [R, H] fp32 out; rows past
 * expert_offsets[E] are not written.
 */
moe_status moe_grouped_fc2(moe_dtype dt, moe_weight_layout wl, const void* act, const int32_t* expert_offsets,
                           const void* w2, int32_t R, int32_t I, int32_t E, int32_t H,
                           float* y_rows, void* stream);

/*
 * moe_gather_combine -- weighted gather of the routed outputs back to tokens.
 *
 * Source: VeOmni docs "Fused MoE Kernel Notes", section "Scatter/gather
 * layout" (moe_gather sums routed outputs back to [tokens, hidden]); the
 * hf-adapters PR #2 commit on the loop-on-topk decode combine (a per-token
 * reduction over the k slots, free of the read-modify-write hazard that
 * duplicate indices cause).
 *
 *   y[t] = (accumulate ? y[t] : 0) + sum_{j ascending} topk_weights[t, j] * y_rows[scatter_index[t, j]]
 *
 * Slots with scatter_index -1 add nothing.  y_rows [R, H] fp32,
 * scatter_index [T, top_k] int32, topk_weights [T, top_k] fp32,
 * y [T, H] fp32 in/out.  Each output element is written by exactly one thread.
 */
moe_status moe_gather_combine(const float* y_rows, const int32_t* scatter_index, const float* topk_weights,
                              int32_t T, int32_t H, int32_t top_k, int32_t accumulate, float* y,
                              void* stream);

/* Workspace bytes moe_shared_expert needs (the [T, I_s] activation and the
 * per-token gate). */
size_t moe_shared_expert_workspace_bytes(moe_dtype dt, int32_t T, int32_t I_s);

/*
 * moe_shared_expert -- the shared expert, optionally sigmoid-gated.
 *
 * Source: PLENA_Compiler PR #69 section "Group C -- shared experts" (a dense
 * FFN over every token, added unweighted; Qwen2-MoE scales it by
 * sigmoid(x @ w_gate), one scalar per token; DeepSeek's n shared experts are
 * one fused MLP of width moe_inter * n_shared).
 *
 *   a  = silu(x @ ws1[:, 0:I_s]) * (x @ ws1[:, I_s:2I_s])   (stored as dt)
 *   ys = a @ ws2;   if w_gate: ys[t] *= 1 / (1 + exp(-(x[t] . w_gate)))
 *   y  = (accumulate ? y : 0) + ys                           (fp32)
 *
 * x [T, H] (dt), ws1 (dt) [H, 2 I_s] (MOE_W_KN) or [2 I_s, H] (MOE_W_NK),
 * ws2 (dt) [I_s, H] or [H, I_s], w_gate [H] (dt) or NULL for the ungated
 * variant, y [T, H] fp32 in/out, workspace of at least
 * moe_shared_expert_workspace_bytes(dt, T, I_s) bytes.
 */
moe_status moe_shared_expert(moe_dtype dt, moe_weight_layout wl, const void* x, const void* ws1, const void* ws2,
                             const void* w_gate, int32_t T, int32_t H, int32_t I_s,
                             int32_t accumulate, float* y, void* workspace, size_t workspace_bytes,
                             void* stream);

/*
 * moe_grouped_swiglu_fc1_and_shared / moe_grouped_fc2_and_shared -- the routed
 * expert FFNs and the shared expert computed together, one launch per half.
 *
 * Source: as for moe_grouped_swiglu_fc1, moe_grouped_fc2 and moe_shared_expert
 * (VeOmni docs "Fused MoE Kernel Notes", "Backward grouped-GEMM launch bound";
 * PLENA_Compiler PR #69, "Group C -- shared experts").  Routed groups stream
 * expert weights that are read once, while the shared expert reuses one weight
 * across all T tokens; interleaving both kinds of tiles in one persistent
 * launch lets them overlap on every CU.
 *
 * fc1 half:  act        [R, I]   = SwiGLU of the routed rows (as moe_grouped_swiglu_fc1)
 *            act_shared [T, I_s] = SwiGLU(x @ ws1)            (dt, caller buffer)
 * fc2 half:  y_rows     [R, H]   = routed expert outputs, fp32 (as moe_grouped_fc2)
 *            y          [T, H]   = (accumulate ? y : 0) + gate * (act_shared @ ws2), fp32,
 *                                  gate = sigmoid(x . w_gate) per token, or 1 when w_gate is NULL
 * The routed outputs are then added with moe_gather_combine(accumulate = 1).
 * moe_grouped_fc2_and_shared needs a workspace of at least
 * moe_shared_expert_workspace_bytes(dt, T, I_s) bytes (it holds the gate).
 * Other arguments (wl covers w1/w2 and ws1/ws2 alike) are those of the
 * three separate calls.  Each call chooses
 * from the shapes whether its two computations share one launch (bf16, H, I
 * and I_s multiples of 64, and a shared expert whose FLOPs are small next to
 * the routed weight bytes) or run one after the other; results are the same
 * either way.
 */
/*
 * MXFP8 expert weights: moe_grouped_swiglu_fc1_mx8, moe_grouped_fc2_mx8,
 * moe_shared_expert_mx8.
 *
 * Source: PLENA_Compiler PR #69, section "Group C -- shared experts" (the
 * fusion-identity paragraph: expert weights are MXFP8 -- e4m3 values, one e8m0
 * scale per block of 8 along the intermediate axis).  Encodings (the OCP
 * microscaling definitions): e4m3 = sign, 4-bit exponent (bias 7, subnormals at
 * 0), 3-bit mantissa, no infinities, 0x7F/0xFF NaN; e8m0 = 2^(byte - 127), 0xFF
 * NaN.  A weight element is e4m3(code) * e8m0(scale of its block).
 *
 * Each call computes exactly what its bf16 counterpart computes on the
 * dequantized weights (activations, act and the outputs keep their bf16/fp32
 * types; dt is implicitly MOE_BF16).  Codes are stored [N, K] per matrix (K
 * contiguous, one byte each), the layout of MOE_W_NK:
 *   fc1:    w1q [E, 2I, H], scales w1s [E, 2I/8, H] (blocks of 8 along the
 *           intermediate axis 2I: scale w1s[e][n/8][k] for code w1q[e][n][k]);
 *   fc2:    w2q [E, H, I],  scales w2s [E, H, I/8]  (blocks along I:
 *           w2s[e][n][k/8] for w2q[e][n][k]);
 *   shared: ws1q [2I_s, H] / ws1s [2I_s/8, H] and ws2q [H, I_s] / ws2s [H, I_s/8].
 * The weights are dequantized to bf16 inside the kernels; this is exact while
 * every scale exponent lies in 10..246 (the products stay normal bf16 numbers).
 * Limits: the reduction size of each product (H for fc1 and the shared fc1, I
 * for fc2, I_s for the shared fc2) must be a multiple of 128
 * (MOE_ERR_UNSUPPORTED otherwise).  Other arguments, ownership and errors are
 * those of the bf16 calls.
 */
moe_status moe_grouped_swiglu_fc1_mx8(const void* x_scattered, const int32_t* expert_offsets, const uint8_t* w1q,
                                      const uint8_t* w1s, int32_t R, int32_t H, int32_t E, int32_t I, void* act,
                                      void* stream);
moe_status moe_grouped_fc2_mx8(const void* act, const int32_t* expert_offsets, const uint8_t* w2q,
                               const uint8_t* w2s, int32_t R, int32_t I, int32_t E, int32_t H, float* y_rows,
                               void* stream);
moe_status moe_shared_expert_mx8(const void* x, const uint8_t* ws1q, const uint8_t* ws1s, const uint8_t* ws2q,
                                 const uint8_t* ws2s, const void* w_gate, int32_t T, int32_t H, int32_t I_s,
                                 int32_t accumulate, float* y, void* workspace, size_t workspace_bytes,
                                 void* stream);

/* MXFP8 counterparts of moe_grouped_swiglu_fc1_and_shared and
 * moe_grouped_fc2_and_shared: the routed groups and the shared expert in one
 * launch per half (always), weights and scales as for the *_mx8 calls above,
 * other arguments as for the bf16 calls.  Limits: H, I and I_s multiples of
 * 128. */
moe_status moe_grouped_swiglu_fc1_and_shared_mx8(const void* x_scattered, const int32_t* expert_offsets,
                                                 const uint8_t* w1q, const uint8_t* w1s, int32_t R, int32_t H,
                                                 int32_t E, int32_t I, void* act, const void* x, const uint8_t* ws1q,
                                                 const uint8_t* ws1s, int32_t T, int32_t I_s, void* act_shared,
                                                 void* stream);
moe_status moe_grouped_fc2_and_shared_mx8(const void* act, const int32_t* expert_offsets, const uint8_t* w2q,
                                          const uint8_t* w2s, int32_t R, int32_t I, int32_t E, int32_t H,
                                          float* y_rows, const void* act_shared, const uint8_t* ws2q,
                                          const uint8_t* ws2s, const void* x, const void* w_gate, int32_t T,
                                          int32_t I_s, int32_t accumulate, float* y, void* workspace,
                                          size_t workspace_bytes, void* stream);

/* Kernel launches one moe_grouped_swiglu_fc1_and_shared call makes for these
 * sizes (R = T * top_k routed rows): 1 when the routed experts and the shared
 * expert share one launch, 2 when they run one after the other; 0 for invalid
 * sizes.  moe_grouped_fc2_and_shared makes the same choice (plus one small
 * gate launch when w_gate is given).  For profiling and reporting only. */
int32_t moe_and_shared_launches(moe_dtype dt, int32_t R, int32_t H, int32_t E, int32_t I, int32_t T, int32_t I_s);

moe_status moe_grouped_swiglu_fc1_and_shared(moe_dtype dt, moe_weight_layout wl, const void* x_scattered,
                                             const int32_t* expert_offsets, const void* w1, int32_t R, int32_t H,
                                             int32_t E, int32_t I, void* act, const void* x, const void* ws1,
                                             int32_t T, int32_t I_s, void* act_shared, void* stream);

moe_status moe_grouped_fc2_and_shared(moe_dtype dt, moe_weight_layout wl, const void* act,
                                      const int32_t* expert_offsets, const void* w2, int32_t R, int32_t I, int32_t E,
                                      int32_t H, float* y_rows, const void* act_shared, const void* ws2,
                                      const void* x, const void* w_gate, int32_t T, int32_t I_s, int32_t accumulate,
                                      float* y, void* workspace, size_t workspace_bytes, void* stream);

/*
 * moe_grouped_swiglu_fc1_gather / moe_grouped_swiglu_fc1_and_shared_gather --
 * moe_grouped_swiglu_fc1 / moe_grouped_swiglu_fc1_and_shared with the routed
 * rows gathered from x on load instead of read from x_scattered.
 *
 * Source: as for moe_grouped_swiglu_fc1 (VeOmni docs "Fused MoE Kernel Notes",
 * section "Scatter/gather layout": row r of the expert-grouped layout is token
 * row_token[r]).  Row r of the product is x[row_token[r]] -- exactly the row
 * moe_build_scatter would have copied to x_scattered[r] -- so act (and
 * act_shared) are bit-identical to the non-gather calls.  x [T, H] (dt) in;
 * row_token [R] int32 in, from moe_build_scatter or moe_route_and_scatter for
 * the same routes (values are clamped to [0, T) on the device; only rows
 * r < expert_offsets[E] are read).  Every other argument, the layouts, the
 * ownership and the errors are those of the non-gather calls; additionally T
 * must be >= 1.  bf16 and fp32; MXFP8 weights have no gather variant.
 */
moe_status moe_grouped_swiglu_fc1_gather(moe_dtype dt, moe_weight_layout wl, const void* x, const int32_t* row_token,
                                         const int32_t* expert_offsets, const void* w1, int32_t T, int32_t R,
                                         int32_t H, int32_t E, int32_t I, void* act, void* stream);
moe_status moe_grouped_swiglu_fc1_and_shared_gather(moe_dtype dt, moe_weight_layout wl, const void* x,
                                                    const int32_t* row_token, const int32_t* expert_offsets,
                                                    const void* w1, int32_t R, int32_t H, int32_t E, int32_t I,
                                                    void* act, const void* ws1, int32_t T, int32_t I_s,
                                                    void* act_shared, void* stream);

/*
 * Backward of the routed experts, routes held fixed:
 *
 *   forward (training):  moe_build_scatter -> moe_grouped_swiglu_fc1_save -> moe_grouped_fc2
 *                        -> moe_gather_combine
 *   backward:            moe_scatter_grad -> moe_grouped_fc2_backward -> moe_grouped_fc1_backward
 *
 * Source: VeOmni docs "Fused MoE Kernel Notes", sections "Backward grouped-GEMM
 * launch bound" (the fc2 output gradient is moe_scatter of the output gradient
 * through scatter_index; the input-gradient GEMMs are same-N/K grouped GEMMs
 * that must cover the largest group, and the weight-gradient GEMMs are
 * same-M/N grouped GEMMs whose reduction runs over a group's rows), "Duplicate
 * top-k routes" and "Regression test pattern" (every gradient finite when all
 * slots of every token name one expert).  The formulas are the chain rule of
 * the forward calls above.  Every bound comes from the realized
 * expert_offsets, so a group of any size up to R rows is covered.  Precision:
 * fp32 accumulation; h_pre, act, d_rows, d_h, d_w1 and d_w2 are stored as dt
 * (bf16 round-to-nearest-even); d_x and d_topk_weights are fp32.
 */

/* moe_grouped_swiglu_fc1_save -- moe_grouped_swiglu_fc1 that also stores the
 * pre-activation for the backward: h_pre[r] = [g | u] (gate columns [0, I),
 * up columns [I, 2I)), h_pre [R, 2I] (dt) out.  act is computed from the
 * unrounded g and u exactly as in moe_grouped_swiglu_fc1.  Other arguments as
 * for moe_grouped_swiglu_fc1. */
moe_status moe_grouped_swiglu_fc1_save(moe_dtype dt, moe_weight_layout wl, const void* x_scattered,
                                       const int32_t* expert_offsets, const void* w1, int32_t R, int32_t H,
                                       int32_t E, int32_t I, void* act, void* h_pre, void* stream);

/*
 * moe_scatter_grad -- output gradient into the expert-grouped rows, and the
 * route weights' gradient (the adjoint of moe_gather_combine).
 *
 * For every pair (t, j) with r = scatter_index[t, j] in [0, R):
 *   d_rows[r]         = topk_weights[t, j] * dy[t]   (product in fp32, stored as dt)
 *   d_topk_weights[t, j] = dy[t] . y_rows[r]          (fp32, fixed summation order)
 * Pairs with any other index get d_topk_weights 0 and write no row; rows that
 * no pair names are not written.
 *
 * dy [T, H] fp32 (gradient of the layer output y), y_rows [R, H] fp32 (the
 * moe_grouped_fc2 output of the forward), topk_weights and scatter_index
 * [T, top_k], d_rows [R, H] (dt) out, d_topk_weights [T, top_k] fp32 out.
 */
moe_status moe_scatter_grad(moe_dtype dt, const float* dy, const float* y_rows, const float* topk_weights,
                            const int32_t* scatter_index, int32_t T, int32_t H, int32_t top_k, int32_t R,
                            void* d_rows, float* d_topk_weights, void* stream);

/*
 * moe_grouped_fc2_backward -- gradients through the down projection and SwiGLU.
 *
 * For every expert e and row r of its group, with da = d_rows[r] @ w2[e]^T:
 *   d_h[r][i]     = da[i] * u * s * (1 + g * (1 - s))   (gate half; g = h_pre[r][i],
 *   d_h[r][I + i] = da[i] * g * s                        u = h_pre[r][I + i], s = sigmoid(g))
 *   d_w2[e]       = act[group e]^T @ d_rows[group e]     (zero for an empty expert)
 * d_rows [R, H] (dt), act [R, I] (dt) and h_pre [R, 2I] (dt) from the forward,
 * expert_offsets [E+1], w2 (dt) in layout wl, d_h [R, 2I] (dt) out, d_w2 (dt)
 * out in the layout of w2 ([E, I, H] for MOE_W_KN, [E, H, I] for MOE_W_NK).
 * Two launches: the input gradient (a same-N/K grouped GEMM, SwiGLU'
 * in its epilogue) and the weight gradient (same-M/N).
 */
moe_status moe_grouped_fc2_backward(moe_dtype dt, moe_weight_layout wl, const void* d_rows, const void* act,
                                    const void* h_pre, const int32_t* expert_offsets, const void* w2, int32_t R,
                                    int32_t I, int32_t E, int32_t H, void* d_h, void* d_w2, void* stream);

/* Workspace bytes moe_grouped_fc1_backward needs (the fp32 [R, H] input
 * gradient of the scattered rows); 0 for invalid sizes. */
size_t moe_grouped_fc1_backward_workspace_bytes(int32_t R, int32_t H);

/*
 * moe_grouped_fc1_backward -- gradients through the gate/up projection, and
 * the input gradient gathered back to tokens.
 *
 *   d_xs[r]  = d_h[r] @ w1[e]^T                    (fp32, in the workspace)
 *   d_x[t]   = (accumulate ? d_x[t] : 0) + sum_{j ascending} d_xs[scatter_index[t, j]]
 *   d_w1[e]  = x_scattered[group e]^T @ d_h[group e]   (zero for an empty expert)
 * d_h [R, 2I] (dt), x_scattered [R, H] (dt), expert_offsets [E+1], w1 (dt) in
 * layout wl, scatter_index [T, top_k], d_x [T, H] fp32 in/out, d_w1 (dt) out in
 * the layout of w1 ([E, H, 2I] for MOE_W_KN, [E, 2I, H] for MOE_W_NK),
 * workspace of at least moe_grouped_fc1_backward_workspace_bytes(R, H) bytes.
 */
moe_status moe_grouped_fc1_backward(moe_dtype dt, moe_weight_layout wl, const void* d_h, const void* x_scattered,
                                    const int32_t* expert_offsets, const void* w1, int32_t R, int32_t H, int32_t E,
                                    int32_t I, const int32_t* scatter_index, int32_t T, int32_t top_k,
                                    int32_t accumulate, float* d_x, void* d_w1, void* workspace,
                                    size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* LIBMOE_H */
