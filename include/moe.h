/*
 * moe.h -- C ABI of libmoe: the forward pass of a top-k Mixture-of-Experts
 * SwiGLU FFN layer on one AMD Instinct MI355X (gfx950).
 *
 * The layer (after "MoE: dynamism the compiler cannot remove", the natural
 * implementation: router logits -> top-k -> per-expert FFN -> accumulate, and
 * its capacity and grouped-GEMM sections):
 *
 *   logits  = x W_r^T (+ logit_bias)                       [T, E]  fp32
 *   scores  = softmax(logits)  or  sigmoid(logits)          fp32
 *   key     = scores (+ select_bias, sigmoid scoring only)
 *   idx     = top-k(key), ties -> lower expert index        [T, k]  int32
 *   gates   = gate_scale * scores[idx] (/ sum_j scores[idx_j] if renorm)
 *   assignment: (t, j) pairs walked t-major; the r-th pair of expert e is
 *           dropped when a capacity cap = ceil(C T k / E) is set and r >= cap
 *   y_row   = (silu(x_t W_gate_e^T) * (x_t W_up_e^T)) W_down_e^T   per kept pair
 *   out_t   = sum_{kept j} gates[t, j] y_row(t, j) + sum_s FFN_shared_s(x_t)
 *
 * Conventions for every entry point:
 *  - Pointers named as device data (x, weights, outputs, ws) are device
 *    pointers, caller-owned and caller-allocated, row-major, and at least
 *    16-byte aligned.  `cfg` and `w` (the structs) are host pointers, read
 *    during the call only.  `stream` is a hipStream_t (NULL = default stream).
 *  - The library never allocates, frees or synchronises, and never reads
 *    device data on the host: each call validates its arguments on the host,
 *    enqueues kernels on `stream` and returns.  Every launch shape depends
 *    only on the cfg, so moe_forward can be captured in a HIP graph.
 *  - Errors are returned before any launch (negative moe_status); nothing is
 *    thrown.  A launch failure returns MOE_ERR_HIP.  moe_last_error() gives a
 *    thread-local description of the last failure.
 *  - T == 0 (for a valid cfg) returns MOE_OK at once: nothing is launched and
 *    no buffer is touched.
 *  - Drops are data, not errors (drop_mask).
 *  - Weight layout (MOE_LAYOUT_ROWS): every matrix is stored one K-contiguous
 *    row per output channel: w_gate, w_up [E][ffn][d], w_down [E][d][ffn];
 *    shared experts [S][ffn_shared][d] and [S][d][ffn_shared].  INT4 experts:
 *    packed bytes [E][N][K/2] (byte i holds element 2i in its low nibble and
 *    2i+1 in its high nibble, two's complement) plus bf16 scales
 *    [E][N][K/128]; the weight is q * s for the 128-element group along K.
 *    MOE_LAYOUT_TILED holds the same bytes permuted by moe_pack_weights (the
 *    INT4 scales and the router weight keep the row layout).
 *  - Calls on one stream run in order; two calls that share a workspace must
 *    not overlap.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 4

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = -1,  /* null pointer, bad size, bad enum value       */
  MOE_ERR_UNSUPPORTED = -2,  /* valid but outside the shapes the kernels take */
  MOE_ERR_WORKSPACE = -3,    /* ws NULL or ws_bytes < moe_workspace_bytes     */
  MOE_ERR_HIP = -4           /* a HIP launch failed                           */
} moe_status;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1, MOE_INT4_G128 = 2, MOE_FP8_E4M3 = 3, MOE_FP8_E4M3_A8 = 4 } moe_dtype;
typedef enum { MOE_SCORE_SOFTMAX = 0, MOE_SCORE_SIGMOID = 1 } moe_score;
typedef enum { MOE_LAYOUT_ROWS = 0, MOE_LAYOUT_TILED = 1 } moe_layout;

/* Layer shape and routing rule.  Supported: 0 <= T <= 1048576, 1 <= E <= 256,
 * 1 <= k <= min(E, 8), d, ffn, ffn_shared multiples of 128, 0 <= n_shared <= 8,
 * act_dtype MOE_F32 or MOE_BF16 (x, w_router, y_rows, y_shared, out),
 * expert_dtype equal to act_dtype, or MOE_INT4_G128 with act_dtype MOE_BF16,
 * or MOE_FP8_E4M3 with act_dtype MOE_BF16,
 * and every expert matrix (ffn x d, ffn_shared x d) under 2 GiB.
 * FP8 experts ("MoE at the inference level", workarounds: fp8 expert weights
 * halve the bytes): one byte per weight in the OCP E4M3 format ("fn":
 * exponent bias 7, no infinities, largest value 448), w = fp8 * s with one
 * fp32 scale per output channel, s_gate / s_up [E][ffn], s_down [E][d]
 * (shared experts: shs_gate / shs_up [S][ffn_shared], shs_down [S][d]); the
 * activations stay bf16.  The decode kernels convert each byte to bf16 exactly
 * and apply the scale in fp32; the prefill kernels round fp8 * s to bf16 once.
 * MOE_FP8_E4M3_A8 (act_dtype MOE_BF16): the same weights, and
 * the activations of both expert GEMMs in FP8 as well, so that the GEMMs run
 * on the FP8 matrix unit ("MoE at the inference level", Fields, weight_dtype,
 * and workarounds: fp8 expert weights).  Each GEMM row is quantised on its own:
 * x_t for gate/up, and for down the bf16 SwiGLU output row (for the shared
 * experts, their rows concatenated); with amax = max |v| over the row,
 * inv = 448 / amax and scale = amax / 448 in IEEE fp32, code_i = E4M3(v_i * inv) rounded to
 * nearest even (an all-zero row: codes 0, scale 0), and the row stands for
 * code_i * scale.  The GEMMs accumulate code products in fp32 and scale by the
 * row's and the output channel's scales.  Up to 32 tokens the streaming FP8
 * kernels run on the codes held as exact bf16 values, with the row scales in
 * their epilogues; above, the tiled FP8 MFMA kernels.  A forward is seven
 * launches (two row quantisations added).
 * Group-limited selection ("MoE Research", section 2, node-limited routing;
 * "MoE at the inference level", workarounds, device-limited routing): with
 * n_groups = G > 0 the experts form G equal groups of consecutive indices
 * (E % G == 0, G <= 64), a group scores the largest selection key in it, and a
 * token picks its k experts only inside its topk_groups = M best groups (equal
 * group scores: the lower group), 1 <= M <= G, k <= M * E / G.  0 / 0: none. */
typedef struct moe_cfg {
  int32_t T;            /* tokens                                              */
  int32_t d;            /* hidden size                                         */
  int32_t E;            /* routed experts                                      */
  int32_t k;            /* experts per token                                   */
  int32_t ffn;          /* routed expert intermediate size                     */
  int32_t n_shared;     /* always-on shared experts (weight 1, never dropped)  */
  int32_t ffn_shared;   /* shared expert intermediate size (ignored if none)   */
  int32_t act_dtype;    /* moe_dtype                                           */
  int32_t expert_dtype; /* moe_dtype (shared experts use the same dtype)       */
  int32_t score;        /* moe_score                                           */
  int32_t renorm;       /* 1: gates divided by their sum over the k picks      */
  float gate_scale;     /* multiplies routed gates (1.0; 2.5 for DeepSeek-V3)  */
  int32_t cap_num;      /* capacity factor C = cap_num / cap_den;              */
  int32_t cap_den;      /*   0 / 0 = dropless; cap_num = 0 drops every pair    */
  int32_t weight_layout; /* moe_layout of the routed and shared expert weights  */
  int32_t n_groups;     /* expert groups for group-limited selection (0: none) */
  int32_t topk_groups;  /* groups a token may pick from (0: none)              */
} moe_cfg;

/* Expert weights (device pointers, layout above).  s_* are the INT4 or FP8
 * scales (NULL unless expert_dtype is MOE_INT4_G128 or MOE_FP8_E4M3); sh_* /
 * shs_* the shared experts (NULL when n_shared == 0). */
typedef struct moe_experts {
  const void *w_gate, *w_up, *w_down;
  const void *s_gate, *s_up, *s_down;
  const void *sh_gate, *sh_up, *sh_down;
  const void *shs_gate, *shs_up, *shs_down;
} moe_experts;

/* Checks a cfg on the host (no device access).  MOE_OK, or the reason.
 * "MoE: dynamism the compiler cannot remove", batch-1 recipe: every shape a
 * replayed forward uses is fixed ahead of time, so a cfg is accepted or
 * rejected once, on the host, and never inside a captured launch sequence.
 *   cfg: host pointer, read during the call only.  MOE_ERR_INVALID_ARG for a
 *   NULL cfg or a bad enum / size, MOE_ERR_UNSUPPORTED for a valid layer
 *   outside the shapes the kernels take; moe_last_error() names the field. */
moe_status moe_validate(const moe_cfg* cfg);

/* Rows R of the expert-major row buffers (row_token, y_rows): T*k dropless,
 * min(T*k, E*cap) with a capacity.  Negative on an invalid cfg. */
int64_t moe_rows(const moe_cfg* cfg);

/* Capacity cap = ceil(C*T*k/E) in exact integer arithmetic ("MoE: dynamism
 * the compiler cannot remove", capacity section), or -1 when dropless;
 * -2 on an invalid cfg. */
int64_t moe_capacity(const moe_cfg* cfg);

/* Workspace bytes every entry point needs for this cfg (worst case, static).
 * "MoE: dynamism the compiler cannot remove", batch-1 recipe: buffers are
 * allocated once at fixed addresses and nothing is allocated during a replay;
 * the size depends on the cfg only (R = T*k rows dropless, E*cap with a
 * capacity, never on how the tokens route), so one caller-owned buffer of this
 * size serves every forward of that cfg.  0 on an invalid cfg.  The workspace
 * needs no initialisation; its contents after a call are unspecified.
 * The environment variable MOE_ROWS256_MIN_AVG (a test and tuning override of
 * which GEMMs take 256-row tile items: a positive n from n rows per expert on,
 * 0 never, unset the built-in rule) is read by every call and changes this
 * size: size a workspace under the setting it will be used with (a call whose
 * plan needs more than ws_bytes returns MOE_ERR_WORKSPACE). */
size_t moe_workspace_bytes(const moe_cfg* cfg);

/* Router: logits, scores, top-k and gates ("MoE: dynamism ...", natural
 * implementation; FP32 gate probabilities from a max-subtract-expsum softmax
 * as in the launch-bound study's Sub-study 1; sigmoid scoring with a
 * selection-only per-expert bias as in "MoE Research" section 2).
 *   x [T][d] act dtype; w_router [E][d] act dtype; logit_bias [E] fp32 or NULL
 *   (added to the logits); select_bias [E] fp32 or NULL (sigmoid only: added to
 *   the selection key, never to a gate).
 *   Out: topk_idx [T][k] int32 in descending key order (ties -> lower index),
 *   topk_w [T][k] fp32 gates, scores [T][E] fp32 (unbiased) or NULL. */
moe_status moe_route(const moe_cfg* cfg, const void* x, const void* w_router,
                     const float* logit_bias, const float* select_bias,
                     int32_t* topk_idx, float* topk_w, float* scores,
                     void* ws, size_t ws_bytes, void* stream);

/* Permutation: expert histogram, prefix sum, optional capacity with drops,
 * fixed-shape assignment ("MoE: dynamism ...", capacity section and batch-1
 * recipe: fixed-shape scatter into preallocated buffers).
 *   topk_idx [T][k] int32 (a value outside [0, E) is treated as dropped).
 *   Out: counts [E] (pairs routed to each expert, before capacity),
 *   offsets [E+1] (exclusive prefix sum of kept pairs; offsets[E] = kept total),
 *   row_token [R] (token of each expert-major row; rows >= offsets[E] are left
 *   unwritten), slot_row [T][k] (row of each pair, -1 if dropped),
 *   drop_mask [T][k] uint8 (1 = dropped).  Ranks are stable in (t, j) order. */
moe_status moe_permute(const moe_cfg* cfg, const int32_t* topk_idx,
                       int32_t* counts, int32_t* offsets, int32_t* row_token,
                       int32_t* slot_row, uint8_t* drop_mask,
                       void* ws, size_t ws_bytes, void* stream);

/* Grouped expert SwiGLU FFN over ragged per-expert row ranges ("MoE:
 * dynamism ...", grouped GEMM section: one launch over a fixed grid, groups
 * found from a device-side descriptor).
 *   x [T][d]; offsets [E+1] and row_token [R] as produced by moe_permute.
 *   Out: y_rows [R][d] act dtype (row r = FFN_e(x[row_token[r]]) for the expert
 *   e whose range holds r; rows >= offsets[E] unwritten), y_shared [T][d] =
 *   sum over shared experts of FFN_s(x_t) (NULL iff n_shared == 0). */
moe_status moe_expert_ffn(const moe_cfg* cfg, const void* x, const int32_t* offsets,
                          const int32_t* row_token, const moe_experts* w,
                          void* y_rows, void* y_shared,
                          void* ws, size_t ws_bytes, void* stream);

/* Weighted combine ("MoE: dynamism the compiler cannot remove": the natural
 * implementation accumulates each selected expert's output into its token's
 * row, here weighted by the gate; the batch-1 recipe's fixed-shape scatter
 * becomes a gather by slot_row, so every token writes its row once; "MoE
 * Research" section 2: shared experts are added with weight 1).  Fixed order
 * over j, fp32 accumulation, one rounding:
 *   out[t] = sum_{j: slot_row[t,j] in [0, R)} topk_w[t,j] * y_rows[slot_row[t,j]]
 *            + y_shared[t]  (y_shared NULL iff n_shared == 0).  out [T][d].
 *   y_rows [R][d], y_shared [T][d], out [T][d] act dtype, 16-byte aligned;
 *   slot_row [T][k] int32 and topk_w [T][k] fp32, 4-byte aligned.  A slot_row
 *   entry outside [0, R) (a dropped pair) contributes nothing. */
moe_status moe_combine(const moe_cfg* cfg, const void* y_rows, const int32_t* slot_row,
                       const float* topk_w, const void* y_shared, void* out, void* stream);

/* The whole layer in a handful of static-shape launches: route, permute,
 * gate/up SwiGLU GEMM, down GEMM, combine.  "MoE: dynamism the compiler
 * cannot remove", batch-1 recipe and its graph-capture answer: fixed shapes,
 * no host logic and no allocation between launches, so the five launches
 * (four for a single token, moe_forward_launches) capture into one HIP
 * graph per token count; the launch-bound study (picx.dev summary) is why they
 * are five and not one per expert.
 *   x [T][d], w_router [E][d] act dtype; logit_bias, select_bias as in
 *   moe_route; w: expert weights.  Outputs out [T][d] act dtype, topk_idx
 *   [T][k] int32, topk_w [T][k] fp32, drop_mask [T][k] uint8.  ws: workspace of
 *   moe_workspace_bytes(cfg) bytes.  Same results, bit for bit, as moe_route ->
 *   moe_permute -> moe_expert_ffn -> moe_combine on the same inputs. */
moe_status moe_forward(const moe_cfg* cfg, const void* x, const void* w_router,
                       const float* logit_bias, const float* select_bias,
                       const moe_experts* w, void* out, int32_t* topk_idx,
                       float* topk_w, uint8_t* drop_mask,
                       void* ws, size_t ws_bytes, void* stream);

/* moe_forward for callers that cannot allocate (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): the same launches,
 * with the workspace taken from a built-in device array of
 * moe_noalloc_scratch_bytes() = 64 MiB per device (held from library load to
 * process end) instead of a caller buffer.  Nothing is allocated: the array's
 * address on the current device is looked up once (hipGetSymbolAddress) and
 * cached.  Enough for every decode-sized forward (e.g. DeepSeek-V3-shaped at
 * T = 256: 37 MiB); a cfg whose moe_workspace_bytes exceeds it returns
 * MOE_ERR_WORKSPACE before any launch, with no device access.
 * The current device must own `stream` and every pointer.  All calls on one
 * device share its array, which keeps the last call's contents (the layer
 * needs none of them): two calls that overlap in time on one device race and
 * must be ordered, e.g. on one stream.  Arguments as moe_forward. */
moe_status moe_forward_noalloc(const moe_cfg* cfg, const void* x, const void* w_router,
                               const float* logit_bias, const float* select_bias,
                               const moe_experts* w, void* out, int32_t* topk_idx,
                               float* topk_w, uint8_t* drop_mask, void* stream);

/* Bytes of the built-in workspace of moe_forward_noalloc (per device). */
int64_t moe_noalloc_scratch_bytes(void);

/* Route replay (the launch-bound study's Sub-study 2: the routes of one
 * model replayed through a layer's expert weights; replaying the layer's own
 * routes must return its baseline exactly).  The layer from given routes:
 * permute, gate/up SwiGLU GEMM, down GEMM, combine, with no router.
 *   x [T][d]; topk_idx [T][k] int32 (a value outside [0, E) is dropped, as
 *   in moe_permute; indices of one token should be distinct, as top-k makes
 *   them); topk_w [T][k] fp32 gates, used as given.  Capacity applies to the
 *   given routes in (t, j) order.  Out: out [T][d], drop_mask [T][k].
 *   Bit for bit what moe_forward returns when topk_idx / topk_w are its own
 *   routes (and what moe_permute -> moe_expert_ffn -> moe_combine return). */
moe_status moe_forward_with_routes(const moe_cfg* cfg, const void* x, const int32_t* topk_idx,
                                   const float* topk_w, const moe_experts* w, void* out,
                                   uint8_t* drop_mask, void* ws, size_t ws_bytes, void* stream);

/* Repacks weight rows from MOE_LAYOUT_ROWS into MOE_LAYOUT_TILED (out of
 * place; a pure byte permutation, so results do not change, bit for bit).
 * Not from the pages: an MI355X data-layout choice.  A 16-byte load per lane
 * of the matrix cores' operand layout reads 16 rows x 64 bytes, four rows per
 * group of four lanes; the tiled layout stores each 16-row x 64-byte fragment
 * as one contiguous KB in that lane order, so one wave-wide load reads 1 KB of
 * consecutive addresses.  Byte b of row n (R = bytes per row) moves to
 *   ((n/16)*(R/64) + b/64)*1024 + ((b%64)/16)*256 + (n%16)*16 + b%16.
 *   src, dst: device, 16-byte aligned, not overlapping, rows*R bytes each;
 *   rows: a multiple of 16 (a stack [E][N][K] is E*N rows); K elements per row
 *   of `dtype` (MOE_INT4_G128: K/2 packed bytes, K a multiple of 128), R a
 *   multiple of 64.  Pack w_gate, w_up, w_down and the shared matrices once at
 *   load time; scales are not packed.  Async on `stream`. */
moe_status moe_pack_weights(int32_t dtype, const void* src, void* dst, int64_t rows, int32_t K, void* stream);

/* Kernel launches moe_forward enqueues for this cfg (0 on an invalid cfg): 5
 * (router, route / permutation, gate/up, down, combine), or 4 for a single
 * token (T = 1: the down projection and the combine are one launch). */
int32_t moe_forward_launches(const moe_cfg* cfg);

/* Measurement hook for per-kernel timing with HIP events.  When `events` is
 * not NULL, later moe_forward calls on this host thread record events[i] (a
 * caller-created hipEvent_t) on their stream just before their i-th launch
 * and events[n] after the last one, n = moe_forward_launches(cfg); the caller
 * reads them with hipEventElapsedTime after synchronising.  n_events must be
 * at least n + 1 or the hook is ignored.  NULL turns it off.  Meant for eager
 * timing runs, not for graph capture.  Always MOE_OK. */
moe_status moe_set_timing_events(void* const* events, int32_t n_events);

const char* moe_status_str(moe_status s);
const char* moe_last_error(void);
int32_t moe_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H */
