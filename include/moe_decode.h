/*
 * moe_decode.h -- C ABI of the MI355X (gfx950) small-batch decode forward of
 * one Mixture-of-Experts FFN layer.
 *
 * What the layer computes (the pages this follows):
 *   - "DeaMoE: Efficient MoE Structure for Fast Small-Batch Decoding",
 *     section 2.1: Eq. (1) SwiGLU expert, Eq. (2) top-k of the router
 *     logits W_r x, Eq. (3) weighted sum of the selected experts' outputs;
 *     section 3.2: the department backbone is computed once for all of a
 *     department's tokens.  Two department forms: the slice form (an
 *     expert's intermediate is [department-shared slice ; private slice])
 *     and the factorised form of section 3.1, where expert i of department
 *     j computes (W_d^j)^T s(A_d^i^T (SiLU(A_g^i s(W_g^j x)) * (A_u^i
 *     s(W_u^j x)))), s = SiLU, in section 3.2's two-stage order.
 *   - "DeepSeekMoE Guide: Fine-Grained Experts & Dynamic Routing",
 *     "Shared Expert Isolation" and "Auxiliary-Loss-Free Dynamic Load
 *     Balancing": an always-on shared expert; selection on score + bias with
 *     the weights taken from the unbiased scores.
 *   - "MoE inference engineering, clearly explained", "How a batch becomes
 *     expert-specific matrices" and "Local MoE execution pipeline": route ->
 *     dispatch (group assignments by expert, keep each row's token id and an
 *     inverse map) -> grouped expert compute -> combine (restore token order,
 *     apply the routing weights, add).
 *
 * Conventions shared by every call
 *   - Pointers named x, y, w_*, *_out, topk_*, workspace are DEVICE pointers
 *     owned by the caller; `desc`, `weights` and `plan` structs are HOST
 *     memory read during the call only.  The library never allocates or frees
 *     memory and never synchronises the host: every call is asynchronous on
 *     `stream` (a hipStream_t; NULL = the default stream) and may be captured
 *     into a HIP graph.  Nothing is written with hipMemset.
 *   - Every argument is validated on the host before anything is launched; a
 *     call that returns an error has launched nothing and written nothing.
 *     An asynchronous device fault surfaces as MOE_ERR_HIP from a later call.
 *   - T = 0 is a valid no-op (returns MOE_OK, launches nothing).
 *   - Inputs must be finite; NaN/Inf give undefined routing.
 *   - Calls that share a workspace must be ordered on one stream; calls with
 *     distinct workspaces are independent and reentrant.  There is no global
 *     mutable state.
 *   - The workspace (256-byte aligned, moe_workspace_bytes() long) holds a
 *     few completion counters that must read zero before the first call:
 *     run moe_workspace_init() once after allocating it (or zero-fill it).
 *     Every call leaves the counters at zero again.
 *
 * Layouts (row-major, element counts; I = d_ff, S = d_ff_dept, Is = d_ff_shared)
 *   x, y                 [T][d]        act_dtype
 *   w_router             [E][d]        w_dtype          (router "centroids")
 *   router_bias          [E]           float32, may be NULL (= zeros)
 *   w_gate, w_up         [E][I][d]     w_dtype          (nn.Linear out x in)
 *   w_down               [E][d][I]     w_dtype
 *   wd_gate, wd_up       [m][S][d]     w_dtype          (department slices)
 *   wd_down              [m][d][S]     w_dtype
 *   ws_gate, ws_up       [Is][d]       w_dtype          (shared expert)
 *   ws_down              [d][Is]       w_dtype
 *   Factorised department form (dept_form = MOE_DEPT_FACTORISED, I = S):
 *   wd_gate, wd_up       [m][S][d]     W_g^j, W_u^j     (department backbones)
 *   wd_down              [m][d][S]     (W_d^j)^T
 *   w_gate, w_up         [E][S][S]     A_g^i, A_u^i     (private transforms)
 *   w_down               [E][S][S]     (A_d^i)^T
 *   Every pointer must be 16-byte aligned; d, I, S, Is must be multiples of 8.
 *
 * FP8 expert weights (w_dtype = MOE_FP8_E4M3; plain and slice forms)
 *   The DeaMoE page sizes a DeepSeek-V3 expert stored in FP8 (section 2.2)
 *   without fixing a format: here every expert matrix above (routed,
 *   department, shared) holds OCP E4M3 codes, one byte per weight, in the
 *   same layout, and each of its output rows carries one float32 scale:
 *     *_gate_scale, *_up_scale   [.][I] / [m][S] / [Is]  (one per gate/up row)
 *     *_down_scale               [.][d] / [m][d] / [d]   (one per output column)
 *   weight = scale[row] * value(code).  The router stays in act_dtype (BF16).
 *   d, I, S, Is must be multiples of 16 and at most MOE_FP8_MAX_WIDTH.
 */
#ifndef MOE_DECODE_H
#define MOE_DECODE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1,   /* bad descriptor field, NULL/misaligned pointer, T out of range */
  MOE_ERR_UNSUPPORTED = 2,   /* valid request outside the limits below */
  MOE_ERR_WORKSPACE = 3,     /* workspace NULL or smaller than moe_workspace_bytes() */
  MOE_ERR_HIP = 4            /* the HIP runtime reported an error (launch or earlier fault) */
} moe_status;

typedef enum {
  MOE_F32 = 0,
  MOE_BF16 = 1,
  /* OCP 8-bit floating point E4M3 (bias 7, no infinities, S.1111.111 = NaN)
   * expert codes with per-row float32 scales; w_dtype only */
  MOE_FP8_E4M3 = 2
} moe_dtype;

typedef enum {
  /* rank the logits; weights = softmax over the selected logits
   * (DeaMoE Eq. (2)-(3)) */
  MOE_SCORE_SOFTMAX = 0,
  /* rank fp32(sigmoid(l)) + bias; weights = the selected unbiased sigmoid
   * scores, normalised to sum 1 */
  MOE_SCORE_SIGMOID = 1,
  /* rank l + bias; weights = softmax of the selected unbiased logits
   * (the DeepSeekMoE guide's router) */
  MOE_SCORE_SOFTMAX_BIAS = 2
} moe_score_fn;

typedef enum {
  /* expert intermediate = [department slice S ; private slice I] */
  MOE_DEPT_SLICE = 0,
  /* DeaMoE section 3.1: department backbones W^j (S x d) and private
   * S x S transforms A^i, computed in section 3.2's two-stage order */
  MOE_DEPT_FACTORISED = 1
} moe_dept_form;

/* Hard limits (MOE_ERR_UNSUPPORTED beyond them). */
#define MOE_MAX_EXPERTS 2048
#define MOE_MAX_TOP_K 32
#define MOE_MAX_ASSIGNMENTS 4096      /* max_tokens * top_k */
#define MOE_MAX_DEPT_PAIRS 4096       /* max_tokens * n_depts */
#define MOE_MAX_DEPTS_GROUPED 64      /* n_depts limit when k_dept > 0 */
#define MOE_FP8_MAX_WIDTH 8192        /* FP8 layers: largest d, I, S, Is */

typedef struct {
  int32_t d_model;       /* d */
  int32_t n_experts;     /* E, 1..MOE_MAX_EXPERTS */
  int32_t top_k;         /* k, 1..min(E, MOE_MAX_TOP_K) */
  int32_t d_ff;          /* I: routed expert intermediate (the private slice P in the department form) */
  int32_t n_depts;       /* m: 0 = vanilla; else E % m == 0, expert e is in department e / (E/m) */
  int32_t d_ff_dept;     /* S: department-shared slice width (n_depts > 0) */
  int32_t d_ff_shared;   /* Is: always-on shared expert width, 0 = none */
  int32_t score_fn;      /* moe_score_fn */
  int32_t renormalize;   /* 1: weights sum to route_scale; 0: softmax probabilities / raw sigmoid */
  float route_scale;     /* multiplies every routing weight */
  int32_t w_dtype;       /* moe_dtype of all weight matrices; MOE_FP8_E4M3: the expert
                          * matrices (codes + per-row scales, see above), the router in
                          * act_dtype, which must be MOE_BF16 (factorised form: unsupported) */
  int32_t act_dtype;     /* moe_dtype of x and y (MOE_F32 with MOE_F32 weights, else MOE_BF16) */
  int32_t max_tokens;    /* largest T a workspace sized for this descriptor accepts */
  int32_t dept_form;     /* moe_dept_form (n_depts > 0); factorised requires d_ff == d_ff_dept */
  int32_t k_dept;        /* 0 = no cap; else each token's experts come from at most k_dept
                          * departments (DeaMoE section 3.4's group top-k): departments are
                          * ranked by their best expert's selection score (ties to the lower
                          * index), the k_dept best kept, then the top k inside them.
                          * 1 <= k_dept <= n_depts <= MOE_MAX_DEPTS_GROUPED,
                          * top_k <= k_dept * (E / n_depts). */
  int32_t dept_strict;   /* 0 or 1.  1: exactly k_dept departments per token (DeaMoE's
                          * appendix on enforcing k_dept coverage): after the top k above,
                          * while fewer than k_dept departments are covered, the
                          * lowest-ranked chosen expert whose department keeps another
                          * chosen expert gives way to the best expert of the best
                          * uncovered department; slots stay in (score desc, index asc)
                          * order.  Requires k_dept >= 1 and top_k >= k_dept. */
} moe_layer_desc;

typedef struct {
  const void* w_router;
  const float* router_bias;   /* NULL = no bias */
  const void* w_gate;
  const void* w_up;
  const void* w_down;
  const void* wd_gate;        /* department slices: required iff n_depts > 0 */
  const void* wd_up;
  const void* wd_down;
  const void* ws_gate;        /* shared expert: required iff d_ff_shared > 0 */
  const void* ws_up;
  const void* ws_down;
  /* per-row float32 scales of FP8 expert matrices (w_dtype = MOE_FP8_E4M3):
   * required for each matrix present, ignored otherwise */
  const float* w_gate_scale;  /* [E][I] */
  const float* w_up_scale;    /* [E][I] */
  const float* w_down_scale;  /* [E][d] */
  const float* wd_gate_scale; /* [m][S] */
  const float* wd_up_scale;   /* [m][S] */
  const float* wd_down_scale; /* [m][d] */
  const float* ws_gate_scale; /* [Is] */
  const float* ws_up_scale;   /* [Is] */
  const float* ws_down_scale; /* [d] */
} moe_weights;

/* Plan header entries (int32, device). */
#define MOE_PLAN_N_ROWS 0          /* dispatched assignment rows */
#define MOE_PLAN_N_ACTIVE 1        /* experts with >= 1 row */
#define MOE_PLAN_N_DEPT_ROWS 2     /* (token, department) pairs */
#define MOE_PLAN_N_ACTIVE_DEPTS 3  /* departments with >= 1 pair */
#define MOE_PLAN_N_INVALID 4       /* caller-given expert ids outside [0, E) (dropped) */
#define MOE_PLAN_HEADER_LEN 16

/* The dispatch plan: device arrays inside the caller's workspace.
 * Row order: experts ascending, and inside an expert the assignment index
 * a = t*k + j ascending (so token-ascending).  A = max_tokens * top_k. */
typedef struct {
  int32_t* header;          /* [MOE_PLAN_HEADER_LEN] */
  int32_t* counts;          /* [E]   rows per expert */
  int32_t* offsets;         /* [E+1] exclusive prefix of counts */
  int32_t* row_token;       /* [A]   token of each row */
  int32_t* row_slot;        /* [A]   slot j of each row */
  int32_t* row_expert;      /* [A]   expert of each row */
  float* row_weight;        /* [A]   routing weight of each row */
  int32_t* inv_perm;        /* [A]   row of assignment a (-1 if dropped) */
  int32_t* active;          /* [E]   experts with rows, ascending (first header[N_ACTIVE]) */
  int32_t* dept_counts;     /* [m]   pairs per department */
  int32_t* dept_offsets;    /* [m+1] */
  int32_t* dept_row_token;  /* [Pm]  token of each pair (Pm = max_tokens * min(m, k)) */
  int32_t* dept_row_dept;   /* [Pm]  department of each pair */
  float* dept_row_scale;    /* [Pm]  c_{t,j}: sum of the token's weights over its experts in department j */
  int32_t* dept_inv;        /* [max_tokens*m] pair of (t, j), -1 if none */
  int32_t* active_depts;    /* [m]   departments with pairs, ascending */
  int32_t* row_pair;        /* [A]   factorised form: the (token, department) pair of each row */
  int32_t n_tokens;         /* T the plan was built for (host copy) */
} moe_plan;

/* Per-step routing statistics, written on the device by moe_layer_decode
 * (DeepSeekMoE Guide, "Sequence-Level and Batch-Level Expert Routing
 * Balance Metrics": the expert load balance factor is the largest per-expert
 * token count over the mean count of the N_r routed experts; MoE inference
 * engineering, "Expert load imbalance and rank-level tail latency": record
 * the assignment counts of every serving step).  The caller owns the struct
 * in DEVICE memory (8-byte aligned); the top-k + plan kernel fills it in the
 * same launch that builds the plan, so reading it needs no extra launch and
 * the call stays legal in a HIP graph.  Nothing else reads it. */
typedef struct {
  int32_t n_tokens;             /* T of the step */
  int32_t n_assignments;        /* dispatched (token, expert) rows: T*k */
  int32_t n_active_experts;     /* experts with >= 1 row */
  int32_t n_active_depts;       /* departments with >= 1 (token, department) pair; 0 if vanilla */
  int32_t max_expert_rows;      /* max_e rows of expert e */
  int32_t n_invalid;            /* dropped ids (always 0 here: the router picks valid experts) */
  float mean_expert_rows;       /* n_assignments / E */
  float imbalance_ratio;        /* max_expert_rows / mean_expert_rows (0 when T = 0) */
  uint64_t loaded_weight_bytes; /* moe_loaded_weight_bytes(desc, n_active_experts, n_active_depts) */
  int32_t expert_rows[MOE_MAX_EXPERTS]; /* rows of expert e, e < E (entries past E untouched) */
} moe_step_stats;

/* Kernel timing for moe_layer_decode_timed: stage_events is an array of
 * 2 * MOE_N_STAGES hipEvent_t created by the caller (with timing enabled);
 * stage i's kernel is launched with hipExtLaunchKernel so that the runtime
 * records stage_events[2i] when it starts and stage_events[2i+1] when it
 * ends -- the interval is that kernel alone.  In the factorised form the
 * GATEUP stage runs from the start of the backbone gate/up kernel to the end
 * of the private gate/up kernel, and DOWN from the start of the private down
 * kernel to the end of the department down kernel (pair sums in between). */
#define MOE_STAGE_ROUTE 0     /* router logits, split over d across the chip */
#define MOE_STAGE_DISPATCH 1  /* top-k + weights + dispatch plan (one block) */
#define MOE_STAGE_GATEUP 2    /* grouped gate/up with SiLU(g)*u */
#define MOE_STAGE_DOWN 3      /* grouped down */
#define MOE_STAGE_COMBINE 4   /* weighted combine to token order */
#define MOE_N_STAGES 5

/* Bytes of device workspace moe_layer_decode (and every other call) needs for
 * `desc` (T <= desc->max_tokens).  0 if the descriptor is invalid. */
size_t moe_workspace_bytes(const moe_layer_desc* desc);

/* Zeroes the workspace's completion counters (one small kernel on `stream`;
 * no hipMemset).  Call once per workspace before its first use. */
moe_status moe_workspace_init(const moe_layer_desc* desc, void* workspace, size_t ws_bytes,
                              void* stream);

/* Host-only check of a descriptor (no HIP call). */
moe_status moe_validate_desc(const moe_layer_desc* desc);

/* Host-only: fill `plan` with the device addresses of the plan arrays inside
 * `workspace` (the arrays moe_dispatch / moe_layer_decode write), for T tokens. */
moe_status moe_plan_from_workspace(const moe_layer_desc* desc, void* workspace,
                                   size_t ws_bytes, int32_t T, moe_plan* plan);

/* Router: DeaMoE Eq. (2) plus the weights of Eq. (3).
 * logits l[t][e] = sum_c x[t][c] * w_router[e][c] (fp32 accumulate); the
 * selection score per score_fn; the k best per token, slots ordered by
 * (score desc, expert index asc) so ties go to the lower index; weights per
 * score_fn, times route_scale.
 * Writes topk_ids int32[T][k], topk_w float[T][k] and, if sel_scores is not
 * NULL, sel_scores float[T][E] = the exact fp32 values that were ranked.
 * Uses the logits region of `workspace`. */
moe_status moe_route(const moe_layer_desc* desc, const void* x, const void* w_router,
                     const float* router_bias, int32_t T, int32_t* topk_ids,
                     float* topk_w, float* sel_scores, void* workspace,
                     size_t ws_bytes, void* stream);

/* Dispatch ("How a batch becomes expert-specific matrices"): group the T*k
 * assignments (topk_ids[t][j], topk_w[t][j]) by expert, stable in a = t*k+j,
 * with the inverse map, the active-expert list and, for n_depts > 0, the
 * (token, department) pairs with c_{t,j}.  Any ids are accepted; ids outside
 * [0, E) are dropped and counted in header[MOE_PLAN_N_INVALID].  The plan is
 * written into `workspace`; `plan` (host) receives its addresses. */
moe_status moe_dispatch(const moe_layer_desc* desc, const int32_t* topk_ids,
                        const float* topk_w, int32_t T, void* workspace,
                        size_t ws_bytes, moe_plan* plan, void* stream);

/* Grouped expert FFN (DeaMoE Eq. (1)), unweighted, for a plan from
 * moe_dispatch on the same workspace:
 *   row_out[r][:]    = expert row_expert[r] on token row_token[r]      float [n_rows][d]
 *                      (the private slice only when n_depts > 0)
 *   dept_out[q][:]   = department slice dept_row_dept[q] on its token  float [n_dept_rows][d]
 *                      (required iff n_depts > 0)
 *   shared_out[t][:] = shared expert on token t                        float [T][d]
 *                      (required iff d_ff_shared > 0)
 * The intermediates h = SiLU(gate x) * (up x) are kept in act_dtype in
 * `workspace`.
 * Factorised form: row_out[r][:] (float [n_rows][S], row stride S) receives
 * Z = SiLU((A_d^i)^T Y) of row r, and dept_out[q][:] the department output
 * (W_d^j)^T (sum over the pair's rows of weight * Z), so the routing weights
 * are applied here and moe_combine adds dept_out unscaled. */
moe_status moe_expert_ffn(const moe_layer_desc* desc, const moe_weights* weights,
                          const void* x, int32_t T, const moe_plan* plan,
                          void* workspace, size_t ws_bytes, float* row_out,
                          float* dept_out, float* shared_out, void* stream);

/* Combine ("How a batch becomes expert-specific matrices", the combine
 * that restores token order, with DeaMoE section 2.1 Eq. (3)'s weighted
 * sum of the selected experts' outputs; the department term is section
 * 3.2's backbone output scaled by the token's weights in that department;
 * the shared expert of "Shared Expert Isolation" is added with weight 1):
 *   y[t] = sum_j topk weight(t,j) * row_out[inv_perm[t*k+j]]  (slot order)
 *        + sum_J c_{t,J} * dept_out[dept_inv[t*m+J]]           (J ascending)
 *        + shared_out[t]
 * written in act_dtype (bf16: round to nearest even).  Factorised form:
 * y[t] = sum_J dept_out[dept_inv[t*m+J]] + shared_out[t] (row_out unused, may
 * be NULL).  row_out / dept_out / shared_out are device float arrays laid
 * out as moe_expert_ffn writes them; y is the caller's device [T][d]. */
moe_status moe_combine(const moe_layer_desc* desc, const moe_plan* plan,
                       const float* row_out, const float* dept_out,
                       const float* shared_out, int32_t T, void* y, void* stream);

/* The whole decode step of DeaMoE section 2.1 (Eq. (1)-(3)) with the
 * department form of section 3.2 and the shared expert of the DeepSeekMoE
 * Guide, in the order of "Local MoE execution pipeline": route -> top-k +
 * dispatch -> grouped gate/up -> grouped down -> combine, y[T][d] in
 * act_dtype (the kernels on `stream` that moe_layer_kernel_count reports:
 * the down launch writes y itself at T <= 4).  x and y are the caller's
 * device arrays; intermediates live in `workspace`.  `stats`: NULL, or a
 * DEVICE moe_step_stats the step fills (see above).  Errors: every argument
 * is checked before the first launch (nothing written on failure). */
moe_status moe_layer_decode(const moe_layer_desc* desc, const moe_weights* weights,
                            const void* x, int32_t T, void* y, void* workspace,
                            size_t ws_bytes, moe_step_stats* stats, void* stream);

/* moe_layer_decode with per-stage kernel timing (a measurement variant, not
 * a step of the layer): stage_events as described at MOE_N_STAGES, or NULL
 * (then it is exactly moe_layer_decode). */
moe_status moe_layer_decode_timed(const moe_layer_desc* desc, const moe_weights* weights,
                                  const void* x, int32_t T, void* y, void* workspace,
                                  size_t ws_bytes, moe_step_stats* stats,
                                  void* const* stage_events, void* stream);

/* Static text for a status code. */
const char* moe_status_string(moe_status status);

/* Allocation-free decode step, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): moe_layer_decode with no workspace argument.  Its
 * intermediates live in a fixed per-GPU scratch array of
 * MOE_NOALLOC_SCRATCH_BYTES that the library holds from its first use on a
 * GPU until the process ends; the call allocates nothing (no hipMalloc, no
 * hipFree, no allocating library routine).  The caller passes x, y and the
 * optional device stats as for moe_layer_decode.
 *   - The scratch is laid out for exactly T tokens (desc->max_tokens only
 *     bounds T); MOE_ERR_UNSUPPORTED when that layout exceeds
 *     MOE_NOALLOC_SCRATCH_BYTES (moe_workspace_bytes of the descriptor with
 *     max_tokens = T tells the size), before anything is launched.
 *   - The first call on each GPU looks up that GPU's copy of the array (its
 *     device address) and clears its counter region with a small kernel on
 *     `stream`; later calls launch only the layer's kernels.
 *   - Every call on one GPU shares that GPU's array and leaves its contents
 *     behind: calls that overlap on one GPU (different streams, or threads
 *     without ordering) race and give undefined results; order them on one
 *     stream. */
#define MOE_NOALLOC_SCRATCH_BYTES (32u << 20)
moe_status moe_layer_decode_noalloc(const moe_layer_desc* desc, const moe_weights* weights,
                                    const void* x, int32_t T, void* y, moe_step_stats* stats,
                                    void* stream);

/* Host-only: the number of kernels moe_layer_decode launches for T tokens
 * (0 for T = 0, -1 for an invalid descriptor or T): 5 (route, top-k + plan,
 * gate/up, down, combine); 4 where the down projection writes y itself (bf16
 * plain and slice forms at T <= 4 whose rows of h fit its LDS budget -- the
 * combine stage is then an empty interval); 8 in the factorised form
 * (backbone gate/up, private gate/up, private down, pair sums, department
 * down).  One more where the selection runs per token ahead of a separate
 * plan launch (T > 16, or more than 256 experts). */
int32_t moe_layer_kernel_count(const moe_layer_desc* desc, int32_t T);

/* Host-only: work-items of the grouped gate/up (stage MOE_STAGE_GATEUP) or
 * down (MOE_STAGE_DOWN) launch of moe_layer_decode for T tokens -- the grid
 * is sized on the host from T alone, so a profiler's kernel trace can be
 * matched to a stage by its grid size.  Plain and slice forms with bf16 or
 * fp32 weights; 0 for T = 0, FP8 weights or the factorised form; -1 for an
 * invalid descriptor, T or stage. */
int64_t moe_layer_launch_workitems(const moe_layer_desc* desc, int32_t T, int32_t stage);

/* Bytes of weights one step streams for the given active counts: router,
 * n_active routed experts, n_active_depts department slices, the shared
 * expert (each matrix read once; FP8 layers: one byte per expert weight plus
 * the 4-byte row scales, the router in act_dtype).  Host-only. */
uint64_t moe_loaded_weight_bytes(const moe_layer_desc* desc, int32_t n_active,
                                 int32_t n_active_depts);

/* Measurement helper, not a step of the layer: reads `bytes` of device
 * memory at `src` once with the load pattern of the expert kernels (16-byte
 * streaming loads, one 4 KiB row per wave, four rows per 256-thread block)
 * and writes, for every 16 KiB block of the input, the sum of its bf16
 * values as a float into sink[block] (ceil(bytes / 16384) floats, caller
 * owned).  Timing it gives the HBM read rate this access pattern can reach,
 * the reference the expert kernels' roofline fraction is read against.
 * bytes must be a positive multiple of 16384; src and sink 16-byte aligned;
 * errors return before any launch. */
moe_status moe_stream_read(const void* src, size_t bytes, float* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_DECODE_H */
