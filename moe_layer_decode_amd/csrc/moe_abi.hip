// C ABI of the MoE decode layer: argument validation, workspace layout and
// the launch sequence.  Every check runs on the host before any launch, so a
// call that fails has launched nothing and written nothing.
#include <math.h>
#include <stdint.h>
#include <string.h>

#include "moe_internal.h"

namespace {

using moe::MatSeg;
using moe::SegSet;

enum Region {
  R_LOGITS, R_TOPK_IDS, R_TOPK_W, R_HEADER, R_COUNTS, R_OFFSETS, R_ROW_TOKEN, R_ROW_SLOT,
  R_ROW_EXPERT, R_ROW_WEIGHT, R_INV_PERM, R_ACTIVE, R_DCOUNTS, R_DOFFSETS, R_DROW_TOKEN,
  R_DROW_DEPT, R_DROW_SCALE, R_DINV, R_ACTIVE_DEPTS, R_H, R_HD, R_HS, R_ROW_OUT, R_DEPT_OUT,
  R_SHARED_OUT, R_COUNT
};

struct Layout {
  size_t off[R_COUNT];
  size_t total;
};

constexpr size_t kAlign = 256;
size_t round_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

// Largest number of (token, department) pairs: a token covers at most
// min(m, k) departments.
int64_t max_dept_pairs(const moe_layer_desc& d) {
  if (d.n_depts <= 0) return 0;
  return (int64_t)d.max_tokens * (d.n_depts < d.top_k ? d.n_depts : d.top_k);
}

Layout layout_of(const moe_layer_desc& d) {
  const int64_t Tm = d.max_tokens, E = d.n_experts, k = d.top_k, A = Tm * k;
  const int64_t m = d.n_depts > 0 ? d.n_depts : 0, Pm = max_dept_pairs(d);
  size_t sz[R_COUNT];
  sz[R_LOGITS] = Tm * E * 4;
  sz[R_TOPK_IDS] = A * 4;
  sz[R_TOPK_W] = A * 4;
  sz[R_HEADER] = MOE_PLAN_HEADER_LEN * 4;
  sz[R_COUNTS] = E * 4;
  sz[R_OFFSETS] = (E + 1) * 4;
  sz[R_ROW_TOKEN] = sz[R_ROW_SLOT] = sz[R_ROW_EXPERT] = sz[R_ROW_WEIGHT] = sz[R_INV_PERM] = A * 4;
  sz[R_ACTIVE] = E * 4;
  sz[R_DCOUNTS] = m * 4;
  sz[R_DOFFSETS] = (m + 1) * 4;
  sz[R_DROW_TOKEN] = sz[R_DROW_DEPT] = sz[R_DROW_SCALE] = Pm * 4;
  sz[R_DINV] = Tm * m * 4;
  sz[R_ACTIVE_DEPTS] = m * 4;
  sz[R_H] = A * (int64_t)d.d_ff * 4;
  sz[R_HD] = Pm * (int64_t)(m ? d.d_ff_dept : 0) * 4;
  sz[R_HS] = Tm * (int64_t)d.d_ff_shared * 4;
  sz[R_ROW_OUT] = A * (int64_t)d.d_model * 4;
  sz[R_DEPT_OUT] = Pm * (int64_t)d.d_model * 4;
  sz[R_SHARED_OUT] = (d.d_ff_shared > 0 ? Tm : 0) * (int64_t)d.d_model * 4;
  Layout L;
  size_t o = 0;
  for (int r = 0; r < R_COUNT; ++r) {
    L.off[r] = o;
    o += round_up(sz[r] ? sz[r] : 1);
  }
  L.total = o;
  return L;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
bool ok_ptr(const void* p) { return p != nullptr && aligned16(p); }
bool ok_opt(const void* p) { return p == nullptr || aligned16(p); }

moe_status check_desc(const moe_layer_desc* d) {
  if (!d) return MOE_ERR_INVALID_ARG;
  if (d->d_model <= 0 || d->d_model % 8) return MOE_ERR_INVALID_ARG;
  if (d->n_experts <= 0) return MOE_ERR_INVALID_ARG;
  if (d->top_k <= 0 || d->top_k > d->n_experts) return MOE_ERR_INVALID_ARG;
  if (d->d_ff <= 0 || d->d_ff % 8) return MOE_ERR_INVALID_ARG;
  if (d->n_depts < 0 || d->d_ff_shared < 0 || d->d_ff_shared % 8) return MOE_ERR_INVALID_ARG;
  if (d->n_depts > 0) {
    if (d->n_experts % d->n_depts) return MOE_ERR_INVALID_ARG;
    if (d->d_ff_dept <= 0 || d->d_ff_dept % 8) return MOE_ERR_INVALID_ARG;
  }
  if (d->score_fn < MOE_SCORE_SOFTMAX || d->score_fn > MOE_SCORE_SOFTMAX_BIAS)
    return MOE_ERR_INVALID_ARG;
  if (d->renormalize != 0 && d->renormalize != 1) return MOE_ERR_INVALID_ARG;
  if (!isfinite(d->route_scale)) return MOE_ERR_INVALID_ARG;
  if (d->max_tokens <= 0) return MOE_ERR_INVALID_ARG;
  if (d->w_dtype != MOE_F32 && d->w_dtype != MOE_BF16) return MOE_ERR_INVALID_ARG;
  if (d->act_dtype != MOE_F32 && d->act_dtype != MOE_BF16) return MOE_ERR_INVALID_ARG;
  if (d->w_dtype != d->act_dtype) return MOE_ERR_UNSUPPORTED;
  if (d->n_experts > MOE_MAX_EXPERTS || d->top_k > MOE_MAX_TOP_K) return MOE_ERR_UNSUPPORTED;
  if ((int64_t)d->max_tokens * d->top_k > MOE_MAX_ASSIGNMENTS) return MOE_ERR_UNSUPPORTED;
  if ((int64_t)d->max_tokens * d->n_depts > MOE_MAX_DEPT_PAIRS) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

moe_status check_tokens(const moe_layer_desc* d, int32_t T) {
  return (T < 0 || T > d->max_tokens) ? MOE_ERR_INVALID_ARG : MOE_OK;
}

moe_status check_ws(const moe_layer_desc* d, const void* ws, size_t ws_bytes) {
  if (!ws || ((uintptr_t)ws & (kAlign - 1))) return MOE_ERR_WORKSPACE;
  return ws_bytes < layout_of(*d).total ? MOE_ERR_WORKSPACE : MOE_OK;
}

moe_status check_weights(const moe_layer_desc* d, const moe_weights* w, bool need_router,
                         bool need_experts) {
  if (!w) return MOE_ERR_INVALID_ARG;
  if (need_router && (!ok_ptr(w->w_router) || !ok_opt(w->router_bias)))
    return MOE_ERR_INVALID_ARG;
  if (need_router && d->score_fn == MOE_SCORE_SOFTMAX && w->router_bias)
    return MOE_ERR_INVALID_ARG;  // softmax mode ranks the logits alone
  if (!need_experts) return MOE_OK;
  if (!ok_ptr(w->w_gate) || !ok_ptr(w->w_up) || !ok_ptr(w->w_down)) return MOE_ERR_INVALID_ARG;
  if (d->n_depts > 0 && (!ok_ptr(w->wd_gate) || !ok_ptr(w->wd_up) || !ok_ptr(w->wd_down)))
    return MOE_ERR_INVALID_ARG;
  if (d->d_ff_shared > 0 && (!ok_ptr(w->ws_gate) || !ok_ptr(w->ws_up) || !ok_ptr(w->ws_down)))
    return MOE_ERR_INVALID_ARG;
  return MOE_OK;
}

template <typename T>
T* at(void* ws, const Layout& L, Region r) {
  return reinterpret_cast<T*>(static_cast<char*>(ws) + L.off[r]);
}

void fill_plan(const moe_layer_desc& d, void* ws, int32_t T, moe_plan* p) {
  const Layout L = layout_of(d);
  p->header = at<int32_t>(ws, L, R_HEADER);
  p->counts = at<int32_t>(ws, L, R_COUNTS);
  p->offsets = at<int32_t>(ws, L, R_OFFSETS);
  p->row_token = at<int32_t>(ws, L, R_ROW_TOKEN);
  p->row_slot = at<int32_t>(ws, L, R_ROW_SLOT);
  p->row_expert = at<int32_t>(ws, L, R_ROW_EXPERT);
  p->row_weight = at<float>(ws, L, R_ROW_WEIGHT);
  p->inv_perm = at<int32_t>(ws, L, R_INV_PERM);
  p->active = at<int32_t>(ws, L, R_ACTIVE);
  p->dept_counts = at<int32_t>(ws, L, R_DCOUNTS);
  p->dept_offsets = at<int32_t>(ws, L, R_DOFFSETS);
  p->dept_row_token = at<int32_t>(ws, L, R_DROW_TOKEN);
  p->dept_row_dept = at<int32_t>(ws, L, R_DROW_DEPT);
  p->dept_row_scale = at<float>(ws, L, R_DROW_SCALE);
  p->dept_inv = at<int32_t>(ws, L, R_DINV);
  p->active_depts = at<int32_t>(ws, L, R_ACTIVE_DEPTS);
  p->n_tokens = T;
}

moe_status plan_matches(const moe_layer_desc& d, void* ws, const moe_plan* p, int32_t T) {
  if (!p || p->n_tokens != T) return MOE_ERR_INVALID_ARG;
  moe_plan q;
  fill_plan(d, ws, T, &q);
  return (q.header == p->header && q.active == p->active && q.dept_inv == p->dept_inv)
             ? MOE_OK
             : MOE_ERR_INVALID_ARG;
}

int ceil_div(int a, int b) { return (a + b - 1) / b; }

// Matrix families of a step: routed experts (private slices in the department
// form), department slices, the shared expert; outputs per family.
SegSet make_segset(const moe_layer_desc& d, const moe_weights& w, const moe_plan& p, void* ws,
                   int32_t T, float* row_out, float* dept_out, float* shared_out) {
  const Layout L = layout_of(d);
  SegSet set{};
  int n = 0;
  auto add = [&](const MatSeg& s) { set.s[n++] = s; };
  const int tk = T * d.top_k;
  {
    MatSeg s{};
    s.gate = w.w_gate;
    s.up = w.w_up;
    s.down = w.w_down;
    s.rows = d.d_ff;
    s.active = p.active;
    s.n_active = p.header + MOE_PLAN_N_ACTIVE;
    s.grp_off = p.offsets;
    s.grp_token = p.row_token;
    s.h = at<float>(ws, L, R_H);
    s.out = row_out;
    s.max_slots = tk < d.n_experts ? tk : d.n_experts;
    add(s);
  }
  if (d.n_depts > 0) {
    MatSeg s{};
    s.gate = w.wd_gate;
    s.up = w.wd_up;
    s.down = w.wd_down;
    s.rows = d.d_ff_dept;
    s.active = p.active_depts;
    s.n_active = p.header + MOE_PLAN_N_ACTIVE_DEPTS;
    s.grp_off = p.dept_offsets;
    s.grp_token = p.dept_row_token;
    s.h = at<float>(ws, L, R_HD);
    s.out = dept_out;
    s.max_slots = tk < d.n_depts ? tk : d.n_depts;
    add(s);
  }
  if (d.d_ff_shared > 0) {
    MatSeg s{};
    s.gate = w.ws_gate;
    s.up = w.ws_up;
    s.down = w.ws_down;
    s.rows = d.d_ff_shared;
    s.h = at<float>(ws, L, R_HS);
    s.out = shared_out;
    s.max_slots = 1;
    add(s);
  }
  set.n = n;
  set.blk_start[0] = 0;
  for (int i = 0; i < n; ++i) {
    set.s[i].tiles_gu = ceil_div(set.s[i].rows, moe::kGuTile);
    set.s[i].tiles_dn = ceil_div(d.d_model, moe::kDnTile);
  }
  return set;
}

void set_blocks(SegSet& set, bool gateup) {
  set.blk_start[0] = 0;
  for (int i = 0; i < set.n; ++i)
    set.blk_start[i + 1] =
        set.blk_start[i] + set.s[i].max_slots * (gateup ? set.s[i].tiles_gu : set.s[i].tiles_dn);
  for (int i = set.n + 1; i < 4; ++i) set.blk_start[i] = set.blk_start[set.n];
}

moe_status hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

}  // namespace

extern "C" {

size_t moe_workspace_bytes(const moe_layer_desc* desc) {
  if (check_desc(desc) != MOE_OK) return 0;
  return layout_of(*desc).total;
}

moe_status moe_validate_desc(const moe_layer_desc* desc) { return check_desc(desc); }

moe_status moe_plan_from_workspace(const moe_layer_desc* desc, void* workspace, size_t ws_bytes,
                                   int32_t T, moe_plan* plan) {
  moe_status s = check_desc(desc);
  if (s != MOE_OK) return s;
  if ((s = check_tokens(desc, T)) != MOE_OK) return s;
  if ((s = check_ws(desc, workspace, ws_bytes)) != MOE_OK) return s;
  if (!plan) return MOE_ERR_INVALID_ARG;
  fill_plan(*desc, workspace, T, plan);
  return MOE_OK;
}

moe_status moe_route(const moe_layer_desc* desc, const void* x, const void* w_router,
                     const float* router_bias, int32_t T, int32_t* topk_ids, float* topk_w,
                     float* sel_scores, void* workspace, size_t ws_bytes, void* stream) {
  moe_status s = check_desc(desc);
  if (s != MOE_OK) return s;
  if ((s = check_tokens(desc, T)) != MOE_OK) return s;
  if (T == 0) return MOE_OK;
  if (!ok_ptr(x) || !ok_ptr(w_router) || !ok_opt(router_bias) || !ok_ptr(topk_ids) ||
      !ok_ptr(topk_w) || !ok_opt(sel_scores))
    return MOE_ERR_INVALID_ARG;
  if (desc->score_fn == MOE_SCORE_SOFTMAX && router_bias) return MOE_ERR_INVALID_ARG;
  if ((s = check_ws(desc, workspace, ws_bytes)) != MOE_OK) return s;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const Layout L = layout_of(*desc);
  float* logits = at<float>(workspace, L, R_LOGITS);
  hipError_t e = moe::launch_router_logits(desc->w_dtype, x, w_router, T, desc->d_model,
                                           desc->n_experts, logits, st);
  if (e != hipSuccess) return MOE_ERR_HIP;
  moe::TopkArgs tk{logits, router_bias, T, desc->n_experts, desc->top_k, desc->score_fn,
                   desc->renormalize, desc->route_scale, topk_ids, topk_w, sel_scores};
  return hip_status(moe::launch_topk_dispatch(&tk, nullptr, st));
}

moe_status moe_dispatch(const moe_layer_desc* desc, const int32_t* topk_ids, const float* topk_w,
                        int32_t T, void* workspace, size_t ws_bytes, moe_plan* plan,
                        void* stream) {
  moe_status s = check_desc(desc);
  if (s != MOE_OK) return s;
  if ((s = check_tokens(desc, T)) != MOE_OK) return s;
  if (!plan) return MOE_ERR_INVALID_ARG;
  if (T == 0) {
    memset(plan, 0, sizeof(*plan));
    if (check_ws(desc, workspace, ws_bytes) == MOE_OK) fill_plan(*desc, workspace, 0, plan);
    return MOE_OK;
  }
  if (!ok_ptr(topk_ids) || !ok_ptr(topk_w)) return MOE_ERR_INVALID_ARG;
  if ((s = check_ws(desc, workspace, ws_bytes)) != MOE_OK) return s;
  fill_plan(*desc, workspace, T, plan);
  moe::DispatchArgs dp{topk_ids, topk_w, T, desc->n_experts, desc->top_k, desc->n_depts, *plan};
  return hip_status(moe::launch_topk_dispatch(nullptr, &dp, static_cast<hipStream_t>(stream)));
}

moe_status moe_expert_ffn(const moe_layer_desc* desc, const moe_weights* weights, const void* x,
                          int32_t T, const moe_plan* plan, void* workspace, size_t ws_bytes,
                          float* row_out, float* dept_out, float* shared_out, void* stream) {
  moe_status s = check_desc(desc);
  if (s != MOE_OK) return s;
  if ((s = check_tokens(desc, T)) != MOE_OK) return s;
  if (T == 0) return MOE_OK;
  if ((s = check_weights(desc, weights, false, true)) != MOE_OK) return s;
  if (!ok_ptr(x) || !ok_ptr(row_out)) return MOE_ERR_INVALID_ARG;
  if (desc->n_depts > 0 ? !ok_ptr(dept_out) : dept_out != nullptr) return MOE_ERR_INVALID_ARG;
  if (desc->d_ff_shared > 0 ? !ok_ptr(shared_out) : shared_out != nullptr)
    return MOE_ERR_INVALID_ARG;
  if ((s = check_ws(desc, workspace, ws_bytes)) != MOE_OK) return s;
  if ((s = plan_matches(*desc, workspace, plan, T)) != MOE_OK) return s;
  hipStream_t st = static_cast<hipStream_t>(stream);
  SegSet set = make_segset(*desc, *weights, *plan, workspace, T, row_out, dept_out, shared_out);
  set_blocks(set, true);
  hipError_t e = moe::launch_gateup(desc->w_dtype, set, x, T, desc->d_model, st);
  if (e != hipSuccess) return MOE_ERR_HIP;
  set_blocks(set, false);
  return hip_status(moe::launch_down(desc->w_dtype, set, T, desc->d_model, st));
}

moe_status moe_combine(const moe_layer_desc* desc, const moe_plan* plan, const float* row_out,
                       const float* dept_out, const float* shared_out, int32_t T, void* y,
                       void* stream) {
  moe_status s = check_desc(desc);
  if (s != MOE_OK) return s;
  if ((s = check_tokens(desc, T)) != MOE_OK) return s;
  if (T == 0) return MOE_OK;
  if (!plan || plan->n_tokens != T || !plan->inv_perm || !plan->row_weight)
    return MOE_ERR_INVALID_ARG;
  if (!ok_ptr(row_out) || !ok_ptr(y) || !ok_opt(dept_out) || !ok_opt(shared_out))
    return MOE_ERR_INVALID_ARG;
  if (desc->n_depts > 0 ? !ok_ptr(dept_out) : dept_out != nullptr) return MOE_ERR_INVALID_ARG;
  if (desc->d_ff_shared > 0 ? !ok_ptr(shared_out) : shared_out != nullptr)
    return MOE_ERR_INVALID_ARG;
  if (desc->n_depts > 0 && (!plan->dept_inv || !plan->dept_row_scale)) return MOE_ERR_INVALID_ARG;
  moe::CombineArgs a{plan->inv_perm, plan->row_weight, row_out, plan->dept_inv,
                     plan->dept_row_scale, dept_out, shared_out, T, desc->top_k,
                     desc->n_depts, desc->d_model};
  return hip_status(moe::launch_combine(desc->act_dtype, a, y, static_cast<hipStream_t>(stream)));
}

moe_status moe_layer_decode(const moe_layer_desc* desc, const moe_weights* weights, const void* x,
                            int32_t T, void* y, void* workspace, size_t ws_bytes,
                            void* const* stage_events, void* stream) {
  moe_status s = check_desc(desc);
  if (s != MOE_OK) return s;
  if ((s = check_tokens(desc, T)) != MOE_OK) return s;
  if (T == 0) return MOE_OK;
  if ((s = check_weights(desc, weights, true, true)) != MOE_OK) return s;
  if (!ok_ptr(x) || !ok_ptr(y)) return MOE_ERR_INVALID_ARG;
  if ((s = check_ws(desc, workspace, ws_bytes)) != MOE_OK) return s;
  if (stage_events)
    for (int i = 0; i <= MOE_N_STAGES; ++i)
      if (!stage_events[i]) return MOE_ERR_INVALID_ARG;

  hipStream_t st = static_cast<hipStream_t>(stream);
  auto mark = [&](int i) -> bool {
    return !stage_events || hipEventRecord(static_cast<hipEvent_t>(stage_events[i]), st) == hipSuccess;
  };
  const Layout L = layout_of(*desc);
  moe_plan plan;
  fill_plan(*desc, workspace, T, &plan);
  float* logits = at<float>(workspace, L, R_LOGITS);
  float* row_out = at<float>(workspace, L, R_ROW_OUT);
  float* dept_out = desc->n_depts > 0 ? at<float>(workspace, L, R_DEPT_OUT) : nullptr;
  float* shared_out = desc->d_ff_shared > 0 ? at<float>(workspace, L, R_SHARED_OUT) : nullptr;

  if (!mark(MOE_STAGE_ROUTE)) return MOE_ERR_HIP;
  if (moe::launch_router_logits(desc->w_dtype, x, weights->w_router, T, desc->d_model,
                                desc->n_experts, logits, st) != hipSuccess)
    return MOE_ERR_HIP;
  if (!mark(MOE_STAGE_DISPATCH)) return MOE_ERR_HIP;
  moe::TopkArgs tk{logits, weights->router_bias, T, desc->n_experts, desc->top_k,
                   desc->score_fn, desc->renormalize, desc->route_scale,
                   at<int32_t>(workspace, L, R_TOPK_IDS), at<float>(workspace, L, R_TOPK_W),
                   nullptr};
  moe::DispatchArgs dp{nullptr, nullptr, T, desc->n_experts, desc->top_k, desc->n_depts, plan};
  if (moe::launch_topk_dispatch(&tk, &dp, st) != hipSuccess) return MOE_ERR_HIP;
  SegSet set = make_segset(*desc, *weights, plan, workspace, T, row_out, dept_out, shared_out);
  if (!mark(MOE_STAGE_GATEUP)) return MOE_ERR_HIP;
  set_blocks(set, true);
  if (moe::launch_gateup(desc->w_dtype, set, x, T, desc->d_model, st) != hipSuccess)
    return MOE_ERR_HIP;
  if (!mark(MOE_STAGE_DOWN)) return MOE_ERR_HIP;
  set_blocks(set, false);
  if (moe::launch_down(desc->w_dtype, set, T, desc->d_model, st) != hipSuccess)
    return MOE_ERR_HIP;
  if (!mark(MOE_STAGE_COMBINE)) return MOE_ERR_HIP;
  moe::CombineArgs a{plan.inv_perm, plan.row_weight, row_out, plan.dept_inv,
                     plan.dept_row_scale, dept_out, shared_out, T, desc->top_k,
                     desc->n_depts, desc->d_model};
  if (moe::launch_combine(desc->act_dtype, a, y, st) != hipSuccess) return MOE_ERR_HIP;
  if (!mark(MOE_N_STAGES)) return MOE_ERR_HIP;
  return MOE_OK;
}

const char* moe_status_string(moe_status status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported configuration";
    case MOE_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
    case MOE_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

uint64_t moe_loaded_weight_bytes(const moe_layer_desc* desc, int32_t n_active,
                                 int32_t n_active_depts) {
  if (check_desc(desc) != MOE_OK) return 0;
  const uint64_t wb = desc->w_dtype == MOE_BF16 ? 2 : 4;
  const uint64_t d = desc->d_model;
  uint64_t n = (uint64_t)desc->n_experts * d;
  n += (uint64_t)n_active * 3 * d * desc->d_ff;
  n += (uint64_t)desc->d_ff_shared * 3 * d;
  if (desc->n_depts > 0) n += (uint64_t)n_active_depts * 3 * d * desc->d_ff_dept;
  return n * wb;
}

}  // extern "C"
