// C ABI of the MoE decode layer: argument validation, workspace layout, the
// choice of GEMV tiling, and the launch sequence.  Every check runs on the
// host before any launch, so a call that fails has launched nothing and
// written nothing.
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <mutex>

#include "moe_internal.h"

// Scratch of the allocation-free entry point: one fixed array per GPU, held
// by the loaded module until the process ends.  In host code this name only
// stands for the symbol; the device address of each GPU's copy comes from
// hipGetSymbolAddress (see noalloc_scratch below) and is the only address
// ever handed to a kernel or copy.
constexpr size_t kNoAllocScratchBytes = (size_t)MOE_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {

using moe::Family;
using moe::FamilySet;
using moe::WorkDesc;

enum Region {
  R_COUNTERS, R_LOGITS, R_TOPK_IDS, R_TOPK_W, R_HEADER, R_COUNTS, R_OFFSETS, R_ROW_TOKEN,
  R_ROW_SLOT, R_ROW_EXPERT, R_ROW_WEIGHT, R_INV_PERM, R_ACTIVE, R_WORK, R_DCOUNTS, R_DOFFSETS,
  R_DROW_TOKEN, R_DROW_DEPT, R_DROW_SCALE, R_DINV, R_ACTIVE_DEPTS, R_DWORK, R_H, R_HD, R_HS,
  R_ROW_OUT, R_DEPT_OUT, R_SHARED_OUT, R_XG, R_XU, R_ROW_PAIR, R_COUNT
};

bool factorised(const moe_layer_desc& d) {
  return d.n_depts > 0 && d.dept_form == MOE_DEPT_FACTORISED;
}

struct Layout {
  size_t off[R_COUNT];
  size_t total;
};

constexpr size_t kAlign = 256;
size_t round_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

int ceil_div(int a, int b) { return (a + b - 1) / b; }

// Completion counters (reserved; every kernel boundary orders the steps today).
size_t n_counters(const moe_layer_desc& d) { return 16 + (size_t)ceil_div(d.d_model, 8); }

int n_route_chunks(const moe_layer_desc& d) { return ceil_div(d.d_model, moe::kRouteChunk); }

bool fp8(const moe_layer_desc& d) { return d.w_dtype == MOE_FP8_E4M3; }

// Element type of the router: the activation dtype when the experts are FP8.
int router_dtype(const moe_layer_desc& d) { return fp8(d) ? d.act_dtype : d.w_dtype; }

// K pieces (partial-logit planes) of the bf16 router: enough (16-expert tile,
// piece) blocks to reach about 512 blocks, at most kMaxRouteSplit planes, and
// at least 128 elements of K per wave (measured: at d = 2048 four planes beat
// eight -- the top-k then reads half the partials -- while at d = 7168 eight
// beat four).  fp32 layers use one plane.
int route_ksplit(const moe_layer_desc& d) {
  if (router_dtype(d) != MOE_BF16) return 1;
  const int tiles = ceil_div(d.n_experts, 16);
  int s = ceil_div(512, tiles);
  if (s > moe::kMaxRouteSplit) s = moe::kMaxRouteSplit;
  const int kmax = d.d_model / (moe::kWaves * 128);
  if (s > kmax) s = kmax;
  return s < 1 ? 1 : s;
}

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
  sz[R_COUNTERS] = n_counters(d) * 4;
  sz[R_LOGITS] = (int64_t)route_ksplit(d) * Tm * E * 4;
  sz[R_TOPK_IDS] = sz[R_TOPK_W] = A * 4;
  sz[R_HEADER] = MOE_PLAN_HEADER_LEN * 4;
  sz[R_COUNTS] = E * 4;
  sz[R_OFFSETS] = (E + 1) * 4;
  sz[R_ROW_TOKEN] = sz[R_ROW_SLOT] = sz[R_ROW_EXPERT] = sz[R_ROW_WEIGHT] = sz[R_INV_PERM] = A * 4;
  sz[R_ACTIVE] = E * 4;
  sz[R_WORK] = 2 * E * sizeof(WorkDesc);
  sz[R_DCOUNTS] = m * 4;
  sz[R_DOFFSETS] = (m + 1) * 4;
  sz[R_DROW_TOKEN] = sz[R_DROW_DEPT] = sz[R_DROW_SCALE] = Pm * 4;
  sz[R_DINV] = Tm * m * 4;
  sz[R_ACTIVE_DEPTS] = m * 4;
  sz[R_DWORK] = 2 * m * sizeof(WorkDesc);
  sz[R_H] = A * (int64_t)d.d_ff * 4;
  sz[R_HD] = Pm * (int64_t)(m ? d.d_ff_dept : 0) * 4;
  sz[R_HS] = Tm * (int64_t)d.d_ff_shared * 4;
  // factorised form: row_out holds the private outputs Z, S wide
  const int64_t row_w = factorised(d) && d.d_ff > d.d_model ? d.d_ff : d.d_model;
  sz[R_ROW_OUT] = A * row_w * 4;
  sz[R_DEPT_OUT] = Pm * (int64_t)d.d_model * 4;
  sz[R_SHARED_OUT] = (d.d_ff_shared > 0 ? Tm : 0) * (int64_t)d.d_model * 4;
  // factorised form: the backbone outputs sigma(W_g^j x), sigma(W_u^j x) per pair
  sz[R_XG] = sz[R_XU] = factorised(d) ? Pm * (int64_t)d.d_ff_dept * 4 : 0;
  sz[R_ROW_PAIR] = A * 4;
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
  if (d->dept_form != MOE_DEPT_SLICE && d->dept_form != MOE_DEPT_FACTORISED)
    return MOE_ERR_INVALID_ARG;
  if (d->n_depts > 0) {
    if (d->n_experts % d->n_depts) return MOE_ERR_INVALID_ARG;
    if (d->d_ff_dept <= 0 || d->d_ff_dept % 8) return MOE_ERR_INVALID_ARG;
    // the private transforms are S x S
    if (d->dept_form == MOE_DEPT_FACTORISED && d->d_ff != d->d_ff_dept) return MOE_ERR_INVALID_ARG;
  } else if (d->dept_form != MOE_DEPT_SLICE) {
    return MOE_ERR_INVALID_ARG;
  }
  if (d->k_dept < 0 || d->k_dept > (d->n_depts > 0 ? d->n_depts : 0)) return MOE_ERR_INVALID_ARG;
  if (d->k_dept > 0 && (int64_t)d->k_dept * (d->n_experts / d->n_depts) < d->top_k)
    return MOE_ERR_INVALID_ARG;  // not enough experts in k_dept departments
  if (d->k_dept > 0 && d->n_depts > MOE_MAX_DEPTS_GROUPED) return MOE_ERR_UNSUPPORTED;
  if (d->dept_strict != 0 && d->dept_strict != 1) return MOE_ERR_INVALID_ARG;
  if (d->dept_strict && (d->k_dept < 1 || d->top_k < d->k_dept))
    return MOE_ERR_INVALID_ARG;  // exact coverage needs a cap and k >= k_dept
  if (d->score_fn < MOE_SCORE_SOFTMAX || d->score_fn > MOE_SCORE_SOFTMAX_BIAS)
    return MOE_ERR_INVALID_ARG;
  if (d->renormalize != 0 && d->renormalize != 1) return MOE_ERR_INVALID_ARG;
  if (!isfinite(d->route_scale)) return MOE_ERR_INVALID_ARG;
  if (d->max_tokens <= 0) return MOE_ERR_INVALID_ARG;
  if (d->w_dtype != MOE_F32 && d->w_dtype != MOE_BF16 && d->w_dtype != MOE_FP8_E4M3)
    return MOE_ERR_INVALID_ARG;
  if (d->act_dtype != MOE_F32 && d->act_dtype != MOE_BF16) return MOE_ERR_INVALID_ARG;
  if (d->w_dtype == MOE_FP8_E4M3) {
    // E4M3 codes with bf16 activations, plain and slice forms; 16 codes per
    // 16-byte load; rows staged in LDS (four of them) bound the widths
    if (d->act_dtype != MOE_BF16 || d->dept_form == MOE_DEPT_FACTORISED)
      return MOE_ERR_UNSUPPORTED;
    const int32_t widths[4] = {d->d_model, d->d_ff, d->n_depts > 0 ? d->d_ff_dept : 0,
                               d->d_ff_shared};
    for (int32_t wdt : widths) {
      if (wdt % 16) return MOE_ERR_INVALID_ARG;
      if (wdt > MOE_FP8_MAX_WIDTH) return MOE_ERR_UNSUPPORTED;
    }
  } else if (d->w_dtype != d->act_dtype) {
    return MOE_ERR_UNSUPPORTED;
  }
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
  if (d->w_dtype == MOE_FP8_E4M3) {  // every matrix present needs its per-row scales
    if (!ok_ptr(w->w_gate_scale) || !ok_ptr(w->w_up_scale) || !ok_ptr(w->w_down_scale))
      return MOE_ERR_INVALID_ARG;
    if (d->n_depts > 0 &&
        (!ok_ptr(w->wd_gate_scale) || !ok_ptr(w->wd_up_scale) || !ok_ptr(w->wd_down_scale)))
      return MOE_ERR_INVALID_ARG;
    if (d->d_ff_shared > 0 &&
        (!ok_ptr(w->ws_gate_scale) || !ok_ptr(w->ws_up_scale) || !ok_ptr(w->ws_down_scale)))
      return MOE_ERR_INVALID_ARG;
  }
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
  p->row_pair = at<int32_t>(ws, L, R_ROW_PAIR);
  p->n_tokens = T;
}

moe::PlanArgs plan_args(const moe_layer_desc& d, void* ws, int32_t T, const moe_plan& p) {
  const Layout L = layout_of(d);
  moe::PlanArgs pa;
  pa.T = T;
  pa.E = d.n_experts;
  pa.k = d.top_k;
  pa.m = d.n_depts;
  pa.factorised = factorised(d) ? 1 : 0;
  pa.plan = p;
  pa.work = at<WorkDesc>(ws, L, R_WORK);
  pa.dwork = at<WorkDesc>(ws, L, R_DWORK);
  pa.stats = nullptr;
  pa.bytes_fixed = pa.bytes_expert = pa.bytes_dept = 0;
  return pa;
}

moe_status plan_matches(const moe_layer_desc& d, void* ws, const moe_plan* p, int32_t T) {
  if (!p || p->n_tokens != T) return MOE_ERR_INVALID_ARG;
  moe_plan q;
  fill_plan(d, ws, T, &q);
  return (q.header == p->header && q.active == p->active && q.dept_inv == p->dept_inv)
             ? MOE_OK
             : MOE_ERR_INVALID_ARG;
}

moe::RouteArgs route_args(const moe_layer_desc& d, void* ws, const void* x, const void* wr,
                          const float* bias, int32_t T, int32_t* ids, float* w, float* sel) {
  const Layout L = layout_of(d);
  moe::RouteArgs ra;
  ra.x = x;
  ra.wr = wr;
  ra.bias = bias;
  ra.T = T;
  ra.d = d.d_model;
  ra.E = d.n_experts;
  ra.k = d.top_k;
  ra.score_fn = d.score_fn;
  ra.renorm = d.renormalize;
  ra.scale = d.route_scale;
  ra.n_chunks = n_route_chunks(d);
  ra.ksplit = route_ksplit(d);
  ra.m = d.n_depts;
  ra.k_dept = d.k_dept;
  ra.strict = d.dept_strict;
  ra.logits = at<float>(ws, L, R_LOGITS);
  ra.ids_out = ids;
  ra.w_out = w;
  ra.sel_out = sel;
  return ra;
}

// ---------------------------------------------------------------------------
// GEMV tiling.  Measured on MI355X: the weight streams run fastest with the
// least work per wave (one gate row + one up row per wave; two column groups
// per wave in down), which keeps the most loads in flight per CU.  Down takes
// as many lanes per weight row as divide every family's row length in
// 16-byte chunks (64, 32 or 16), so no lane idles.
// ---------------------------------------------------------------------------
int family_rows(const moe_layer_desc& d, int f) {
  return f == 0 ? d.d_ff : f == 1 ? d.d_ff_dept : d.d_ff_shared;
}

moe::GemvConfig choose_config(const moe_layer_desc& d, int32_t T) {
  (void)T;
  moe::GemvConfig c;
  c.rows_per_wave = 1;
  c.rows_per_pass = 1;
  int lpr = 64;
  for (int cand : {64, 32, 16}) {
    bool ok = true;
    for (int f = 0; f < 3; ++f) {
      const int r = family_rows(d, f);
      if (r > 0 && (f != 1 || d.n_depts > 0) && (r / 8) % cand) ok = false;
    }
    if (ok) {
      lpr = cand;
      break;
    }
  }
  c.lpr = lpr;
  // Down: two column groups per wave, or four where the routed rows are
  // short (one 8 * lpr step) and d is wide: a small-group block then streams
  // a few KB over hundreds of column tiles per group, and doubling its
  // columns halves the blocks.  Measured on the DeaMoE transform of the
  // DeepSeek-V3-shaped layer (d = 7168, private rows 256): down 168 -> 153 us
  // at batch 8 and 224 -> 199 us at 16; on the DeepSeek-V3-shaped layer
  // itself (rows 2048) four groups ran 9% slower at batch 4, and at d = 2048
  // they gained nothing.
  const int rr = family_rows(d, 0);
  c.col_groups = d.d_model > 2048 && rr > 0 && rr <= 8 * lpr ? 4 : 2;
  return c;
}

// The families one expert launch carries.
enum class Stage {
  kAll,              // vanilla and slice form: every family in one gate/up and one down launch
  kFactBackbone,     // factorised: department backbones sigma(W_g x), sigma(W_u x) (+ shared gate/up)
  kFactPrivateUp,    // factorised: SiLU(A_g x_g) * (A_u x_u) per row, inputs indexed by pair
  kFactPrivateDown,  // factorised: SiLU((A_d)^T y) per row
  kFactDeptDown,     // factorised: (W_d^j)^T of the pair sums (+ shared down)
};

// Matrix families of a step -- routed experts (private slices in the
// department form), department slices, the shared expert -- each split into
// the part for groups of at most four rows and the part for larger groups.
// A part is left out when no group of its size can occur at this T.
FamilySet make_families(const moe_layer_desc& d, const moe_weights& w, const moe_plan& p,
                        void* ws, int32_t T, float* row_out, float* dept_out, float* shared_out,
                        Stage stage = Stage::kAll) {
  const Layout L = layout_of(d);
  const bool routed = stage == Stage::kAll || stage == Stage::kFactPrivateUp ||
                      stage == Stage::kFactPrivateDown;
  const bool dept_shared = stage == Stage::kAll || stage == Stage::kFactBackbone ||
                           stage == Stage::kFactDeptDown;
  FamilySet set{};
  int n = 0;
  const int tk = T * d.top_k;
  const int small_max = moe::kTokInline;
  // Small and large groups come from separate compacted work lists (the
  // large one starts n_mats descriptors in); a large group has more than
  // small_max rows, which bounds how many there can be.
  auto add_parts = [&](Family f, bool can_small, bool can_large, int hdr_small, int hdr_large) {
    if (f.in_rows == 0) f.in_rows = T;  // inputs are x: one row per token
    if (can_small) {
      Family g = f;
      g.large = 0;
      if (g.work) g.n_active = p.header + hdr_small;
      set.f[n++] = g;
    }
    if (can_large) {
      Family g = f;
      g.large = 1;
      if (g.work) {
        g.work = f.work + f.n_mats;
        g.n_active = p.header + hdr_large;
        const int cap = f.max_rows / (small_max + 1);
        if (cap < g.max_slots) g.max_slots = cap;
      }
      if (g.max_slots > 0) set.f[n++] = g;
    }
  };
  const int pairs_max = (int)((int64_t)T * (d.n_depts < d.top_k ? d.n_depts : d.top_k));
  if (routed) {
    Family f{};
    f.gate = w.w_gate;
    f.up = w.w_up;
    f.down = w.w_down;
    f.rows = d.d_ff;
    f.routed = 1;
    f.work = at<WorkDesc>(ws, L, R_WORK);
    f.n_active = p.header + MOE_PLAN_N_ACTIVE;
    f.grp_token = p.row_token;
    f.h = at<void>(ws, L, R_H);
    f.out = row_out;
    f.max_slots = tk < d.n_experts ? tk : d.n_experts;
    f.n_mats = d.n_experts;
    f.max_rows = tk;
    f.gate_scale = w.w_gate_scale;
    f.up_scale = w.w_up_scale;
    f.down_scale = w.w_down_scale;
    if (stage == Stage::kFactPrivateUp) {
      // inputs: the backbone outputs of the row's (token, department) pair
      f.x_gate = at<void>(ws, L, R_XG);
      f.x_up = at<void>(ws, L, R_XU);
      f.grp_token = p.row_pair;
      f.in_rows = pairs_max;
    }
    if (stage == Stage::kFactPrivateDown) f.epi = 1;
    add_parts(f, true, T > small_max, moe::kHdrSmall, moe::kHdrLarge);
  }
  if (d.n_depts > 0 && dept_shared) {
    Family f{};
    f.gate = w.wd_gate;
    f.up = w.wd_up;
    f.down = w.wd_down;
    f.rows = d.d_ff_dept;
    f.work = at<WorkDesc>(ws, L, R_DWORK);
    f.n_active = p.header + MOE_PLAN_N_ACTIVE_DEPTS;
    f.grp_token = p.dept_row_token;
    f.h = at<void>(ws, L, R_HD);
    f.out = dept_out;
    f.max_slots = tk < d.n_depts ? tk : d.n_depts;
    f.n_mats = d.n_depts;
    f.max_rows = pairs_max;
    f.gate_scale = w.wd_gate_scale;
    f.up_scale = w.wd_up_scale;
    f.down_scale = w.wd_down_scale;
    if (stage == Stage::kFactBackbone) {
      f.h = at<void>(ws, L, R_XG);
      f.h2 = at<void>(ws, L, R_XU);
      f.epi = 1;
    }
    add_parts(f, true, T > small_max, moe::kHdrDeptSmall, moe::kHdrDeptLarge);
  }
  if (d.d_ff_shared > 0 && dept_shared) {
    Family f{};
    f.gate = w.ws_gate;
    f.up = w.ws_up;
    f.down = w.ws_down;
    f.rows = d.d_ff_shared;
    f.h = at<void>(ws, L, R_HS);
    f.out = shared_out;
    f.max_slots = 1;
    f.n_mats = 1;
    f.max_rows = T;
    f.gate_scale = w.ws_gate_scale;
    f.up_scale = w.ws_up_scale;
    f.down_scale = w.ws_down_scale;
    add_parts(f, T <= small_max, T > small_max, 0, 0);
  }
  // Large parts first: their blocks stream whole 16-row tiles and live far
  // longer than a small-group block, so they are dispatched first and overlap
  // the many short blocks instead of forming the launch's tail.
  FamilySet ordered = set;
  int o = 0;
  for (int pass = 1; pass >= 0; --pass)
    for (int i = 0; i < n; ++i)
      if (set.f[i].large == pass) ordered.f[o++] = set.f[i];
  ordered.n = n;
  return ordered;
}

// Tiles per slot and the block prefix for one launch: small parts tile by the
// GEMV configuration; large parts of bf16 layers by one 64-row (gate/up) or
// 64-column (down) matrix-core tile per block (each wave 16 of them over the
// whole K), except at decode batches: there gate/up (T <= kSplitKMaxT, 16
// for two-input launches) takes one 16-row tile per block against up to
// two 16-token tiles, and down at d > kSplitKDownMinD (T <= kSplitKDownMaxT,
// intermediate width >= kSplitKMinK) kSplitKCols columns per block, the four
// waves splitting K.  Measured at batch 16: K-split gate/up is faster at
// d = 2048 and at d = 7168 (the DeaMoE transform of the DeepSeek-V3-shaped
// layer: 382 -> 369 us); K-split down is 2-3% faster at d = 7168 but 5%
// slower for the DeaMoE-7B-shaped department groups at d = 2048, and slower
// still over 128-wide experts, where a wave's quarter of K is half a tile.
// fp32 layers tile by 16 rows or columns.
void set_tiles(FamilySet& set, int d, bool gateup, int w_dtype, const moe::GemvConfig& c,
               int T) {
  set.blk_start[0] = 0;
  // At d > 2048 past eight tokens the K-split tiles pay off only where few
  // large groups can exist (each then needs the 4x blocks); with more, the
  // whole-K tiles (gate/up row tiles, 64-column down tiles) stream better
  // (DeaMoE on the DeepSeek-V3 geometry: batch 16 597 -> 586 us, batch 32
  // 704 -> 688 us; its factorised 864-expert form, eight department groups,
  // keeps the split: 772 us against 812).  The bound is the large parts'
  // slot counts.
  int large_groups = 0;
  for (int i = 0; i < set.n; ++i)
    if (set.f[i].large) large_groups += set.f[i].max_slots;
  const bool few_large = d <= 2048 || T <= 8 || large_groups <= moe::kSplitKMaxGroups;
  for (int i = 0; i < set.n; ++i) {
    Family& f = set.f[i];
    // (a launch with two inputs per row passes 16 tokens at a time)
    f.splitk = w_dtype == MOE_BF16 && f.large &&
               (gateup ? T <= (f.x_up ? 16 : moe::kSplitKMaxT) && (f.x_up || few_large)
                       : T <= moe::kSplitKDownMaxT && d > moe::kSplitKDownMinD &&
                             f.rows >= moe::kSplitKMinK && few_large);
    // past kSplitKDownMaxT the routed experts' groups, mostly of a few rows,
    // take row tiles of kDownRowCols columns (DeepSeek-V3-shaped down: 1011 ->
    // 878 us at batch 128); the department slices' and the shared expert's
    // larger groups keep one 64-column tile per block (two per block ran them
    // one after the other: DeaMoE-7B-shaped batch-32 down 23.4 -> 31.6 us)
    if (w_dtype == MOE_BF16 && f.large && !gateup && f.routed && T > moe::kSplitKDownMaxT)
      f.splitk = 2;
    const int lt = w_dtype != MOE_BF16 ? 16
                   : f.splitk == 2    ? moe::kDownRowCols
                   : !f.splitk        ? moe::kWideRows
                   : gateup           ? 16
                                      : moe::kSplitKCols;
    if (f.large)
      f.tiles = ceil_div(gateup ? f.rows : d, lt);
    else
      f.tiles = gateup ? ceil_div(f.rows, moe::kWaves * c.rows_per_wave)
                       : ceil_div(d, moe::kWaves * c.col_groups * (64 / c.lpr));
    set.blk_start[i + 1] = set.blk_start[i] + f.max_slots * f.tiles;
  }
  for (int i = set.n + 1; i <= moe::kMaxParts; ++i) set.blk_start[i] = set.blk_start[set.n];
}

moe::CombineArgs combine_args(const moe_layer_desc& d, const moe_plan& p, const float* row_out,
                              const float* dept_out, const float* shared_out, int32_t T) {
  moe::CombineArgs a;
  a.inv_perm = p.inv_perm;
  a.row_weight = p.row_weight;
  // factorised form: the weights are applied before the department down
  a.row_out = factorised(d) ? nullptr : row_out;
  a.dept_inv = p.dept_inv;
  a.dept_scale = factorised(d) ? nullptr : p.dept_row_scale;
  a.dept_out = dept_out;
  a.shared_out = shared_out;
  a.T = T;
  a.k = d.top_k;
  a.m = d.n_depts;
  a.d = d.d_model;
  a.max_rows = T * d.top_k;
  a.max_dept_rows = (int)((int64_t)T * (d.n_depts < d.top_k ? d.n_depts : d.top_k));
  return a;
}

moe_status hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

// The grouped expert launches of one step.  Vanilla and slice form: one
// gate/up and one down launch over every family.  Factorised form (DeaMoE
// section 3.2): backbone gate/up (sigma(W_g^j x), sigma(W_u^j x) once per
// (token, department)), private gate/up on those, private down with SiLU,
// the weighted pair sums, department down.  ev_gu / ev_dn (may be null)
// bracket the gate/up and the down launches.
moe_status run_experts(const moe_layer_desc& d, const moe_weights& w, const void* x, int32_t T,
                       const moe_plan& p, void* ws, float* row_out, float* dept_out,
                       float* shared_out, hipStream_t st, const moe::KernelEvents* ev_gu,
                       const moe::KernelEvents* ev_dn, bool gateup_only = false) {
  const moe::GemvConfig cfg = choose_config(d, T);
  const int dm = d.d_model;
  if (fp8(d)) {
    // FP8 experts.  Register GEMVs, every part tiled like a small one
    // (kFp8RowsPerWave gate/up rows per wave; down: kFp8DownColGroups *
    // 64 / lpr columns per wave), kTokInline tokens a pass; or every part on
    // 64-row (gate/up) or 64-column (down) matrix-core tiles, 16 or 32 tokens
    // a pass.  Measured: the GEMVs are faster at T = 8 (d = 7168) and at
    // T = 16 with d = 2048, the tiles from T = 16 at d = 7168 (624 against
    // 656 us a step) and far ahead beyond (T = 128: 1293 against 3512 us).
    FamilySet set = make_families(d, w, p, ws, T, row_out, dept_out, shared_out);
    const bool wide = T > 16 || (T > 8 && dm > 2048);
    // FP8 down: 16 lanes per weight row (8 columns per wave) for every row
    // length; measured faster than 32 or 64 lanes on 2048-code rows
    const int lpr = 16;
    set.blk_start[0] = 0;
    for (int i = 0; i < set.n; ++i) {
      Family& f = set.f[i];
      f.tiles = wide ? ceil_div(f.rows, moe::kWideRows)
                     : ceil_div(f.rows, moe::kWaves * moe::kFp8RowsPerWave);
      set.blk_start[i + 1] = set.blk_start[i] + f.max_slots * f.tiles;
    }
    for (int i = set.n + 1; i <= moe::kMaxParts; ++i) set.blk_start[i] = set.blk_start[set.n];
    if ((wide ? moe::launch_fp8_wide(true, set, x, T, dm, st, ev_gu)
              : moe::launch_gateup_fp8(set, x, T, dm, st, ev_gu)) != hipSuccess)
      return MOE_ERR_HIP;
    if (gateup_only) return MOE_OK;
    set.blk_start[0] = 0;
    for (int i = 0; i < set.n; ++i) {
      Family& f = set.f[i];
      f.tiles = wide ? ceil_div(dm, moe::kWideRows)
                     : ceil_div(dm, moe::kWaves * moe::kFp8DownColGroups * (64 / lpr));
      set.blk_start[i + 1] = set.blk_start[i] + f.max_slots * f.tiles;
    }
    for (int i = set.n + 1; i <= moe::kMaxParts; ++i) set.blk_start[i] = set.blk_start[set.n];
    return hip_status(wide ? moe::launch_fp8_wide(false, set, nullptr, T, dm, st, ev_dn)
                           : moe::launch_down_fp8(set, T, dm, lpr, st, ev_dn));
  }
  if (!factorised(d)) {
    FamilySet set = make_families(d, w, p, ws, T, row_out, dept_out, shared_out);
    set_tiles(set, dm, true, d.w_dtype, cfg, T);
    if (moe::launch_gateup(d.w_dtype, set, x, T, dm, cfg.rows_per_wave, cfg.rows_per_pass, st,
                           ev_gu) != hipSuccess)
      return MOE_ERR_HIP;
    if (gateup_only) return MOE_OK;
    set_tiles(set, dm, false, d.w_dtype, cfg, T);
    return hip_status(
        moe::launch_down(d.w_dtype, set, T, dm, cfg.lpr, cfg.col_groups, st, ev_dn));
  }
  const Layout L = layout_of(d);
  const int S = d.d_ff_dept;
  moe::KernelEvents gu0{}, gu1{}, dn0{}, dn1{};
  if (ev_gu) {
    gu0.start = ev_gu->start;
    gu1.stop = ev_gu->stop;
  }
  if (ev_dn) {
    dn0.start = ev_dn->start;
    dn1.stop = ev_dn->stop;
  }
  FamilySet a = make_families(d, w, p, ws, T, row_out, dept_out, shared_out, Stage::kFactBackbone);
  set_tiles(a, dm, true, d.w_dtype, cfg, T);
  if (moe::launch_gateup(d.w_dtype, a, x, T, dm, cfg.rows_per_wave, cfg.rows_per_pass, st,
                         ev_gu ? &gu0 : nullptr) != hipSuccess)
    return MOE_ERR_HIP;
  FamilySet b = make_families(d, w, p, ws, T, row_out, dept_out, shared_out, Stage::kFactPrivateUp);
  set_tiles(b, S, true, d.w_dtype, cfg, T);
  if (moe::launch_gateup(d.w_dtype, b, x, T, S, cfg.rows_per_wave, cfg.rows_per_pass, st,
                         ev_gu ? &gu1 : nullptr) != hipSuccess)
    return MOE_ERR_HIP;
  FamilySet c =
      make_families(d, w, p, ws, T, row_out, dept_out, shared_out, Stage::kFactPrivateDown);
  set_tiles(c, S, false, d.w_dtype, cfg, T);
  if (moe::launch_down(d.w_dtype, c, T, S, cfg.lpr, cfg.col_groups, st, ev_dn ? &dn0 : nullptr) !=
      hipSuccess)
    return MOE_ERR_HIP;
  moe::PairCombineArgs pc;
  pc.n_pairs = p.header + MOE_PLAN_N_DEPT_ROWS;
  pc.pair_token = p.dept_row_token;
  pc.pair_dept = p.dept_row_dept;
  pc.inv_perm = p.inv_perm;
  pc.row_expert = p.row_expert;
  pc.row_weight = p.row_weight;
  pc.z = row_out;
  pc.T = T;
  pc.k = d.top_k;
  pc.group = d.n_experts / d.n_depts;
  pc.cols = S;
  pc.max_rows = T * d.top_k;
  const int pairs_max = T * (d.n_depts < d.top_k ? d.n_depts : d.top_k);
  if (moe::launch_pair_combine(d.act_dtype, pc, at<void>(ws, L, R_HD), pairs_max, st) !=
      hipSuccess)
    return MOE_ERR_HIP;
  FamilySet e = make_families(d, w, p, ws, T, row_out, dept_out, shared_out, Stage::kFactDeptDown);
  set_tiles(e, dm, false, d.w_dtype, cfg, T);
  return hip_status(moe::launch_down(d.w_dtype, e, T, dm, cfg.lpr, cfg.col_groups, st,
                                     ev_dn ? &dn1 : nullptr));
}

// The down projection with the combine as its epilogue (one launch writing y)
// serves bf16-activation layers (bf16 or FP8 weights) in the plain and slice
// forms at batches of at most
// kTokInline tokens, where every group is small, when the rows of h it stages
// fit kDcMaxLds (two blocks per CU) and no intermediate row is longer than
// kDcMaxRows.  Returns false (and fills nothing) otherwise; the step then
// takes the separate down and combine launches.
constexpr size_t kDcMaxLds = 80 * 1024;
bool down_combine_args(const moe_layer_desc& d, const moe_weights& w, const moe_plan& p,
                       void* ws, int32_t T, moe::DownCombineArgs* out) {
  if ((d.w_dtype != MOE_BF16 && !fp8(d)) || d.act_dtype != MOE_BF16 || factorised(d))
    return false;
  if (T < 1 || T > moe::kTokInline) return false;
  const Layout L = layout_of(d);
  moe::DownCombineArgs a{};
  const int tk = T * d.top_k;
  const int pairs = (int)((int64_t)T * (d.n_depts < d.top_k ? d.n_depts : d.top_k));
  int64_t off = 0, items = 0;
  bool fits = true;
  auto add = [&](moe::DcFamily f) {
    if (f.rows > moe::kDcMaxRows) fits = false;
    f.lds_off = (int)off;
    off += (int64_t)f.max_hrows * f.rows;
    items += f.max_items;
    a.f[a.nf++] = f;
  };
  {
    moe::DcFamily f{};
    f.down = w.w_down;
    f.down_scale = w.w_down_scale;
    f.work = at<WorkDesc>(ws, L, R_WORK);  // the small list: every group at T <= kTokInline
    f.n_items = p.header + moe::kHdrSmall;
    f.wrow = p.row_weight;
    f.h = at<void>(ws, L, R_H);
    f.n_hrows = p.header + MOE_PLAN_N_ROWS;
    f.rows = d.d_ff;
    f.max_items = tk < d.n_experts ? tk : d.n_experts;
    f.max_hrows = tk;
    f.n_mats = d.n_experts;
    add(f);
  }
  if (d.n_depts > 0) {
    moe::DcFamily f{};
    f.down = w.wd_down;
    f.down_scale = w.wd_down_scale;
    f.work = at<WorkDesc>(ws, L, R_DWORK);
    f.n_items = p.header + moe::kHdrDeptSmall;
    f.wrow = p.dept_row_scale;
    f.h = at<void>(ws, L, R_HD);
    f.n_hrows = p.header + MOE_PLAN_N_DEPT_ROWS;
    f.rows = d.d_ff_dept;
    f.max_items = pairs < d.n_depts ? pairs : d.n_depts;
    f.max_hrows = pairs;
    f.n_mats = d.n_depts;
    add(f);
  }
  if (d.d_ff_shared > 0) {
    moe::DcFamily f{};
    f.down = w.ws_down;
    f.down_scale = w.ws_down_scale;
    f.h = at<void>(ws, L, R_HS);
    f.rows = d.d_ff_shared;
    f.max_items = 1;
    f.max_hrows = T;
    f.n_mats = 1;
    add(f);
  }
  a.T = T;
  a.d = d.d_model;
  a.fp8 = fp8(d) ? 1 : 0;
  a.h_elems = (int)off;
  a.max_items = (int)items;
  if (!fits || off > (int64_t)kDcMaxLds || moe::down_combine_lds_bytes(a) > kDcMaxLds)
    return false;
  *out = a;
  return true;
}

// Per-device address of `scratch`, looked up once per device with that
// device current (the first moe_layer_decode_noalloc call on it), together
// with a one-time clearing of the workspace's counter region on the caller's
// stream (a fill kernel, no hipMemset).
constexpr int kMaxScratchDevices = 64;
struct ScratchSlot {
  std::once_flag once;
  void* ptr = nullptr;
  hipError_t err = hipSuccess;
};
ScratchSlot g_scratch[kMaxScratchDevices];

moe_status noalloc_scratch(hipStream_t st, void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return MOE_ERR_HIP;
  if (dev < 0 || dev >= kMaxScratchDevices) return MOE_ERR_UNSUPPORTED;
  ScratchSlot& sl = g_scratch[dev];
  std::call_once(sl.once, [&] {
    void* p = nullptr;
    sl.err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (sl.err == hipSuccess && p == nullptr) sl.err = hipErrorInvalidSymbol;
    // counters region: at the start of every layout, never longer than
    // (16 + d/8) words; d is not known yet, so clear the first 64 KiB
    if (sl.err == hipSuccess)
      sl.err = moe::launch_zero(static_cast<unsigned int*>(p), (64u << 10) / 4, st);
    if (sl.err == hipSuccess) sl.ptr = p;
  });
  if (sl.err != hipSuccess || !sl.ptr) return MOE_ERR_HIP;
  *out = sl.ptr;
  return MOE_OK;
}

}  // namespace

extern "C" {

size_t moe_workspace_bytes(const moe_layer_desc* desc) {
  if (check_desc(desc) != MOE_OK) return 0;
  return layout_of(*desc).total;
}

moe_status moe_validate_desc(const moe_layer_desc* desc) { return check_desc(desc); }

moe_status moe_stream_read(const void* src, size_t bytes, float* sink, void* stream) {
  constexpr size_t kBlockBytes = 16384;
  if (!ok_ptr(src) || !ok_ptr(sink) || bytes == 0 || bytes % kBlockBytes) return MOE_ERR_INVALID_ARG;
  const size_t blocks = bytes / kBlockBytes;
  if (blocks > 0x7fffffffu) return MOE_ERR_UNSUPPORTED;
  return hip_status(moe::launch_stream_read(src, blocks, sink, static_cast<hipStream_t>(stream)));
}

moe_status moe_workspace_init(const moe_layer_desc* desc, void* workspace, size_t ws_bytes,
                              void* stream) {
  moe_status s = check_desc(desc);
  if (s != MOE_OK) return s;
  if ((s = check_ws(desc, workspace, ws_bytes)) != MOE_OK) return s;
  const Layout L = layout_of(*desc);
  return hip_status(moe::launch_zero(at<unsigned int>(workspace, L, R_COUNTERS),
                                     n_counters(*desc), static_cast<hipStream_t>(stream)));
}

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
  const moe::RouteArgs ra = route_args(*desc, workspace, x, w_router, router_bias, T, topk_ids,
                                       topk_w, sel_scores);
  return hip_status(
      moe::launch_route(router_dtype(*desc), ra, nullptr, static_cast<hipStream_t>(stream),
                        nullptr));
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
  const moe::PlanArgs pa = plan_args(*desc, workspace, T, *plan);
  return hip_status(moe::launch_dispatch(topk_ids, topk_w, pa, static_cast<hipStream_t>(stream)));
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
  return run_experts(*desc, *weights, x, T, *plan, workspace, row_out, dept_out, shared_out,
                     static_cast<hipStream_t>(stream), nullptr, nullptr);
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
  if (!(factorised(*desc) ? ok_opt(row_out) : ok_ptr(row_out)) || !ok_ptr(y) ||
      !ok_opt(dept_out) || !ok_opt(shared_out))
    return MOE_ERR_INVALID_ARG;
  if (desc->n_depts > 0 ? !ok_ptr(dept_out) : dept_out != nullptr) return MOE_ERR_INVALID_ARG;
  if (desc->d_ff_shared > 0 ? !ok_ptr(shared_out) : shared_out != nullptr)
    return MOE_ERR_INVALID_ARG;
  if (desc->n_depts > 0 && (!plan->dept_inv || !plan->dept_row_scale)) return MOE_ERR_INVALID_ARG;
  const moe::CombineArgs a = combine_args(*desc, *plan, row_out, dept_out, shared_out, T);
  return hip_status(
      moe::launch_combine(desc->act_dtype, a, y, static_cast<hipStream_t>(stream), nullptr));
}

moe_status moe_layer_decode_timed(const moe_layer_desc* desc, const moe_weights* weights,
                                  const void* x, int32_t T, void* y, void* workspace,
                                  size_t ws_bytes, moe_step_stats* stats,
                                  void* const* stage_events, void* stream) {
  moe_status s = check_desc(desc);
  if (s != MOE_OK) return s;
  if ((s = check_tokens(desc, T)) != MOE_OK) return s;
  if (T == 0) return MOE_OK;
  if ((s = check_weights(desc, weights, true, true)) != MOE_OK) return s;
  if (!ok_ptr(x) || !ok_ptr(y)) return MOE_ERR_INVALID_ARG;
  if (stats && ((uintptr_t)stats & 7u)) return MOE_ERR_INVALID_ARG;
  if ((s = check_ws(desc, workspace, ws_bytes)) != MOE_OK) return s;
  moe::KernelEvents ev[MOE_N_STAGES];
  if (stage_events) {
    for (int i = 0; i < 2 * MOE_N_STAGES; ++i)
      if (!stage_events[i]) return MOE_ERR_INVALID_ARG;
    for (int i = 0; i < MOE_N_STAGES; ++i)
      ev[i] = {static_cast<hipEvent_t>(stage_events[2 * i]),
               static_cast<hipEvent_t>(stage_events[2 * i + 1])};
  }
  auto evp = [&](int i) -> const moe::KernelEvents* { return stage_events ? ev + i : nullptr; };

  hipStream_t st = static_cast<hipStream_t>(stream);
  const Layout L = layout_of(*desc);
  moe_plan plan;
  fill_plan(*desc, workspace, T, &plan);
  float* row_out = at<float>(workspace, L, R_ROW_OUT);
  float* dept_out = desc->n_depts > 0 ? at<float>(workspace, L, R_DEPT_OUT) : nullptr;
  float* shared_out = desc->d_ff_shared > 0 ? at<float>(workspace, L, R_SHARED_OUT) : nullptr;

  // router logits, then top-k + dispatch plan (+ the step's statistics)
  const moe::RouteArgs ra =
      route_args(*desc, workspace, x, weights->w_router, weights->router_bias, T,
                 at<int32_t>(workspace, L, R_TOPK_IDS), at<float>(workspace, L, R_TOPK_W), nullptr);
  moe::PlanArgs pa = plan_args(*desc, workspace, T, plan);
  if (stats) {
    const uint64_t b0 = moe_loaded_weight_bytes(desc, 0, 0);
    pa.stats = stats;
    pa.bytes_fixed = b0;
    pa.bytes_expert = moe_loaded_weight_bytes(desc, 1, 0) - b0;
    pa.bytes_dept = moe_loaded_weight_bytes(desc, 0, 1) - b0;
  }
  if (moe::launch_route(router_dtype(*desc), ra, &pa, st, evp(MOE_STAGE_ROUTE)) != hipSuccess)
    return MOE_ERR_HIP;

  // grouped expert FFN, then the combine back to token order: at decode
  // batches of a few tokens, one down launch that writes y itself (the
  // combine stage is then an empty interval)
  moe::DownCombineArgs dca;
  if (down_combine_args(*desc, *weights, plan, workspace, T, &dca)) {
    if ((s = run_experts(*desc, *weights, x, T, plan, workspace, row_out, dept_out, shared_out,
                         st, evp(MOE_STAGE_GATEUP), nullptr, true)) != MOE_OK)
      return s;
    if (moe::launch_down_combine(dca, y, st, evp(MOE_STAGE_DOWN)) != hipSuccess)
      return MOE_ERR_HIP;
    if (stage_events &&
        (hipEventRecord(ev[MOE_STAGE_COMBINE].start, st) != hipSuccess ||
         hipEventRecord(ev[MOE_STAGE_COMBINE].stop, st) != hipSuccess))
      return MOE_ERR_HIP;
    return MOE_OK;
  }
  if ((s = run_experts(*desc, *weights, x, T, plan, workspace, row_out, dept_out, shared_out, st,
                       evp(MOE_STAGE_GATEUP), evp(MOE_STAGE_DOWN))) != MOE_OK)
    return s;
  const moe::CombineArgs ca = combine_args(*desc, plan, row_out, dept_out, shared_out, T);
  if (moe::launch_combine(desc->act_dtype, ca, y, st, evp(MOE_STAGE_COMBINE)) != hipSuccess)
    return MOE_ERR_HIP;
  return MOE_OK;
}

moe_status moe_layer_decode(const moe_layer_desc* desc, const moe_weights* weights, const void* x,
                            int32_t T, void* y, void* workspace, size_t ws_bytes,
                            moe_step_stats* stats, void* stream) {
  return moe_layer_decode_timed(desc, weights, x, T, y, workspace, ws_bytes, stats, nullptr,
                                stream);
}

moe_status moe_layer_decode_noalloc(const moe_layer_desc* desc, const moe_weights* weights,
                                    const void* x, int32_t T, void* y, moe_step_stats* stats,
                                    void* stream) {
  moe_status s = check_desc(desc);
  if (s != MOE_OK) return s;
  if ((s = check_tokens(desc, T)) != MOE_OK) return s;
  if (T == 0) return MOE_OK;
  // the workspace is laid out for exactly T tokens (same kernels and grids
  // as any max_tokens >= T), so the scratch holds the largest step it can
  moe_layer_desc dt = *desc;
  dt.max_tokens = T;
  if (layout_of(dt).total > kNoAllocScratchBytes) return MOE_ERR_UNSUPPORTED;
  void* ws = nullptr;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if ((s = noalloc_scratch(st, &ws)) != MOE_OK) return s;
  return moe_layer_decode_timed(&dt, weights, x, T, y, ws, kNoAllocScratchBytes, stats, nullptr,
                                stream);
}

int32_t moe_layer_kernel_count(const moe_layer_desc* desc, int32_t T) {
  if (check_desc(desc) != MOE_OK || check_tokens(desc, T) != MOE_OK) return -1;
  if (T == 0) return 0;
  const int split = moe::topk_in_one_block(T, desc->n_experts) ? 0 : 1;
  if (factorised(*desc)) return 8 + split;
  // the eligibility test reads only the descriptor and T; the addresses it
  // forms from a workspace base are never dereferenced here
  void* base = reinterpret_cast<void*>(uintptr_t(1) << 20);
  moe_weights w{};
  moe_plan p;
  fill_plan(*desc, base, T, &p);
  moe::DownCombineArgs a;
  return (down_combine_args(*desc, w, p, base, T, &a) ? 4 : 5) + split;
}

int64_t moe_layer_launch_workitems(const moe_layer_desc* desc, int32_t T, int32_t stage) {
  if (check_desc(desc) != MOE_OK || check_tokens(desc, T) != MOE_OK) return -1;
  if (stage != MOE_STAGE_GATEUP && stage != MOE_STAGE_DOWN) return -1;
  if (T == 0 || factorised(*desc) || fp8(*desc)) return 0;
  // grids are sized on the host from T alone; the workspace addresses formed
  // here are never dereferenced
  void* base = reinterpret_cast<void*>(uintptr_t(1) << 20);
  const Layout L = layout_of(*desc);
  moe_weights w{};
  moe_plan p;
  fill_plan(*desc, base, T, &p);
  moe::DownCombineArgs a;
  if (stage == MOE_STAGE_DOWN && down_combine_args(*desc, w, p, base, T, &a))
    return (int64_t)ceil_div(desc->d_model, moe::kDcWaves) * moe::kDcWaves * 64;
  FamilySet set = make_families(*desc, w, p, base, T, at<float>(base, L, R_ROW_OUT),
                                desc->n_depts > 0 ? at<float>(base, L, R_DEPT_OUT) : nullptr,
                                desc->d_ff_shared > 0 ? at<float>(base, L, R_SHARED_OUT) : nullptr);
  set_tiles(set, desc->d_model, stage == MOE_STAGE_GATEUP, desc->w_dtype,
            choose_config(*desc, T), T);
  return (int64_t)set.blk_start[set.n] * moe::kThreads;
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
  const uint64_t d = desc->d_model;
  if (fp8(*desc)) {
    // router in the activation dtype; one byte per expert weight and a
    // 4-byte scale per output row (gate/up rows are I long, down rows d)
    const uint64_t rb = desc->act_dtype == MOE_BF16 ? 2 : 4;
    auto mat3 = [&](uint64_t r) { return 3 * d * r + 4 * (2 * r + d); };
    uint64_t n = (uint64_t)desc->n_experts * d * rb + (uint64_t)n_active * mat3(desc->d_ff);
    if (desc->d_ff_shared > 0) n += mat3(desc->d_ff_shared);
    if (desc->n_depts > 0) n += (uint64_t)n_active_depts * mat3(desc->d_ff_dept);
    return n;
  }
  const uint64_t wb = desc->w_dtype == MOE_BF16 ? 2 : 4;
  uint64_t n = (uint64_t)desc->n_experts * d;
  // factorised form: each private transform is S x S (d_ff == d_ff_dept)
  n += (uint64_t)n_active * 3 * (desc->n_depts > 0 && desc->dept_form == MOE_DEPT_FACTORISED
                                     ? (uint64_t)desc->d_ff
                                     : d) *
       desc->d_ff;
  n += (uint64_t)desc->d_ff_shared * 3 * d;
  if (desc->n_depts > 0) n += (uint64_t)n_active_depts * 3 * d * desc->d_ff_dept;
  return n * wb;
}

}  // extern "C"
