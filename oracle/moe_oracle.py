"""Plain, slow, obviously-correct CPU oracle of one MoE FFN layer's decode step.

TEST INFRASTRUCTURE ONLY.  Only `tests/`, the package smoke check and the
bench's CPU-baseline leg import this module; the HIP product path never does,
and this module imports nothing from it.  It shares no code, constants or
helpers with the HIP path; the only thing both sides share is the seeded input
generator, which holds none of the layer's arithmetic.

Sources (the pages this follows; sections named, sentences restated):
  [DeaMoE]  "DeaMoE: Efficient MoE Structure for Fast Small-Batch Decoding"
            (arXiv 2608.14385): section 2.1 Eq. (1) expert FFN, Eq. (2) top-k
            on router logits, Eq. (3) weighted combine; section 3.1 and
            section 3.2 (departments, two-stage routing); section 3.3 /
            Figure 2 (weights loaded per step); Table 1.
  [DSMoE]   "DeepSeekMoE Guide: Fine-Grained Experts & Dynamic Routing":
            "Shared Expert Isolation", "Mathematical Formulation of the
            DeepSeekMoE Forward Pass", "Auxiliary-Loss-Free Dynamic Load
            Balancing" (selection bias).
  [MoEInf]  "MoE inference engineering, clearly explained": "How a batch
            becomes expert-specific matrices" (the four-token worked example,
            dispatch and combine), "Local MoE execution pipeline" (permutation
            and its inverse mapping).

Precision: inputs are fp32 (bf16 storage widens exactly).  Every dot product
and every sum is done in float64; the only fp32 roundings are where a decision
is taken (the logits and selection scores that top-k ranks, because the HIP
path ranks fp32 values) and the final cast of y to the output dtype.

Readings where the pages leave a step open (each is also listed with its
justification in the design notes):
  R1 selection ranks the router logits themselves (Eq. (2) applies TopK to
     W_r x), softmax is applied to the selected logits afterwards;
  R2 ties go to the lower expert index; slots are ordered by (score desc,
     index asc);
  R3 inside an expert group rows are ordered by assignment index t*k+j
     (token ascending);
  R4 route_scale multiplies the final weights (the paper's "scaling"; 1.0 in
     every layer shape used here);
  R5 sigmoid mode: rank s+b with s = sigmoid(l) in fp32; weights are the
     selected *unbiased* s renormalised to sum 1;
  R6 softmax_bias mode: rank l+b, weights = softmax of the selected unbiased
     logits (the DeepSeekMoE guide's router);
  R7 the layer output has no residual term;
  R8 the shared expert is added with weight 1;
  R9 department slice form: expert e belongs to department e // (E/m); its
     intermediate is [department slice S ; private slice P];
  R10 c_{t,j} = sum of the token's final weights over its selected experts
     in department j;
  R15 factorised department experts (DeaMoE section 3.1): the interface
     non-linearity sigma is SiLU at all three interfaces (section 3.4 adopts
     it);
  R16 storage of the factorised form: W_d^j is kept as its transpose
     [d][hffn] and A_d^i as its transpose [hffn][hffn], so that each output
     is one contiguous row; the functions below turn them back into W_d^j and
     A_d^i and apply the transposes the pages write;
  R17 the GPU pre-combines a token's p_i * Z^{j,i} over its experts in
     department j before the single (W_d^j)^T product, exact by linearity;
     the oracle keeps the pages' order (one product per expert) and a test
     pins the two equal;
  R18 department-limited (group) top-k (DeaMoE section 3.4, k_dept caps the
     departments a token activates): a department's score is the best
     selection score among its experts; the k_dept best departments are
     taken (ties to the lower department index), then the k best experts
     inside them (ties to the lower expert index).
  R19 strict department coverage (DeaMoE's appendix on enforcing k_dept
     coverage): starting from R18's selection, while it spans fewer than
     k_dept departments, the lowest-ranked selected expert whose department
     keeps another selected expert leaves, and the best expert (score desc,
     index asc) of any uncovered department enters.  Removing an expert that
     is the last of its department would not raise the coverage, so such
     experts are skipped; k >= k_dept makes every step possible.  The final
     slots are ordered by (score desc, index asc) like every selection.
  R20 FP8 expert weights ([DeaMoE] section 2.2 sizes a DeepSeek-V3 expert
     stored in FP8; the pages fix neither the format nor a scaling scheme):
     codes are OCP E4M3 (the OCP 8-bit floating point specification), and
     each output row of each expert matrix carries one fp32 scale, so the
     weight is scale[row] * value(code).  The router stays in the activation
     dtype.  The oracle computes the layer on these dequantized weights
     exactly; the quantization error belongs to the inputs.
"""
from __future__ import annotations

from typing import Callable, Dict, Optional, Sequence

import numpy as np

__all__ = [
    "router_logits", "selection_scores", "topk_select", "routing_weights",
    "route", "dispatch", "swiglu", "expert_outputs", "combine",
    "layer_bruteforce", "layer_grouped", "dept_layer_expanded",
    "dept_layer_factored", "layer_token_output", "loaded_weight_bytes",
    "deamoe_expert", "deamoe_token_output", "deamoe_layer_per_expert",
    "deamoe_layer_two_stage", "deamoe_layer_precombined",
    "select_from_scores", "topk_select_grouped", "topk_select_strict", "silu", "cast_output", "SOFTMAX", "SIGMOID",
    "SOFTMAX_BIAS", "fp8_e4m3_decode", "fp8_dequantize", "dequantize_layer",
    "loaded_weight_bytes_fp8", "expert_load_stats",
]

SOFTMAX, SIGMOID, SOFTMAX_BIAS = "softmax", "sigmoid", "softmax_bias"


def _f64(a) -> np.ndarray:
    """Widen to float64 (exact for fp32 and bf16 sources)."""
    if hasattr(a, "detach"):  # a torch tensor: widen in torch, then hand to numpy
        a = a.detach().to("cpu")
        import torch
        a = a.to(torch.float64).numpy()
    return np.asarray(a, dtype=np.float64)


def silu(z: np.ndarray) -> np.ndarray:
    """SiLU(z) = z * sigmoid(z) = z / (1 + e^-z) [DeaMoE §2.1; §3.4 names SiLU]."""
    return z / (1.0 + np.exp(-z))


# ----------------------------------------------------------------------------
# Router  [DeaMoE §2.1 Eq. (2), Eq. (3)]; [DSMoE formulation, bias routing]
# ----------------------------------------------------------------------------

def router_logits(x, w_router) -> np.ndarray:
    """l[t, e] = sum_c x[t, c] * W_r[e, c] (Eq. (2)'s W_r x), summed in fp64
    and rounded once to fp32 (the value the top-k ranks)."""
    l64 = _f64(x) @ _f64(w_router).T
    return l64.astype(np.float32)


def selection_scores(l32: np.ndarray, score_fn: str, bias=None) -> np.ndarray:
    """The fp32 value each expert is ranked by.

    softmax:      the logit itself (R1);
    softmax_bias: logit + b (fp32 add);
    sigmoid:      fp32(sigmoid(l)) + b (fp32 add) (R5).
    """
    l32 = np.asarray(l32, dtype=np.float32)
    if score_fn == SOFTMAX:
        return l32.copy()
    b = np.zeros(l32.shape[-1], np.float32) if bias is None else _f64(bias).astype(np.float32)
    if score_fn == SOFTMAX_BIAS:
        return (l32 + b).astype(np.float32)
    if score_fn == SIGMOID:
        s32 = (1.0 / (1.0 + np.exp(-l32.astype(np.float64)))).astype(np.float32)
        return (s32 + b).astype(np.float32)
    raise ValueError(score_fn)


def topk_select(sel: np.ndarray, k: int) -> np.ndarray:
    """Indices of the k largest scores per row, by a full stable sort on
    (score descending, index ascending) (R2)."""
    sel = np.asarray(sel)
    T, E = sel.shape
    ids = np.empty((T, k), dtype=np.int32)
    for t in range(T):
        order = sorted(range(E), key=lambda e: (-float(sel[t, e]), e))
        ids[t] = order[:k]
    return ids


select_from_scores = topk_select


def topk_select_grouped(sel: np.ndarray, k: int, n_depts: int, k_dept: int) -> np.ndarray:
    """Department-limited top-k (R18): per token, rank departments by their
    best expert's score (score desc, department index asc), keep the k_dept
    best, and take the k best experts among those departments' experts
    (score desc, index asc)."""
    sel = np.asarray(sel)
    T, E = sel.shape
    g = E // n_depts
    ids = np.empty((T, k), dtype=np.int32)
    for t in range(T):
        dept_score = [max(float(sel[t, e]) for e in range(j * g, (j + 1) * g))
                      for j in range(n_depts)]
        depts = sorted(range(n_depts), key=lambda j: (-dept_score[j], j))[:k_dept]
        allowed = [e for e in range(E) if e // g in depts]
        order = sorted(allowed, key=lambda e: (-float(sel[t, e]), e))
        ids[t] = order[:k]
    return ids


def topk_select_strict(sel: np.ndarray, k: int, n_depts: int, k_dept: int) -> np.ndarray:
    """Strict department coverage (R19): R18's selection, then swaps until
    exactly k_dept departments are covered (needs k >= k_dept)."""
    if k < k_dept:
        raise ValueError("strict coverage needs k >= k_dept")
    sel = np.asarray(sel)
    T, E = sel.shape
    g = E // n_depts
    grouped = topk_select_grouped(sel, k, n_depts, k_dept)
    ids = np.empty((T, k), dtype=np.int32)
    for t in range(T):
        chosen = [int(e) for e in grouped[t]]      # in rank order
        covered = {e // g for e in chosen}
        while len(covered) < k_dept:
            candidates = [e for e in range(E) if e // g not in covered]
            enter = min(candidates, key=lambda e: (-float(sel[t, e]), e))
            for pos in range(len(chosen) - 1, -1, -1):
                dept = chosen[pos] // g
                if sum(1 for e in chosen if e // g == dept) >= 2:
                    del chosen[pos]
                    break
            chosen.append(enter)
            covered.add(enter // g)
        ids[t] = sorted(chosen, key=lambda e: (-float(sel[t, e]), e))
    return ids


def routing_weights(l32: np.ndarray, ids: np.ndarray, score_fn: str,
                    renormalize: bool = True, route_scale: float = 1.0) -> np.ndarray:
    """Per-slot weights p_i of Eq. (3), in fp64.

    softmax (and softmax_bias): softmax of the selected logits when
    renormalised, else the full softmax's probability of each selected
    expert.  sigmoid: s_i / sum_{selected} s when renormalised, else s_i.
    Then times route_scale (R4)."""
    l = np.asarray(l32, dtype=np.float32).astype(np.float64)
    T, k = ids.shape
    w = np.empty((T, k), dtype=np.float64)
    for t in range(T):
        sel_l = l[t, ids[t]]
        if score_fn in (SOFTMAX, SOFTMAX_BIAS):
            if renormalize:
                e = np.exp(sel_l - sel_l.max())
                w[t] = e / e.sum()
            else:
                e_all = np.exp(l[t] - l[t].max())
                w[t] = e_all[ids[t]] / e_all.sum()
        elif score_fn == SIGMOID:
            s = 1.0 / (1.0 + np.exp(-sel_l))
            w[t] = s / s.sum() if renormalize else s
        else:
            raise ValueError(score_fn)
    return w * route_scale


def route(x, w_router, k: int, score_fn: str = SOFTMAX, bias=None,
          renormalize: bool = True, route_scale: float = 1.0, n_depts: int = 0,
          k_dept: int = 0, strict: bool = False):
    """Router of one decode step: (ids int32[T][k], weights f64[T][k],
    selection scores f32[T][E], logits f32[T][E]).  k_dept > 0 limits each
    token to k_dept departments (R18); strict makes it exactly k_dept (R19)."""
    l32 = router_logits(x, w_router)
    sel = selection_scores(l32, score_fn, bias)
    if strict:
        ids = topk_select_strict(sel, k, n_depts, k_dept)
    elif k_dept:
        ids = topk_select_grouped(sel, k, n_depts, k_dept)
    else:
        ids = topk_select(sel, k)
    w = routing_weights(l32, ids, score_fn, renormalize, route_scale)
    return ids, w, sel, l32


# ----------------------------------------------------------------------------
# Dispatch / permutation  [MoEInf "How a batch becomes expert-specific
# matrices", "Local MoE execution pipeline"]
# ----------------------------------------------------------------------------

def dispatch(ids, n_experts: int, weights=None, n_depts: int = 0) -> Dict[str, np.ndarray]:
    """Group the T*k assignments by expert (counting sort, stable in the
    assignment index a = t*k + j) and record the inverse mapping.

    Returns counts[E], offsets[E+1], row_token/row_slot/row_expert[n_rows],
    row_weight[n_rows] (if weights given), inv_perm[T*k] (row of assignment a,
    -1 if its expert id is out of range), active[] (experts with rows,
    ascending).  With n_depts > 0 also the department pairs: every (token,
    department) with at least one selected expert in that department, grouped
    by department and token-ascending inside it: dept_offsets[m+1],
    dept_row_token[], dept_row_dept[], dept_row_scale[] (c_{t,j}, R10),
    dept_inv[T*m] (pair row of (t, j), -1 if none), active_depts[].
    """
    ids = np.asarray(ids, dtype=np.int64)
    T, k = ids.shape
    A = T * k
    flat = ids.reshape(-1)
    wflat = None if weights is None else _f64(weights).reshape(-1)
    rows = []  # (expert, assignment) pairs in row order
    for e in range(n_experts):
        for a in range(A):
            if flat[a] == e:
                rows.append((e, a))
    counts = np.zeros(n_experts, np.int32)
    for e, _ in rows:
        counts[e] += 1
    offsets = np.zeros(n_experts + 1, np.int32)
    offsets[1:] = np.cumsum(counts)
    inv_perm = np.full(A, -1, np.int32)
    row_token = np.array([a // k for _, a in rows], np.int32)
    row_slot = np.array([a % k for _, a in rows], np.int32)
    row_expert = np.array([e for e, _ in rows], np.int32)
    for r, (_, a) in enumerate(rows):
        inv_perm[a] = r
    plan = dict(counts=counts, offsets=offsets, row_token=row_token,
                row_slot=row_slot, row_expert=row_expert, inv_perm=inv_perm,
                active=np.array([e for e in range(n_experts) if counts[e] > 0], np.int32),
                n_rows=len(rows), n_invalid=int(A - len(rows)))
    if wflat is not None:
        plan["row_weight"] = np.array([wflat[a] for _, a in rows], np.float64)
    if n_depts:
        g = n_experts // n_depts
        pairs = []  # (dept, token, scale)
        for j in range(n_depts):
            for t in range(T):
                members = [s for s in range(k) if 0 <= ids[t, s] < n_experts
                           and ids[t, s] // g == j]
                if members:
                    scale = 0.0
                    if wflat is not None:
                        for s in members:  # slot order
                            scale += wflat[t * k + s]
                    pairs.append((j, t, scale))
        dcounts = np.zeros(n_depts, np.int32)
        for j, _, _ in pairs:
            dcounts[j] += 1
        doff = np.zeros(n_depts + 1, np.int32)
        doff[1:] = np.cumsum(dcounts)
        dinv = np.full(T * n_depts, -1, np.int32)
        for q, (j, t, _) in enumerate(pairs):
            dinv[t * n_depts + j] = q
        plan.update(dept_counts=dcounts, dept_offsets=doff,
                    dept_row_dept=np.array([j for j, _, _ in pairs], np.int32),
                    dept_row_token=np.array([t for _, t, _ in pairs], np.int32),
                    dept_row_scale=np.array([s for _, _, s in pairs], np.float64),
                    dept_inv=dinv,
                    active_depts=np.array([j for j in range(n_depts) if dcounts[j] > 0], np.int32),
                    n_dept_rows=len(pairs))
    return plan


# ----------------------------------------------------------------------------
# Expert FFN  [DeaMoE §2.1 Eq. (1)]; shared expert [DSMoE]
# ----------------------------------------------------------------------------

def _pick_rows(a, idx):
    """Rows `idx` of a matrix (all rows if idx is None), widened to fp64."""
    return _f64(a) if idx is None else _f64(a[list(idx)])


def swiglu(x_t, w_gate, w_up, w_down, cols: Optional[Sequence[int]] = None) -> np.ndarray:
    """MoE_i(x) of Eq. (1): the down projection of SiLU(W_gate x) * (W_up x).

    With the nn.Linear layout used here (gate/up [I][d], down [d][I]) this is
    down @ (silu(gate @ x) * (up @ x)).  `cols` restricts the output to the
    listed entries of d (the intermediate h is always computed in full)."""
    x = _f64(x_t)
    g = _f64(w_gate) @ x
    u = _f64(w_up) @ x
    h = silu(g) * u
    return _pick_rows(w_down, cols) @ h


def _expert_mats(weights, e: int, dept_of: Optional[Callable[[int], int]] = None):
    """(gate, up, down) of routed expert e; in the department slice form the
    rows/columns of its department slice come first (R9)."""
    if dept_of is None:
        return weights["w_gate"][e], weights["w_up"][e], weights["w_down"][e]
    j = dept_of(e)
    g = np.concatenate([_f64(weights["wd_gate"][j]), _f64(weights["w_gate"][e])], axis=0)
    u = np.concatenate([_f64(weights["wd_up"][j]), _f64(weights["w_up"][e])], axis=0)
    dn = np.concatenate([_f64(weights["wd_down"][j]), _f64(weights["w_down"][e])], axis=1)
    return g, u, dn


def _dept_of_fn(n_experts: int, n_depts: int):
    if not n_depts:
        return None
    g = n_experts // n_depts
    return lambda e: e // g


def _shared(weights, x_t, cols=None):
    if weights.get("ws_gate") is None:
        return 0.0
    return swiglu(x_t, weights["ws_gate"], weights["ws_up"], weights["ws_down"], cols)


def cast_output(y: np.ndarray, out_dtype: str):
    """Round y to the output dtype: fp32, or bf16 with round-to-nearest-even
    (done via the fp32 bit pattern: add 0x7FFF plus the lowest kept bit)."""
    y32 = y.astype(np.float32)
    if out_dtype == "f32":
        return y32.astype(np.float64)
    bits = y32.view(np.uint32).astype(np.uint64)
    bits = (bits + 0x7FFF + ((bits >> 16) & 1)) & 0xFFFF0000
    return bits.astype(np.uint32).view(np.float32).astype(np.float64)


def layer_token_output(x_t, ids_t, w_t, weights, n_experts: int, n_depts: int = 0,
                       cols: Optional[Sequence[int]] = None) -> np.ndarray:
    """y_t (fp64, no output rounding) of one token by the per-expert
    definition: sum over its slots in slot order of p_j * MoE_{e_j}(x_t)
    [Eq. (3)], plus the shared expert [DSMoE] (R7, R8).  Department experts use
    the expanded per-expert form (R9)."""
    dept_of = _dept_of_fn(n_experts, n_depts)
    y = 0.0
    for j in range(len(ids_t)):
        g, u, dn = _expert_mats(weights, int(ids_t[j]), dept_of)
        y = y + float(w_t[j]) * swiglu(x_t, g, u, dn, cols)
    return y + _shared(weights, x_t, cols)


def layer_bruteforce(x, weights, ids, w, n_experts: int, n_depts: int = 0,
                     out_dtype: str = "f32", round_out: bool = False) -> np.ndarray:
    """The whole layer by a loop over tokens and slots (no grouping)."""
    T = ids.shape[0]
    rows = [layer_token_output(x[t], ids[t], w[t], weights, n_experts, n_depts)
            for t in range(T)]
    y = np.stack(rows) if T else np.zeros((0, _f64(x).shape[1]))
    return cast_output(y, out_dtype) if round_out else y


def expert_outputs(x, weights, plan, n_experts: int, n_depts: int = 0,
                   dept_split: bool = False):
    """Unweighted per-row outputs of the grouped path.

    row_out[r] = MoE_{row_expert[r]}(x[row_token[r]]) for every dispatched
    row.  With dept_split (the department factored form) row_out uses the
    private slice only, and dept_out[q] = SwiGLU of department slice
    dept_row_dept[q] on token dept_row_token[q]; shared_out[t] = shared
    expert on token t (None if the layer has none)."""
    x = _f64(x)
    T = x.shape[0]
    dept_of = None if dept_split else _dept_of_fn(n_experts, n_depts)
    row_out = []
    for r in range(plan["n_rows"]):
        e, t = int(plan["row_expert"][r]), int(plan["row_token"][r])
        g, u, dn = _expert_mats(weights, e, dept_of)
        row_out.append(swiglu(x[t], g, u, dn))
    d = x.shape[1]
    row_out = np.stack(row_out) if row_out else np.zeros((0, d))
    dept_out = None
    if dept_split and n_depts:
        dept_out = []
        for q in range(plan["n_dept_rows"]):
            j, t = int(plan["dept_row_dept"][q]), int(plan["dept_row_token"][q])
            dept_out.append(swiglu(x[t], weights["wd_gate"][j], weights["wd_up"][j],
                                   weights["wd_down"][j]))
        dept_out = np.stack(dept_out) if dept_out else np.zeros((0, d))
    shared_out = None
    if weights.get("ws_gate") is not None:
        shared_out = np.stack([_shared(weights, x[t]) for t in range(T)]) if T else np.zeros((0, d))
    return row_out, dept_out, shared_out


def combine(plan, row_out, T: int, k: int, dept_out=None, shared_out=None,
            n_depts: int = 0, d: Optional[int] = None) -> np.ndarray:
    """Unpermute-and-combine [MoEInf]: y[t] = sum_j p_{t,j} row_out[inv(t,j)]
    (slot order) + sum_j c_{t,j} dept_out[dept_inv(t,j)] (department order)
    + shared_out[t]."""
    row_out = _f64(row_out)
    if d is None:
        d = row_out.shape[1]
    y = np.zeros((T, d))
    for t in range(T):
        for j in range(k):
            r = int(plan["inv_perm"][t * k + j])
            if r >= 0:
                y[t] += plan["row_weight"][r] * row_out[r]
        if dept_out is not None and n_depts:
            for jd in range(n_depts):
                q = int(plan["dept_inv"][t * n_depts + jd])
                if q >= 0:
                    y[t] += plan["dept_row_scale"][q] * _f64(dept_out[q])
        if shared_out is not None:
            y[t] += _f64(shared_out[t])
    return y


def layer_grouped(x, weights, ids, w, n_experts: int, n_depts: int = 0) -> np.ndarray:
    """The layer by dispatch -> per-row expert outputs -> combine, expanded
    department form."""
    T, k = ids.shape
    plan = dispatch(ids, n_experts, w, n_depts)
    row_out, _, shared_out = expert_outputs(x, weights, plan, n_experts, n_depts)
    return combine(plan, row_out, T, k, shared_out=shared_out, d=_f64(x).shape[1])


def dept_layer_expanded(x, weights, ids, w, n_experts: int, n_depts: int) -> np.ndarray:
    """Oracle-A: each selected expert run with its full intermediate
    [department slice ; private slice] (R9)."""
    return layer_bruteforce(x, weights, ids, w, n_experts, n_depts)


def dept_layer_factored(x, weights, ids, w, n_experts: int, n_depts: int) -> np.ndarray:
    """Oracle-B: the department slice once per (token, department), scaled by
    c_{t,j}, plus each selected expert's private slice weighted by p
    [DeaMoE §3.2's reuse of the department backbone, in slice form]."""
    T, k = ids.shape
    plan = dispatch(ids, n_experts, w, n_depts)
    row_out, dept_out, shared_out = expert_outputs(x, weights, plan, n_experts,
                                                   n_depts, dept_split=True)
    return combine(plan, row_out, T, k, dept_out, shared_out, n_depts, d=_f64(x).shape[1])


# ----------------------------------------------------------------------------
# Factorised DeaMoE experts  [DeaMoE §3.1 (expert = department backbone +
# private transforms), §3.2 (two-stage computation), §3.4 (sigma = SiLU)]
# ----------------------------------------------------------------------------

def _sigma(z):
    """The interface non-linearity between department and expert matrices
    (R15: SiLU)."""
    return silu(z)


def deamoe_expert(x_t, wd_gate_j, wd_up_j, wd_down_j, a_gate_i, a_up_i, a_down_i,
                  cols: Optional[Sequence[int]] = None) -> np.ndarray:
    """DeaMoE_i(x) of expert i in department j (section 3.1):

        g_hat(x) = SiLU(A_g^i sigma(W_g^j x))
        u_hat(x) = A_u^i sigma(W_u^j x)
        d_hat(v) = (W_d^j)^T sigma((A_d^i)^T v)
        DeaMoE_i(x) = d_hat(g_hat(x) * u_hat(x))

    W_g^j, W_u^j are [hffn][d]; A_g^i, A_u^i are [hffn][hffn]; wd_down_j holds
    (W_d^j)^T and a_down_i holds (A_d^i)^T (R16).  `cols` restricts the output
    to the listed entries of d."""
    x = _f64(x_t)
    W_g, W_u = _f64(wd_gate_j), _f64(wd_up_j)
    W_d = _f64(wd_down_j).T                 # [hffn][d]
    A_g, A_u = _f64(a_gate_i), _f64(a_up_i)
    A_d = _f64(a_down_i).T                  # [hffn][hffn]
    g_hat = silu(A_g @ _sigma(W_g @ x))
    u_hat = A_u @ _sigma(W_u @ x)
    v = g_hat * u_hat
    z = _sigma(A_d.T @ v)
    W_dT = W_d.T if cols is None else W_d.T[list(cols)]
    return W_dT @ z


def _deamoe_mats(weights, e: int, n_experts: int, n_depts: int):
    j = e // (n_experts // n_depts)
    return (weights["wd_gate"][j], weights["wd_up"][j], weights["wd_down"][j],
            weights["w_gate"][e], weights["w_up"][e], weights["w_down"][e])


def deamoe_token_output(x_t, ids_t, w_t, weights, n_experts: int, n_depts: int,
                        cols: Optional[Sequence[int]] = None) -> np.ndarray:
    """y_t by Eq. (3) over factorised experts: sum over the token's slots in
    slot order of p_j * DeaMoE_{e_j}(x_t), plus the shared expert (R8)."""
    y = 0.0
    for j in range(len(ids_t)):
        y = y + float(w_t[j]) * deamoe_expert(
            x_t, *_deamoe_mats(weights, int(ids_t[j]), n_experts, n_depts), cols=cols)
    return y + _shared(weights, x_t, cols)


def deamoe_layer_per_expert(x, weights, ids, w, n_experts: int, n_depts: int) -> np.ndarray:
    """The whole factorised layer token by token, each selected expert by its
    own DeaMoE_i (no sharing of the department work)."""
    T = ids.shape[0]
    rows = [deamoe_token_output(x[t], ids[t], w[t], weights, n_experts, n_depts)
            for t in range(T)]
    return np.stack(rows) if T else np.zeros((0, _f64(x).shape[1]))


def deamoe_layer_two_stage(x, weights, ids, w, n_experts: int, n_depts: int) -> np.ndarray:
    """Section 3.2's order.  For each department j, collect its tokens X^j and
    compute X_g^j = sigma(W_g^j X^j), X_u^j = sigma(W_u^j X^j) once; hand each
    expert i its rows: Y^{j,i} = SiLU(A_g^i X_g^{j,i}) * (A_u^i X_u^{j,i}),
    Z^{j,i} = sigma((A_d^i)^T Y^{j,i}); collect Z^j and compute the outputs
    O^j = (W_d^j)^T Z^j; the layer combines them by Eq. (3)."""
    x = _f64(x)
    T, k = ids.shape
    d = x.shape[1]
    plan = dispatch(ids, n_experts, w, n_depts)
    g = n_experts // n_depts
    X_g, X_u = {}, {}                       # (t, j) -> sigma(W x_t)
    for q in range(plan["n_dept_rows"]):
        j, t = int(plan["dept_row_dept"][q]), int(plan["dept_row_token"][q])
        X_g[(t, j)] = _sigma(_f64(weights["wd_gate"][j]) @ x[t])
        X_u[(t, j)] = _sigma(_f64(weights["wd_up"][j]) @ x[t])
    y = np.zeros((T, d))
    for r in range(plan["n_rows"]):         # expert by expert, row by row
        e, t = int(plan["row_expert"][r]), int(plan["row_token"][r])
        j = e // g
        A_g, A_u = _f64(weights["w_gate"][e]), _f64(weights["w_up"][e])
        A_d = _f64(weights["w_down"][e]).T
        Y = silu(A_g @ X_g[(t, j)]) * (A_u @ X_u[(t, j)])
        Z = _sigma(A_d.T @ Y)
        W_d = _f64(weights["wd_down"][j]).T
        O = W_d.T @ Z
        y[t] += plan["row_weight"][r] * O
    shared = weights.get("ws_gate") is not None
    for t in range(T):
        if shared:
            y[t] += _shared(weights, x[t])
    return y


def deamoe_layer_precombined(x, weights, ids, w, n_experts: int, n_depts: int) -> np.ndarray:
    """The same layer with a token's weighted Z^{j,i} summed over its experts
    in department j before one (W_d^j)^T product per (token, department)
    (R17; the order the GPU takes)."""
    x = _f64(x)
    T, k = ids.shape
    d = x.shape[1]
    plan = dispatch(ids, n_experts, w, n_depts)
    g = n_experts // n_depts
    y = np.zeros((T, d))
    for q in range(plan["n_dept_rows"]):
        j, t = int(plan["dept_row_dept"][q]), int(plan["dept_row_token"][q])
        xg = _sigma(_f64(weights["wd_gate"][j]) @ x[t])
        xu = _sigma(_f64(weights["wd_up"][j]) @ x[t])
        zc = 0.0
        for s in range(k):                  # slot order
            e = int(ids[t, s])
            if 0 <= e < n_experts and e // g == j:
                A_d = _f64(weights["w_down"][e]).T
                Y = silu(_f64(weights["w_gate"][e]) @ xg) * (_f64(weights["w_up"][e]) @ xu)
                zc = zc + _f64(w)[t, s] * _sigma(A_d.T @ Y)
        W_d = _f64(weights["wd_down"][j]).T
        y[t] += W_d.T @ zc
    if weights.get("ws_gate") is not None:
        for t in range(T):
            y[t] += _shared(weights, x[t])
    return y


# ----------------------------------------------------------------------------
# Weights streamed per step  [DeaMoE §3.3, Figure 2]
# ----------------------------------------------------------------------------

def loaded_weight_bytes(ids, n_experts: int, d: int, d_ff: int, bytes_per_w: int,
                        n_depts: int = 0, d_ff_dept: int = 0, d_ff_shared: int = 0,
                        include_router: bool = True, factorised: bool = False) -> int:
    """Bytes of weights one decode step must read, each matrix once:
    router E*d, every distinct selected expert's three d x I matrices (three
    I x I private transforms in the factorised form, section 3.1), the shared
    expert, and (department forms) every distinct selected department's
    three d x S matrices."""
    ids = np.asarray(ids).reshape(-1)
    experts = {int(e) for e in ids if 0 <= e < n_experts}
    n = (n_experts * d if include_router else 0)
    n += len(experts) * 3 * (d_ff if factorised else d) * d_ff
    n += 3 * d * d_ff_shared
    if n_depts:
        g = n_experts // n_depts
        n += len({e // g for e in experts}) * 3 * d * d_ff_dept
    return n * bytes_per_w


def expert_load_stats(ids, n_experts: int, n_depts: int = 0) -> Dict[str, object]:
    """Routing load of one step ([DSMoE] "Sequence-Level and Batch-Level
    Expert Routing Balance Metrics"; [MoEInf] "Expert load imbalance and
    rank-level tail latency": count assignments per expert every step).
    Tokens_j = assignments to routed expert j; the imbalance ratio is
    max_j Tokens_j divided by the mean (1/N_r) sum_j Tokens_j over all N_r =
    n_experts routed experts (0 when nothing is assigned).  Also the active
    experts, and the departments holding at least one selected expert."""
    ids = np.asarray(ids).reshape(-1)
    counts = [0] * n_experts
    for e in ids:
        if 0 <= int(e) < n_experts:
            counts[int(e)] += 1
    total = sum(counts)
    mean = total / n_experts
    active = [e for e in range(n_experts) if counts[e] > 0]
    depts = set()
    if n_depts:
        g = n_experts // n_depts
        depts = {e // g for e in active}
    return {"counts": counts, "n_assignments": total, "max": max(counts), "mean": mean,
            "imbalance_ratio": (max(counts) / mean) if total else 0.0,
            "n_active_experts": len(active), "n_active_depts": len(depts)}


# ----------------------------------------------------------------------------
# FP8 expert weights  (reading R20: OCP E4M3 codes, one fp32 scale per
# output row)
# ----------------------------------------------------------------------------

def fp8_e4m3_decode(codes) -> np.ndarray:
    """Values of OCP E4M3 codes in float64, from the format's definition:
    bit 7 is the sign, bits 6..3 the exponent field E (bias 7), bits 2..0
    the mantissa field M.  E = 0 holds zero and the subnormals M/8 * 2^-6;
    otherwise the value is (1 + M/8) * 2^(E-7).  The two codes with E = 15
    and M = 7 are NaN; the format has no infinities, so E = 15 with M < 7 is
    finite (up to 448)."""
    c = np.asarray(codes).astype(np.int64) & 0xFF
    sign = np.where(c >= 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, np.ldexp(m, -9), np.ldexp(8.0 + m, e - 10))
    return np.where((c & 0x7F) == 0x7F, np.nan, sign * mag)


def fp8_dequantize(codes, scales) -> np.ndarray:
    """Weight matrix from its codes [..., rows, cols] and per-row scales
    [..., rows]: W[..., r, c] = scales[..., r] * value(codes[..., r, c])."""
    v = fp8_e4m3_decode(codes)
    s = _f64(scales)
    assert s.shape == v.shape[:-1], (s.shape, v.shape)
    return v * s[..., None]


_FP8_MATS = ("w_gate", "w_up", "w_down", "wd_gate", "wd_up", "wd_down",
             "ws_gate", "ws_up", "ws_down")


class _Fp8Stack:
    """A stack of FP8 matrices [n][rows][cols] read one matrix at a time:
    indexing by a matrix number dequantizes that matrix alone (a whole
    DeepSeek-V3-sized layer in float64 would not fit in host memory)."""

    def __init__(self, codes, scales):
        self.codes, self.scales = codes, scales
        self.shape = tuple(codes.shape)

    def __len__(self):
        return self.shape[0]

    def __getitem__(self, i):
        return fp8_dequantize(self.codes[i], self.scales[i])


def dequantize_layer(weights) -> Dict[str, object]:
    """The layer's weights with every FP8 expert matrix (codes under its own
    name, per-row scales under name + "_scale") replaced by its float64
    dequantized values -- stacked matrices lazily, one matrix per index --
    and the router and bias passed through."""
    out = {}
    for k, v in weights.items():
        if k.endswith("_scale"):
            continue
        if k in _FP8_MATS and (k + "_scale") in weights:
            codes = v.detach().cpu().numpy() if hasattr(v, "detach") else np.asarray(v)
            sc = _f64(weights[k + "_scale"])
            out[k] = _Fp8Stack(codes, sc) if codes.ndim == 3 else fp8_dequantize(codes, sc)
        else:
            out[k] = v
    return out


def loaded_weight_bytes_fp8(ids, n_experts: int, d: int, d_ff: int, router_bytes: int,
                            n_depts: int = 0, d_ff_dept: int = 0,
                            d_ff_shared: int = 0) -> int:
    """Bytes one decode step reads with FP8 expert matrices: the router
    (E*d at router_bytes each), one byte per expert weight and a 4-byte
    scale per output row of every matrix read (gate and up rows are I long,
    down rows d)."""
    ids = np.asarray(ids).reshape(-1)
    experts = {int(e) for e in ids if 0 <= e < n_experts}

    def mat3(rows_i):  # gate, up (rows_i rows of d) and down (d rows of rows_i)
        return 3 * d * rows_i + 4 * (2 * rows_i + d)
    n = n_experts * d * router_bytes
    n += len(experts) * mat3(d_ff)
    if d_ff_shared:
        n += mat3(d_ff_shared)
    if n_depts:
        g = n_experts // n_depts
        n += len({e // g for e in experts}) * mat3(d_ff_dept)
    return n
