"""Pins of the CPU oracle against facts the pages and mathematics fix.

Nothing here compares the oracle with itself: each test checks it against a
worked example printed on the pages, a closed form, a library routine, brute
force over tiny inputs, or an invariant the method states.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


def _rand_layer(rng, d, E, I, Is=0, m=0, S=0):
    w = {"w_router": rng.normal(0, 0.3, (E, d)).astype(np.float32),
         "w_gate": rng.normal(0, 0.3, (E, I, d)).astype(np.float32),
         "w_up": rng.normal(0, 0.3, (E, I, d)).astype(np.float32),
         "w_down": rng.normal(0, 0.3, (E, d, I)).astype(np.float32)}
    if Is:
        w.update(ws_gate=rng.normal(0, 0.3, (Is, d)).astype(np.float32),
                 ws_up=rng.normal(0, 0.3, (Is, d)).astype(np.float32),
                 ws_down=rng.normal(0, 0.3, (d, Is)).astype(np.float32))
    if m:
        w.update(wd_gate=rng.normal(0, 0.3, (m, S, d)).astype(np.float32),
                 wd_up=rng.normal(0, 0.3, (m, S, d)).astype(np.float32),
                 wd_down=rng.normal(0, 0.3, (m, d, S)).astype(np.float32))
    return w


# ---------------------------------------------------------------------------
# The worked example of "MoE inference engineering, clearly explained"
# ---------------------------------------------------------------------------

def _golden():
    with open(os.path.join(GOLDEN, "worked_example.json")) as f:
        return json.load(f)


def test_worked_example_dispatch():
    g = _golden()
    ids = np.array(g["topk_ids"], np.int32)
    plan = O.dispatch(ids, g["n_experts"], np.array(g["topk_w"]))
    ex = g["expected"]
    assert plan["n_rows"] == ex["assignments"]
    assert plan["counts"].tolist() == ex["group_rows"]
    assert plan["offsets"].tolist() == ex["expert_offsets"]
    assert plan["row_token"].tolist() == ex["row_token"]
    assert plan["inv_perm"].tolist() == ex["inv_perm"]
    for e, toks in enumerate(ex["group_tokens"]):
        lo, hi = plan["offsets"][e], plan["offsets"][e + 1]
        assert plan["row_token"][lo:hi].tolist() == toks


def test_worked_example_combine():
    g = _golden()
    ids = np.array(g["topk_ids"], np.int32)
    w = np.array(g["topk_w"])
    plan = O.dispatch(ids, g["n_experts"], w)
    d = 5
    row_out = np.stack([np.full(d, float(e + 1)) for e in plan["row_expert"]])
    y = O.combine(plan, row_out, 4, 2)
    want = g["expected"]["combine_constant_rows"]["y"]
    np.testing.assert_allclose(y, np.repeat(np.array(want)[:, None], d, 1), rtol=0, atol=1e-12)
    # the page's weights of each token sum to one
    np.testing.assert_allclose(w.sum(1), 1.0, atol=1e-12)


# ---------------------------------------------------------------------------
# Top-k selection: brute force over all subsets, ties, and the 28 pairs
# ---------------------------------------------------------------------------

def _brute_topk(scores, k):
    """The unique k-subset whose every member precedes every non-member in
    the order (score desc, index asc); returned in that order."""
    E = len(scores)
    key = lambda e: (-scores[e], e)  # noqa: E731
    found = []
    for sub in itertools.combinations(range(E), k):
        rest = [e for e in range(E) if e not in sub]
        if all(key(a) < key(b) for a in sub for b in rest):
            found.append(sorted(sub, key=key))
    assert len(found) == 1
    return found[0]


@pytest.mark.parametrize("seed", range(6))
def test_topk_matches_subset_bruteforce(seed):
    rng = _rng(seed)
    E, k = 7, 3
    for _ in range(20):
        s = rng.normal(size=E).astype(np.float32)
        if seed % 2:  # force ties
            s = np.round(s, 0).astype(np.float32)
        assert O.topk_select(s[None], k)[0].tolist() == _brute_topk(s.tolist(), k)


def test_topk_all_28_pairs_by_bias():
    """Every one of the C(8,2) = 28 top-2 routes of an 8-expert layer is
    reachable and selected exactly, by a selection bias on that pair."""
    rng = _rng(1)
    d, E, k = 16, 8, 2
    x = rng.normal(0, 1, (1, d)).astype(np.float32)
    wr = rng.normal(0, 0.1, (E, d)).astype(np.float32)
    seen = set()
    for a, b in itertools.combinations(range(E), 2):
        bias = np.zeros(E, np.float32)
        bias[a] = bias[b] = 100.0
        ids, w, _, l32 = O.route(x, wr, k, O.SOFTMAX_BIAS, bias)
        assert sorted(ids[0].tolist()) == [a, b]
        seen.add((a, b))
        # weights come from the unbiased logits
        sel = l32[0, ids[0]].astype(np.float64)
        np.testing.assert_allclose(w[0], scipy.special.softmax(sel), rtol=1e-12)
    assert len(seen) == math.comb(8, 2) == 28


def test_topk_ties_lower_index_wins():
    s = np.zeros((1, 6), np.float32)
    assert O.topk_select(s, 3)[0].tolist() == [0, 1, 2]
    s = np.array([[1, 2, 2, 0, 2, 1]], np.float32)
    assert O.topk_select(s, 4)[0].tolist() == [1, 2, 4, 0]


# ---------------------------------------------------------------------------
# Routing weights against library routines and closed forms
# ---------------------------------------------------------------------------

def test_softmax_k_equals_E_is_full_softmax():
    rng = _rng(2)
    x = rng.normal(0, 1, (3, 32)).astype(np.float32)
    wr = rng.normal(0, 0.2, (8, 32)).astype(np.float32)
    ids, w, _, l32 = O.route(x, wr, 8, O.SOFTMAX)
    for t in range(3):
        full = scipy.special.softmax(l32[t].astype(np.float64))
        np.testing.assert_allclose(w[t], full[ids[t]], rtol=1e-12)
        assert list(ids[t]) == list(np.argsort(-l32[t], kind="stable"))


def test_softmax_not_renormalised_is_full_softmax_probability():
    rng = _rng(3)
    x = rng.normal(0, 1, (2, 32)).astype(np.float32)
    wr = rng.normal(0, 0.2, (16, 32)).astype(np.float32)
    ids, w, _, l32 = O.route(x, wr, 4, O.SOFTMAX, renormalize=False)
    for t in range(2):
        p = scipy.special.softmax(l32[t].astype(np.float64))
        np.testing.assert_allclose(w[t], p[ids[t]], rtol=1e-12)
        assert w[t].sum() < 1.0


def test_sigmoid_bias_routing():
    """Selection on sigmoid(l)+b; weights are the selected unbiased sigmoid
    scores normalised to sum 1 (sigmoid from scipy's expit)."""
    rng = _rng(4)
    x = rng.normal(0, 1, (4, 64)).astype(np.float32)
    wr = rng.normal(0, 0.05, (32, 64)).astype(np.float32)
    b = rng.uniform(-0.1, 0.1, 32).astype(np.float32)
    ids, w, sel, l32 = O.route(x, wr, 8, O.SIGMOID, b, route_scale=2.5)
    for t in range(4):
        s = scipy.special.expit(l32[t].astype(np.float64))
        ranked = np.lexsort((np.arange(32), -(s.astype(np.float32) + b)))
        assert ids[t].tolist() == ranked[:8].tolist()
        np.testing.assert_allclose(w[t], 2.5 * s[ids[t]] / s[ids[t]].sum(), rtol=1e-12)
        np.testing.assert_allclose(w[t].sum(), 2.5, rtol=1e-12)
    # the bias changes the selection for at least one token of this seed
    ids0 = O.topk_select(O.selection_scores(l32, O.SIGMOID, None), 8)
    assert not np.array_equal(np.sort(ids0, 1), np.sort(ids, 1))


def test_router_logits_unit_tokens_read_router_columns():
    """[DeaMoE] Eq. (2): l = W_r x.  A one-hot token x = e_c picks column c of
    W_r exactly, so l[:, e] = W_r[e, c] for every expert: a transposed,
    scaled, offset, row- or column-permuted router fails."""
    rng = _rng(21)
    E, d = 6, 10
    wr = rng.normal(0, 1, (E, d)).astype(np.float32)
    x = np.eye(d, dtype=np.float32)           # token c = e_c
    l = O.router_logits(x, wr)
    assert l.shape == (d, E) and l.dtype == np.float32
    for c in range(d):
        for e in range(E):
            assert l[c, e] == wr[e, c], (c, e)
    # a scaled one-hot token scales exactly (powers of two)
    l2 = O.router_logits(4.0 * x[3:4], wr)
    assert np.array_equal(l2[0], 4.0 * wr[:, 3])


def test_router_logits_small_integers_hand_summed():
    """Integer tokens and router rows give integer logits, every one summed
    by hand here: x = [[1, 2, 3], [-1, 0, 4]], W_r = [[1, 0, 0], [0, 1, 1],
    [2, -1, 3], [0, 0, -2]]."""
    x = np.array([[1, 2, 3], [-1, 0, 4]], np.float32)
    wr = np.array([[1, 0, 0], [0, 1, 1], [2, -1, 3], [0, 0, -2]], np.float32)
    want = np.array([[1, 2 + 3, 2 - 2 + 9, -6],
                     [-1, 0 + 4, -2 + 0 + 12, -8]], np.float32)
    assert np.array_equal(O.router_logits(x, wr), want)
    # and the logits are exactly the fp32 rounding of the exact sum: a sum
    # that cancels to 1 from 2^24-scale terms loses nothing in fp64
    xb = np.array([[16777216.0, 1.0, -16777216.0]], np.float32)
    wb = np.ones((1, 3), np.float32)
    assert O.router_logits(xb, wb)[0, 0] == 1.0


def test_sigmoid_not_renormalised_is_expit():
    """Sigmoid mode without renormalisation: each selected weight is the
    expert's own sigmoid score (scipy's expit of the logit), times the
    route scale; selection still ranks sigmoid + bias."""
    rng = _rng(22)
    x = rng.normal(0, 1, (3, 48)).astype(np.float32)
    wr = rng.normal(0, 0.1, (12, 48)).astype(np.float32)
    b = rng.uniform(-0.1, 0.1, 12).astype(np.float32)
    ids, w, _, l32 = O.route(x, wr, 4, O.SIGMOID, b, renormalize=False, route_scale=1.5)
    for t in range(3):
        s = scipy.special.expit(l32[t].astype(np.float64))
        np.testing.assert_allclose(w[t], 1.5 * s[ids[t]], rtol=1e-13)
        assert w[t].sum() != pytest.approx(1.5)   # not renormalised
        ranked = np.lexsort((np.arange(12), -(s.astype(np.float32) + b)))
        assert ids[t].tolist() == ranked[:4].tolist()


def test_zero_input_gives_zero_output_and_tied_logits():
    rng = _rng(5)
    w = _rand_layer(rng, 16, 6, 8, Is=8)
    x = np.zeros((3, 16), np.float32)
    for fn, wsum in ((O.SOFTMAX, 1 / 3), (O.SIGMOID, 1 / 3)):
        ids, rw, _, l32 = O.route(x, w["w_router"], 3, fn)
        assert np.all(l32 == 0)
        assert ids.tolist() == [[0, 1, 2]] * 3
        np.testing.assert_allclose(rw, wsum, rtol=1e-12)
        y = O.layer_bruteforce(x, w, ids, rw, 6)
        assert np.all(y == 0)


# ---------------------------------------------------------------------------
# Expert FFN against a textbook SwiGLU written with torch.nn.functional
# ---------------------------------------------------------------------------

def test_single_expert_is_textbook_swiglu():
    rng = _rng(6)
    d, I = 24, 40
    w = _rand_layer(rng, d, 1, I)
    x = rng.normal(0, 1, (3, d)).astype(np.float32)
    ids, rw, _, _ = O.route(x, w["w_router"], 1, O.SOFTMAX)
    assert np.all(ids == 0) and np.allclose(rw, 1.0)
    y = O.layer_bruteforce(x, w, ids, rw, 1)
    X = torch.tensor(x, dtype=torch.float64)
    Wg, Wu, Wd = (torch.tensor(w[n][0], dtype=torch.float64) for n in ("w_gate", "w_up", "w_down"))
    ref = torch.nn.functional.linear(
        torch.nn.functional.silu(torch.nn.functional.linear(X, Wg)) * torch.nn.functional.linear(X, Wu), Wd)
    np.testing.assert_allclose(y, ref.numpy(), rtol=1e-12, atol=1e-12)


def test_silu_matches_library():
    z = np.linspace(-30, 30, 1001)
    np.testing.assert_allclose(O.silu(z), z * scipy.special.expit(z), rtol=1e-14, atol=1e-300)


def test_shared_expert_is_added_with_weight_one():
    rng = _rng(7)
    d, E, I, Is = 16, 4, 8, 12
    w = _rand_layer(rng, d, E, I, Is=Is)
    x = rng.normal(0, 1, (2, d)).astype(np.float32)
    ids, rw, _, _ = O.route(x, w["w_router"], 2)
    with_shared = O.layer_bruteforce(x, w, ids, rw, E)
    w2 = {k: v for k, v in w.items() if not k.startswith("ws_")}
    without = O.layer_bruteforce(x, w2, ids, rw, E)
    X = torch.tensor(x, dtype=torch.float64)
    F = torch.nn.functional
    sh = F.linear(F.silu(F.linear(X, torch.tensor(w["ws_gate"], dtype=torch.float64)))
                  * F.linear(X, torch.tensor(w["ws_up"], dtype=torch.float64)),
                  torch.tensor(w["ws_down"], dtype=torch.float64))
    np.testing.assert_allclose(with_shared - without, sh.numpy(), rtol=1e-10, atol=1e-12)


# ---------------------------------------------------------------------------
# Brute force (per token, per slot) == grouped path (dispatch, experts, combine)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("seed", range(8))
def test_bruteforce_equals_grouped(seed):
    rng = _rng(100 + seed)
    E = int(rng.integers(1, 9))
    k = int(rng.integers(1, E + 1))
    T = int(rng.integers(0, 5))
    d, I = 8 * int(rng.integers(1, 4)), 8 * int(rng.integers(1, 3))
    Is = 8 if seed % 2 else 0
    w = _rand_layer(rng, d, E, I, Is=Is)
    x = rng.normal(0, 1, (T, d)).astype(np.float32)
    fn = [O.SOFTMAX, O.SIGMOID, O.SOFTMAX_BIAS][seed % 3]
    bias = rng.uniform(-0.1, 0.1, E).astype(np.float32)
    ids, rw, _, _ = O.route(x, w["w_router"], k, fn, bias)
    a = O.layer_bruteforce(x, w, ids, rw, E)
    b = O.layer_grouped(x, w, ids, rw, E)
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-12)
    plan = O.dispatch(ids, E, rw)
    # grouping keeps every assignment (no token dropping) and is a bijection
    assert plan["n_rows"] == T * k == int(plan["counts"].sum())
    assert sorted(plan["inv_perm"].tolist()) == list(range(T * k))
    for e in range(E):
        toks = plan["row_token"][plan["offsets"][e]:plan["offsets"][e + 1]]
        assert list(toks) == sorted(toks)


# ---------------------------------------------------------------------------
# Department variant: expanded per-expert form == factored department form
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("seed", range(4))
def test_department_expanded_equals_factored(seed):
    rng = _rng(200 + seed)
    d, E, m, S, P, k, T = 16, 8, 2 * (seed % 2 + 1), 24, 8, 3, 4
    w = _rand_layer(rng, d, E, P, Is=8 if seed >= 2 else 0, m=m, S=S)
    x = rng.normal(0, 1, (T, d)).astype(np.float32)
    ids, rw, _, _ = O.route(x, w["w_router"], k, [O.SOFTMAX, O.SIGMOID][seed % 2],
                            rng.uniform(-0.1, 0.1, E).astype(np.float32))
    a = O.dept_layer_expanded(x, w, ids, rw, E, m)
    b = O.dept_layer_factored(x, w, ids, rw, E, m)
    np.testing.assert_allclose(a, b, rtol=1e-10, atol=1e-12)


def test_department_one_expert_per_department_is_vanilla():
    """m = E: every department holds one expert, so the layer is a vanilla
    layer whose experts have intermediate [S ; P]."""
    rng = _rng(300)
    d, E, S, P, k, T = 16, 4, 8, 8, 2, 3
    w = _rand_layer(rng, d, E, P, m=E, S=S)
    van = {"w_router": w["w_router"],
           "w_gate": np.concatenate([w["wd_gate"], w["w_gate"]], 1),
           "w_up": np.concatenate([w["wd_up"], w["w_up"]], 1),
           "w_down": np.concatenate([w["wd_down"], w["w_down"]], 2)}
    x = rng.normal(0, 1, (T, d)).astype(np.float32)
    ids, rw, _, _ = O.route(x, w["w_router"], k)
    np.testing.assert_allclose(O.dept_layer_factored(x, w, ids, rw, E, E),
                               O.layer_bruteforce(x, van, ids, rw, E), rtol=1e-10, atol=1e-12)


def test_department_zero_private_is_weighted_department_sum():
    """Private slices zero: y_t = sum_j c_{t,j} F_j(x_t), with c_{t,j} the
    summed weights of the token's experts in department j."""
    rng = _rng(301)
    d, E, m, S, P, k, T = 16, 8, 4, 8, 8, 3, 3
    w = _rand_layer(rng, d, E, P, m=m, S=S)
    for n in ("w_gate", "w_up", "w_down"):
        w[n] = np.zeros_like(w[n])
    x = rng.normal(0, 1, (T, d)).astype(np.float32)
    ids, rw, _, _ = O.route(x, w["w_router"], k)
    y = O.dept_layer_expanded(x, w, ids, rw, E, m)
    for t in range(T):
        ref = np.zeros(d)
        for j in range(m):
            c = sum(rw[t, s] for s in range(k) if ids[t, s] // (E // m) == j)
            if c:
                ref += c * O.swiglu(x[t], w["wd_gate"][j], w["wd_up"][j], w["wd_down"][j])
        np.testing.assert_allclose(y[t], ref, rtol=1e-10, atol=1e-12)


# ---------------------------------------------------------------------------
# Output rounding: bf16 round-to-nearest-even against torch's conversion
# ---------------------------------------------------------------------------

def test_bf16_output_rounding_matches_torch():
    rng = _rng(8)
    v = np.concatenate([rng.normal(0, 1, 10000), rng.normal(0, 1e-3, 1000),
                        [1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -1.0 - 2 ** -8]])
    ours = O.cast_output(v, "bf16")
    ref = torch.tensor(v.astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(ours, ref)


# ---------------------------------------------------------------------------
# Weights loaded per step: the paper's Table 1 and Figure 2 closed forms, and
# the oracle's byte accounting against the expectation under uniform routing
# ---------------------------------------------------------------------------

# (model, k, h, hffn, n, n_dept, n', k_dept, k', FLOPs ratio, Params ratio)
TABLE1 = [
    ("DeepSeek-V3", 8, 7168, 2048, 256, 8, 864, 5, 10, 0.995, 0.996),
    ("DeepSeek-V2", 6, 5120, 1536, 160, 8, 512, 5, 10, 1.010, 1.010),
    ("Qwen3-235B-A22B", 8, 4096, 1536, 128, 8, 320, 5, 8, 1.005, 1.000),
    ("Kimi-K2", 8, 7168, 2048, 384, 16, 1280, 5, 10, 1.000, 0.994),
    ("Baseline-7B", 8, 1024, 384, 256, 8, 672, 4, 10, 1.014, 1.017),
]


@pytest.mark.parametrize("row", TABLE1, ids=[r[0] for r in TABLE1])
def test_table1_budget_ratios(row):
    """DeaMoE Table 1: params and FLOPs of the factorized department form
    (department matrices h x hffn, private A matrices hffn x hffn, router
    counted) over the baseline's.  The DeepSeek-V2 FLOPs cell does not follow
    from the printed configuration and is checked as such."""
    name, k, h, f, n, m, n2, kd, k2, flops_r, params_r = row
    p_base = n * 3 * h * f + n * h
    p_dea = m * 3 * h * f + n2 * 3 * f * f + n2 * h
    f_base = k * 3 * h * f + n * h
    f_dea = kd * 3 * h * f + k2 * 3 * f * f + n2 * h
    assert round(p_dea / p_base, 3) == pytest.approx(params_r, abs=1.5e-3)
    if name == "DeepSeek-V2":
        assert abs(f_dea / f_base - flops_r) > 0.3
    else:
        assert round(f_dea / f_base, 3) == pytest.approx(flops_r, abs=1.5e-3)


def _fig2_ratio(B, n=256, k=8, m=8, n2=864, k2=10, h=7168, f=2048):
    base = n * (1 - (1 - k / n) ** B) * 3 * h * f
    q = math.comb(n2 - n2 // m, k2) / math.comb(n2, k2)
    dea = m * (1 - q ** B) * 3 * h * f + n2 * (1 - (1 - k2 / n2) ** B) * 3 * f * f
    return dea / base


def test_fig2_loading_ratio_range():
    """DeaMoE Figure 2 / section 3.3: for the DeepSeek-V3-matched layer the
    expected weights loaded per step stay between 49.1% and 62.8% of the
    baseline's for 4 to 64 tokens."""
    r = [_fig2_ratio(B) for B in range(4, 65)]
    assert r[0] == pytest.approx(0.628, abs=1.5e-3)
    assert min(r) == pytest.approx(0.491, abs=2.5e-3)
    assert max(r) == pytest.approx(0.628, abs=1.5e-3)
    assert 1 - min(r) == pytest.approx(0.509, abs=2.5e-3)  # "up to 50.9%" fewer


@pytest.mark.parametrize("shape", ["vanilla", "dept"])
def test_loaded_bytes_expectation_under_uniform_routing(shape):
    """Mean of the oracle's per-step byte count over uniformly random routings
    equals the closed-form expectation (distinct experts n(1-(1-k/n)^B),
    distinct departments m(1-q^B))."""
    rng = _rng(9)
    if shape == "vanilla":
        E, k, d, I, m, S, B = 128, 8, 2048, 768, 0, 0, 4
    else:
        E, k, d, I, m, S, B = 64, 8, 2048, 128, 8, 1024, 4
    samples = []
    for _ in range(4000):
        ids = np.stack([rng.choice(E, k, replace=False) for _ in range(B)])
        samples.append(O.loaded_weight_bytes(ids, E, d, I, 2, m, S, include_router=False))
    samples = np.array(samples, np.float64)
    exp = E * (1 - (1 - k / E) ** B) * 3 * d * I * 2
    if m:
        q = math.comb(E - E // m, k) / math.comb(E, k)
        exp += m * (1 - q ** B) * 3 * d * S * 2
    se = samples.std() / math.sqrt(len(samples))
    assert abs(samples.mean() - exp) < 4 * se + 1e-9 * exp


def test_resident_bytes_of_layer_shapes():
    """DeepSeek-V3 experts are three [7168, 2048] matrices (about 44 MB at one
    byte per weight); 256 of them at bf16 are about 22.5 GB."""
    from moe_synth import SHAPES
    s = SHAPES["deepseek_v3_d7168_e256_i2048_s2048_top8"]
    per_expert = 3 * s.d * s.d_ff
    assert per_expert / 1e6 == pytest.approx(44.04, abs=0.01)
    assert s.n_experts * per_expert * 2 / 1e9 == pytest.approx(22.5, abs=0.1)


# ---------------------------------------------------------------------------
# Factorised DeaMoE experts (DeaMoE section 3.1 / 3.2): each pin below would
# fail for a transposed A, a sigma dropped or moved, or a department mixed up
# ---------------------------------------------------------------------------

def _rand_factorised(rng, d, E, m, f, Is=0, a_std=0.3):
    w = {"w_router": rng.normal(0, 0.3, (E, d)).astype(np.float32),
         "wd_gate": rng.normal(0, 0.3, (m, f, d)).astype(np.float32),
         "wd_up": rng.normal(0, 0.3, (m, f, d)).astype(np.float32),
         "wd_down": rng.normal(0, 0.3, (m, d, f)).astype(np.float32),   # (W_d^j)^T
         "w_gate": rng.normal(0, a_std, (E, f, f)).astype(np.float32),
         "w_up": rng.normal(0, a_std, (E, f, f)).astype(np.float32),
         "w_down": rng.normal(0, a_std, (E, f, f)).astype(np.float32)}  # (A_d^i)^T
    if Is:
        w.update(ws_gate=rng.normal(0, 0.3, (Is, d)).astype(np.float32),
                 ws_up=rng.normal(0, 0.3, (Is, d)).astype(np.float32),
                 ws_down=rng.normal(0, 0.3, (d, Is)).astype(np.float32))
    return w


def _silu_ref(z):
    return z * scipy.special.expit(z)


def test_factorised_expert_with_permutation_transforms():
    """A_g, A_u, A_d permutation matrices: every matrix product with an A
    becomes an explicit index shuffle, computed here element by element
    without any matrix product, so the placement and orientation of each A
    (A vs A^T) and of each sigma is checked."""
    rng = _rng(400)
    d, f = 6, 5
    x = rng.normal(0, 1, d)
    Wg, Wu = rng.normal(0, 0.5, (f, d)), rng.normal(0, 0.5, (f, d))
    Wd = rng.normal(0, 0.5, (f, d))                 # W_d^j in the pages' [hffn][h] form
    pg, pu, pd = rng.permutation(f), rng.permutation(f), rng.permutation(f)
    Ag, Au, Ad = np.eye(f)[pg], np.eye(f)[pu], np.eye(f)[pd]   # (A v)[r] = v[p[r]]
    # element by element
    wgx = [sum(Wg[r, c] * x[c] for c in range(d)) for r in range(f)]
    wux = [sum(Wu[r, c] * x[c] for c in range(d)) for r in range(f)]
    g_hat = [_silu_ref(_silu_ref(wgx[pg[r]])) for r in range(f)]
    u_hat = [_silu_ref(wux[pu[r]]) for r in range(f)]
    v = [g_hat[r] * u_hat[r] for r in range(f)]
    # (A_d^T v)[c] = sum_r A_d[r, c] v[r] = v[r] where pd[r] == c
    inv = np.argsort(pd)
    z = [_silu_ref(v[inv[c]]) for c in range(f)]
    y = [sum(Wd[r, c] * z[r] for r in range(f)) for c in range(d)]   # (W_d^T z)[c]
    got = O.deamoe_expert(x, Wg, Wu, Wd.T, Ag, Au, Ad.T)
    np.testing.assert_allclose(got, y, rtol=1e-12, atol=1e-14)


def test_factorised_identity_transforms_make_a_department_one_expert():
    """A = I (the identity start of section 3.4): every expert of a
    department computes the same function, W_d^T SiLU(SiLU(SiLU(W_g x)) *
    SiLU(W_u x)), and experts of different departments differ."""
    rng = _rng(401)
    d, E, m, f = 12, 6, 2, 7
    w = _rand_factorised(rng, d, E, m, f)
    for n in ("w_gate", "w_up", "w_down"):
        w[n] = np.broadcast_to(np.eye(f, dtype=np.float32), (E, f, f)).copy()
    x = rng.normal(0, 1, d)
    outs = [O.deamoe_expert(x, w["wd_gate"][e // 3], w["wd_up"][e // 3], w["wd_down"][e // 3],
                            w["w_gate"][e], w["w_up"][e], w["w_down"][e]) for e in range(E)]
    for j in range(m):
        Wg, Wu, WdT = (w["wd_gate"][j].astype(np.float64), w["wd_up"][j].astype(np.float64),
                       w["wd_down"][j].astype(np.float64))
        ref = WdT @ _silu_ref(_silu_ref(_silu_ref(Wg @ x)) * _silu_ref(Wu @ x))
        for e in range(3 * j, 3 * j + 3):
            np.testing.assert_allclose(outs[e], ref, rtol=1e-12, atol=1e-14)
    assert np.abs(outs[0] - outs[3]).max() > 1e-3


@pytest.mark.parametrize("seed", range(4))
def test_factorised_two_stage_equals_per_expert_and_precombined(seed):
    """Section 3.2's two-stage computation (department work once per token,
    then per-expert transforms) equals running every selected expert's own
    DeaMoE_i, and the GPU's pre-combined order (R17) equals both."""
    rng = _rng(410 + seed)
    d, E, m, f, k, T = 10, 12, [2, 3, 4, 6][seed], 6, 4, 5
    w = _rand_factorised(rng, d, E, m, f, Is=4 if seed % 2 else 0)
    x = rng.normal(0, 1, (T, d)).astype(np.float32)
    ids, rw, _, _ = O.route(x, w["w_router"], k, [O.SOFTMAX, O.SIGMOID][seed % 2],
                            rng.uniform(-0.1, 0.1, E).astype(np.float32))
    a = O.deamoe_layer_per_expert(x, w, ids, rw, E, m)
    b = O.deamoe_layer_two_stage(x, w, ids, rw, E, m)
    c = O.deamoe_layer_precombined(x, w, ids, rw, E, m)
    np.testing.assert_allclose(b, a, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(c, a, rtol=1e-10, atol=1e-12)


def test_factorised_loaded_bytes_reproduce_fig2():
    """The oracle's byte count of the factorised form, averaged over uniform
    routings at the DeepSeek-V3-matched configuration (8 departments, 864
    experts, k = 10, hffn = 2048, h = 7168), over the vanilla layer's count
    (256 experts, k = 8) reproduces Figure 2's ratio at 4 and 16 tokens."""
    rng = _rng(420)
    for B, n_samples in ((4, 3000), (16, 1500)):
        dea, van = [], []
        for _ in range(n_samples):
            ids = np.stack([rng.choice(864, 10, replace=False) for _ in range(B)])
            dea.append(O.loaded_weight_bytes(ids, 864, 7168, 2048, 1, 8, 2048,
                                             include_router=False, factorised=True))
            ids_v = np.stack([rng.choice(256, 8, replace=False) for _ in range(B)])
            van.append(O.loaded_weight_bytes(ids_v, 256, 7168, 2048, 1, include_router=False))
        ratio = np.mean(dea) / np.mean(van)
        assert ratio == pytest.approx(_fig2_ratio(B), rel=5e-3)


# ---------------------------------------------------------------------------
# Department-limited top-k (DeaMoE section 3.4: k_dept caps the departments a
# token activates)
# ---------------------------------------------------------------------------

def test_grouped_topk_hand_example():
    """12 experts in 3 departments of 4.  Plain top-3 takes experts 0, 5 and
    9 (one per department); with k_dept = 2 department 2 (best score 0.6)
    loses to departments 0 (0.9) and 1 (0.8), so the picks are 0, 5, then
    the best remaining in departments 0-1: expert 1 (0.5) over 6 (0.4)."""
    sel = np.array([[0.9, 0.5, 0.1, 0.0, 0.2, 0.8, 0.4, 0.3, 0.1, 0.6, 0.2, 0.05]],
                   np.float32)
    assert O.topk_select(sel, 3).tolist() == [[0, 5, 9]]
    assert O.topk_select_grouped(sel, 3, 3, 2).tolist() == [[0, 5, 1]]
    assert O.topk_select_grouped(sel, 3, 3, 1).tolist() == [[0, 1, 2]]
    # department ties go to the lower index: departments 1 and 2 both best at 0.8
    sel2 = sel.copy()
    sel2[0, 9] = 0.8
    assert O.topk_select_grouped(sel2, 2, 3, 2).tolist() == [[0, 5]]
    sel2[0, 0] = 0.0
    assert O.topk_select_grouped(sel2, 2, 3, 1).tolist() == [[5, 6]]


@pytest.mark.parametrize("seed", range(3))
def test_grouped_topk_properties(seed):
    """Random scores: k_dept = m is the plain top-k; otherwise the picks span
    at most k_dept departments, always include the overall best expert, and
    equal a brute force over every set of k_dept departments (the set whose
    best score tuple is largest)."""
    rng = _rng(500 + seed)
    E, m, k, T = 24, 6, 5, 8
    g = E // m
    sel = rng.normal(0, 1, (T, E)).astype(np.float32)
    assert np.array_equal(O.topk_select_grouped(sel, k, m, m), O.topk_select(sel, k))
    for kd in (2, 3):
        ids = O.topk_select_grouped(sel, k, m, kd)
        for t in range(T):
            assert len({int(e) // g for e in ids[t]}) <= kd
            assert int(np.argmax(sel[t])) in ids[t]
            best = max(itertools.combinations(range(m), kd),
                       key=lambda D: (sorted((sel[t, j * g:(j + 1) * g].max() for j in D),
                                             reverse=True), [-j for j in D]))
            pool = [e for e in range(E) if e // g in best]
            want = sorted(pool, key=lambda e: (-sel[t, e], e))[:k]
            assert ids[t].tolist() == want


# ---------------------------------------------------------------------------
# Strict department coverage (DeaMoE appendix: enforcing k_dept coverage)
# ---------------------------------------------------------------------------

def test_strict_coverage_hand_example():
    """12 experts in 3 departments of 4, k = 4, k_dept = 3.  The top 4 are
    experts 0, 1, 2 (department 0) and 4 (department 1), two departments.
    Department 2's best, expert 8 (0.6), enters; the lowest-ranked expert,
    4, is the only one of department 1 and stays, so 2 leaves."""
    sel = np.array([[0.9, 0.85, 0.8, 0.1, 0.7, 0.2, 0.1, 0.0, 0.6, 0.5, 0.3, 0.2]],
                   np.float32)
    assert O.topk_select_grouped(sel, 4, 3, 3).tolist() == [[0, 1, 2, 4]]
    assert O.topk_select_strict(sel, 4, 3, 3).tolist() == [[0, 1, 4, 8]]
    # k_dept = 2: departments 0 and 1 are chosen and already covered
    assert O.topk_select_strict(sel, 4, 3, 2).tolist() == [[0, 1, 2, 4]]
    # k = 3, k_dept = 2: the top 3 lie in department 0 alone; department
    # 1's best (4), not department 2's, enters in place of expert 2
    assert O.topk_select_grouped(sel, 3, 3, 2).tolist() == [[0, 1, 2]]
    assert O.topk_select_strict(sel, 3, 3, 2).tolist() == [[0, 1, 4]]
    # k = k_dept = 3: one expert per department
    assert O.topk_select_strict(sel, 3, 3, 3).tolist() == [[0, 4, 8]]
    with pytest.raises(ValueError):
        O.topk_select_strict(sel, 2, 3, 3)


@pytest.mark.parametrize("seed", range(3))
def test_strict_coverage_properties(seed):
    """Random scores with few departments per token: exactly k_dept departments
    are covered, all among R18's chosen departments; the result equals R18's
    whenever that already covers k_dept; otherwise k - (k_dept - covered) of
    R18's experts stay, the highest ranked of each department among them, and
    each entering expert is the best of its department; slots are in
    (score desc, index asc) order."""
    rng = _rng(600 + seed)
    E, m, T = 48, 4, 40
    g = E // m
    sel = rng.normal(0, 1, (T, E)).astype(np.float32)
    swaps = 0
    for k, kd in ((6, 3), (4, 4), (5, 2), (3, 3)):
        grouped = O.topk_select_grouped(sel, k, m, kd)
        strict = O.topk_select_strict(sel, k, m, kd)
        for t in range(T):
            s_row, g_row = strict[t].tolist(), grouped[t].tolist()
            dscore = sel[t].reshape(m, g).max(axis=1)
            chosen = sorted(range(m), key=lambda j: (-dscore[j], j))[:kd]
            assert {e // g for e in s_row} == set(chosen)
            assert s_row == sorted(s_row, key=lambda e: (-sel[t, e], e))
            cov = len({e // g for e in g_row})
            if cov == kd:
                assert s_row == g_row
                continue
            swaps += 1
            kept = [e for e in g_row if e in s_row]
            assert len(kept) == k - (kd - cov)
            # removal runs from the bottom of the ranking, so the kept
            # experts are R18's top ones once per-department leaders count
            leaders = {min((e for e in g_row if e // g == j), key=g_row.index)
                       for j in {e // g for e in g_row}}
            assert leaders <= set(kept)
            for e in set(s_row) - set(g_row):
                assert sel[t, e] == dscore[e // g]
                assert e == (e // g) * g + int(np.argmax(sel[t, (e // g) * g:(e // g + 1) * g]))
    assert swaps > 0


def test_strict_coverage_route_weights():
    """Through route(): the weights are the renormalised softmax of the final
    selection's logits and sum to route_scale."""
    rng = _rng(700)
    E, m, d, T, k, kd = 32, 4, 16, 6, 4, 3
    x = rng.normal(0, 1, (T, d)).astype(np.float32)
    wr = rng.normal(0, 0.5, (E, d)).astype(np.float32)
    ids, w, sel, l32 = O.route(x, wr, k, O.SOFTMAX, None, True, 1.0, m, kd, strict=True)
    assert np.array_equal(ids, O.topk_select_strict(sel, k, m, kd))
    for t in range(T):
        e = np.exp(l32[t, ids[t]].astype(np.float64) - l32[t, ids[t]].max())
        np.testing.assert_allclose(w[t], e / e.sum(), rtol=1e-12)


# ---------------------------------------------------------------------------
# FP8 expert weights: OCP E4M3 codes with one fp32 scale per output row.
# The decoder is pinned to the format's definition (named values, structure)
# and to torch's float8_e4m3fn conversion; the dequantized layer to a closed
# form.
# ---------------------------------------------------------------------------

def test_fp8_decode_named_values():
    """Values the E4M3 definition fixes: zero and negative zero, the smallest
    subnormal 2^-9 and the largest 7 * 2^-9, the smallest normal 2^-6, 1.0,
    1.5, 2.0, the exponent-15 codes that are finite (256 .. 448, no
    infinities), and the two NaN codes."""
    v = O.fp8_e4m3_decode(np.arange(256))
    named = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6,
             0x38: 1.0, 0x3C: 1.5, 0x40: 2.0, 0x77: 240.0, 0x78: 256.0,
             0x7E: 448.0, 0xB8: -1.0, 0xFE: -448.0, 0x81: -(2.0 ** -9)}
    for c, want in named.items():
        assert v[c] == want, hex(c)
    assert v[0x80] == 0.0 and np.signbit(v[0x80])
    assert np.isnan(v[0x7F]) and np.isnan(v[0xFF])
    assert np.isfinite(v).sum() == 254


def test_fp8_decode_structure():
    """Positive codes 0x00..0x7E increase strictly, negative codes mirror
    them, every finite value is an integer multiple of 2^-9, and inside each
    binade (exponent field E >= 1) the spacing is 2^(E-10)."""
    v = O.fp8_e4m3_decode(np.arange(256))
    pos = v[:0x7F]
    assert np.all(np.diff(pos) > 0)
    assert np.array_equal(v[0x80:0xFF], -pos)
    fin = v[np.isfinite(v)]
    assert np.array_equal(fin * 512.0, np.round(fin * 512.0))
    for e in range(1, 16):
        codes = [(e << 3) | m for m in range(8) if ((e << 3) | m) < 0x7F]
        steps = np.diff(v[codes])
        assert np.all(steps == 2.0 ** (e - 10)), e


def test_fp8_decode_matches_torch_float8_e4m3fn():
    """Every code against torch's float8_e4m3fn -> float32 conversion."""
    if not hasattr(torch, "float8_e4m3fn"):
        pytest.skip("torch has no float8_e4m3fn")
    t = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float32)
    ref = t.double().numpy()
    v = O.fp8_e4m3_decode(np.arange(256))
    assert np.array_equal(np.isnan(v), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(v[ok], ref[ok])
    assert np.array_equal(np.signbit(v[ok]), np.signbit(ref[ok]))


def test_fp8_dequantize_scales_rows():
    """Each output row takes its own scale: on a non-square [2][3][5] code
    array with a distinct scale per (matrix, row), W[e][r][c] = s[e][r] *
    value(code[e][r][c]) element by element (a column-wise or transposed
    scale fails the shape check or the values)."""
    rng = _rng(3)
    codes = rng.integers(0, 0x7F, (2, 3, 5)).astype(np.uint8)
    codes[1] |= 0x80  # negative half
    s = np.array([[0.5, 2.0, 3.0], [0.25, 8.0, 1.5]])
    W = O.fp8_dequantize(codes, s)
    for e in range(2):
        for r in range(3):
            for c in range(5):
                assert W[e, r, c] == s[e, r] * O.fp8_e4m3_decode(codes[e, r, c])
    with pytest.raises(AssertionError):
        O.fp8_dequantize(codes, s.T)


def test_fp8_layer_with_unit_codes_is_closed_form():
    """Every expert code 0x38 (1.0): gate row i is g_i * (1, ..., 1) with g_i
    its scale, so expert e gives o_c = sd_c * sum_i SiLU(sg_i S) su_i S with
    S = sum(x); the layer output is the routing-weighted sum of those, plus
    the shared expert's own closed form."""
    rng = _rng(5)
    d, E, I, Is, k, T = 24, 5, 16, 8, 2, 3
    x = rng.normal(0, 0.3, (T, d))
    codes = lambda *sh: np.full(sh, 0x38, np.uint8)  # noqa: E731
    w = {"w_router": rng.normal(0, 0.3, (E, d)),
         "w_gate": codes(E, I, d), "w_up": codes(E, I, d), "w_down": codes(E, d, I),
         "ws_gate": codes(Is, d), "ws_up": codes(Is, d), "ws_down": codes(d, Is),
         "w_gate_scale": rng.uniform(0.01, 0.1, (E, I)), "w_up_scale": rng.uniform(0.01, 0.1, (E, I)),
         "w_down_scale": rng.uniform(0.01, 0.1, (E, d)),
         "ws_gate_scale": rng.uniform(0.01, 0.1, Is), "ws_up_scale": rng.uniform(0.01, 0.1, Is),
         "ws_down_scale": rng.uniform(0.01, 0.1, d)}
    wd = O.dequantize_layer(w)
    ids, tw, _, _ = O.route(x, w["w_router"], k)
    y = O.layer_bruteforce(x, wd, ids, tw, E)
    for t in range(T):
        S = x[t].sum()
        want = np.zeros(d)
        for j in range(k):
            e = ids[t, j]
            h = _silu_ref(w["w_gate_scale"][e] * S) * (w["w_up_scale"][e] * S)
            want += tw[t, j] * w["w_down_scale"][e] * h.sum()
        hs = _silu_ref(w["ws_gate_scale"] * S) * (w["ws_up_scale"] * S)
        want += w["ws_down_scale"] * hs.sum()
        np.testing.assert_allclose(y[t], want, rtol=1e-12, atol=1e-15)


def test_fp8_loaded_bytes_of_a_deepseek_v3_expert():
    """[DeaMoE] section 2.2: a DeepSeek-V3 expert in FP8 is about 44 MB.
    One byte per weight of its three [7168, 2048] matrices plus a 4-byte
    scale per output row (2048 + 2048 + 7168 rows) gives 44.09 MB; a step that
    selects one expert reads that plus the router."""
    from moe_synth import SHAPES
    s = SHAPES["deepseek_v3_d7168_e256_i2048_s2048_top8"]
    one = O.loaded_weight_bytes_fp8([[3]], s.n_experts, s.d, s.d_ff, router_bytes=2)
    router = s.n_experts * s.d * 2
    assert (one - router) == 3 * 7168 * 2048 + 4 * (2 * 2048 + 7168)
    assert (one - router) / 1e6 == pytest.approx(44.09, abs=0.01)
    # two distinct experts, the shared expert and a department slice each once
    # (12 experts in 2 departments of 6: experts 3 and 9 sit in different ones)
    two = O.loaded_weight_bytes_fp8([[3, 9], [9, 3]], 12, 16, 4, router_bytes=2,
                                    n_depts=2, d_ff_dept=8, d_ff_shared=8)
    mat3 = lambda r: 3 * 16 * r + 4 * (2 * r + 16)  # noqa: E731
    assert two == 12 * 16 * 2 + 2 * mat3(4) + mat3(8) + 2 * mat3(8)


# ---------------------------------------------------------------------------
# Per-step routing load ("Sequence-Level and Batch-Level Expert Routing
# Balance Metrics": max expert count over the mean count of the routed
# experts)
# ---------------------------------------------------------------------------

def test_load_stats_of_the_worked_example():
    """The worked example's groups hold 3, 2, 2 and 1 rows: the mean over the
    four routed experts is 2 and the largest is 3, so the ratio is 1.5."""
    g = _golden()
    st = O.expert_load_stats(np.array(g["topk_ids"]), g["n_experts"])
    assert st["counts"] == g["expected"]["group_rows"] == [3, 2, 2, 1]
    assert st["n_assignments"] == 8 and st["mean"] == 2.0 and st["max"] == 3
    assert st["imbalance_ratio"] == 1.5
    assert st["n_active_experts"] == 4


def test_load_stats_closed_forms():
    # perfectly balanced: every expert once -> ratio 1
    E = 16
    st = O.expert_load_stats(np.arange(E).reshape(4, 4), E)
    assert st["imbalance_ratio"] == 1.0 and st["n_active_experts"] == E
    # one hot expert taking every assignment -> ratio N_r (mean = total / N_r)
    st = O.expert_load_stats(np.full((8, 1), 5), E)
    assert st["imbalance_ratio"] == E and st["counts"][5] == 8
    assert st["n_active_experts"] == 1
    # the mean divides by every routed expert, active or not: 2 of 8 used
    st = O.expert_load_stats(np.array([[0, 1], [0, 1], [0, 2]]), 8)
    assert st["mean"] == 6 / 8 and st["imbalance_ratio"] == 3 / (6 / 8)
    # departments of 4: experts 0..3 -> department 0, 4..7 -> 1
    st = O.expert_load_stats(np.array([[0, 5], [1, 3]]), 8, n_depts=2)
    assert st["n_active_depts"] == 2
    st = O.expert_load_stats(np.array([[0, 2], [1, 3]]), 8, n_depts=2)
    assert st["n_active_depts"] == 1
    # nothing assigned (ids outside [0, E) are dropped)
    st = O.expert_load_stats(np.array([[-1, 9]]), 8)
    assert st["imbalance_ratio"] == 0.0 and st["n_assignments"] == 0
