"""Parity of the HIP path with the CPU oracle, through the C ABI, on seeded
inputs of every layer shape: router and top-k, dispatch plan, expert FFN,
combine and the fused decode step; ties, ragged shapes and edge cases."""
from __future__ import annotations

import json
import os

import numpy as np
import pytest
import torch

import moe_layer_decode_amd as M
import moe_synth
import oracle as O
from _util import (TAU, TOL_FACTORISED, assert_close, desc_of, gpu_ids_from_plan, oracle_route, reference_ids,
                   select, spread_tokens, to_np)

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
TINY = "tiny_d256_e8_i128_top2"
QWEN = "qwen3_30b_a3b_d2048_e128_i768_top8"
DSV3 = "deepseek_v3_d7168_e256_i2048_s2048_top8"
DEA7 = "deamoe_7b_d2048_e64_m8_s1024_p128_top8"
DEAV3 = "deamoe_dsv3_d7168_e256_m32_s1792_p256_top8"
PAPER = "deamoe_paper_dsv3_d7168_e864_m8_h2048_top10"
# Small factorised layers (DeaMoE section 3.1) the oracle runs in full: fp32
# with ragged sizes, and bf16 with a shared expert, sigmoid routing and
# batches that give large groups of both sizes (T = 20 > 16).
FACT = {
    "fact_f32_d264_e16_m4_h72_top4": moe_synth.LayerShape(
        name="fact_f32_d264_e16_m4_h72_top4", d=264, n_experts=16, top_k=4, d_ff=72,
        n_depts=4, d_ff_dept=72, dept_form="factorised", dtype="f32", w_std=0.05,
        batches=(1, 3, 8)),
    "fact_bf16_d1024_e32_m4_h256_top6": moe_synth.LayerShape(
        name="fact_bf16_d1024_e32_m4_h256_top6", d=1024, n_experts=32, top_k=6, d_ff=256,
        n_depts=4, d_ff_dept=256, d_ff_shared=256, dept_form="factorised", score="sigmoid",
        bias_range=0.1, batches=(1, 5, 20)),
    # department-limited routing (each token within k_dept = 2 of 4 departments)
    "fact_bf16_d1024_e32_m4_h256_top6_kd2": moe_synth.LayerShape(
        name="fact_bf16_d1024_e32_m4_h256_top6_kd2", d=1024, n_experts=32, top_k=6, d_ff=256,
        n_depts=4, d_ff_dept=256, dept_form="factorised", k_dept=2, batches=(1, 5, 20)),
    # ... and exactly k_dept = 3 departments per token (strict coverage)
    "fact_bf16_d1024_e32_m4_h256_top6_kd3s": moe_synth.LayerShape(
        name="fact_bf16_d1024_e32_m4_h256_top6_kd3s", d=1024, n_experts=32, top_k=6, d_ff=256,
        n_depts=4, d_ff_dept=256, dept_form="factorised", k_dept=3, dept_strict=True,
        score="softmax_bias", bias_range=0.1, batches=(1, 5, 20)),
}
# Small FP8 layers (E4M3 expert codes, per-row scales) the oracle runs in
# full: department slices with a shared expert, rows of one to several
# 16-code steps, batches whose groups exceed four rows (T = 9), and batches
# past 16 tokens (T = 20), which take the matrix-core tiles with ragged last
# tiles (48, 208 and 32 rows; 1040 columns) and ragged last K steps.
FP8 = {
    "fp8_d1040_e12_m3_s208_i48_sh32_top4": moe_synth.LayerShape(
        name="fp8_d1040_e12_m3_s208_i48_sh32_top4", d=1040, n_experts=12, top_k=4, d_ff=48,
        n_depts=3, d_ff_dept=208, d_ff_shared=32, score="sigmoid", bias_range=0.1,
        expert_dtype="fp8", batches=(1, 4, 9, 20)),
    "fp8_d512_e6_i1040_top3": moe_synth.LayerShape(
        name="fp8_d512_e6_i1040_top3", d=512, n_experts=6, top_k=3, d_ff=1040,
        expert_dtype="fp8", batches=(1, 3, 9, 20)),
    # rows long enough that the gate/up stages two tokens per chunk, so groups
    # of three and four rows (tokens carried in the descriptor) span chunks
    "fp8_d3088_e6_i96_top3": moe_synth.LayerShape(
        name="fp8_d3088_e6_i96_top3", d=3088, n_experts=6, top_k=3, d_ff=96,
        expert_dtype="fp8", batches=(1, 4, 9)),
}
SH = {**moe_synth.SHAPES, **FACT, **FP8}
GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_example.json")


def setup_module(module):
    M.lib()  # fail loudly if the HIP library is missing


_LAYERS = {}


def gpu_layer(name, seed):
    """Whole layer on the device (cached: the large shapes take seconds)."""
    key = (name, seed)
    if key not in _LAYERS:
        if len(_LAYERS) >= 2:  # keep device memory bounded
            _LAYERS.clear()
            torch.cuda.empty_cache()
        _LAYERS[key] = moe_synth.make_layer(SH[name], seed, DEV)
    return _LAYERS[key]


# ---------------------------------------------------------------------------
# Router: top-k ids bit-exact, weights, selection scores
# ---------------------------------------------------------------------------

def run_route(desc, x, w, T, with_sel=True):
    k, E = desc.top_k, desc.n_experts
    ids = torch.full((T, k), -7, dtype=torch.int32, device=DEV)
    tw = torch.full((T, k), -7.0, dtype=torch.float32, device=DEV)
    sel = torch.full((T, E), -7.0, dtype=torch.float32, device=DEV) if with_sel else None
    ws = M.alloc_workspace(desc, DEV)
    M.moe_route(desc, x, w["w_router"], w.get("router_bias"), ids, tw, ws, sel)
    torch.cuda.synchronize()
    return ids.cpu().numpy(), tw.cpu().numpy().astype(np.float64), (None if sel is None else sel.cpu().numpy())


@pytest.mark.parametrize("name", [TINY, QWEN, DSV3, DEA7, DEAV3, PAPER])
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_route_parity(name, seed):
    shape = SH[name]
    w = moe_synth.make_layer(shape, seed, DEV, router_only=True)
    Tmax = max(shape.batches)
    desc = desc_of(shape)
    xall = moe_synth.make_tokens(shape, seed, Tmax, DEV)
    o_ids_all, o_w_all, o_sel_all, o_l32 = oracle_route(shape, xall.cpu(), {k: v.cpu() for k, v in w.items()})
    near_total = 0
    for T in shape.batches:
        x = xall[:T].contiguous()
        g_ids, g_w, g_sel = run_route(desc, x, w, T)
        # selection on the GPU's own scores is exact: same ids, same slot order
        assert np.array_equal(select(g_sel, shape), g_ids)
        # the scores agree with the oracle's to tau
        o_sel = o_sel_all[:T]
        tol = TAU * np.maximum(1.0, np.abs(o_sel))
        assert np.all(np.abs(g_sel.astype(np.float64) - o_sel) <= tol)
        # the committed seeds have no near-tie token up to 32 tokens: there
        # the ids are the oracle's bit for bit; past 64 tokens the few
        # near-ties take the GPU's choice and are reported
        ids, near = reference_ids(o_ids_all[:T], o_sel, g_ids, shape.top_k,
                                  shape.n_depts, shape.k_dept, allow_near=T >= 64)
        near_total += int(near.sum())
        # weights of the selected experts, from the oracle's logits
        o_w = O.routing_weights(o_l32[:T], g_ids, shape.score, shape.renormalize, shape.route_scale)
        np.testing.assert_allclose(g_w, o_w, rtol=0, atol=1e-5)
        if shape.renormalize:
            np.testing.assert_allclose(g_w.sum(1), shape.route_scale, atol=1e-5)
    print(f"{name} seed {seed}: near-tie tokens {near_total}")


@pytest.mark.parametrize("score,dtype,d,T,E", [
    ("softmax", "f32", 264, 5, 96), ("sigmoid", "f32", 264, 5, 96),
    ("softmax_bias", "f32", 264, 5, 96),
    # bf16 takes the matrix-core router: a ragged K split (some K pieces
    # empty), at T = 20 a second, partly filled token tile, and at E = 330 a
    # ragged last expert tile with fewer partial-logit planes
    ("softmax", "bf16", 1032, 5, 96), ("sigmoid", "bf16", 1032, 20, 96),
    ("softmax_bias", "bf16", 264, 20, 96), ("softmax", "bf16", 2056, 20, 330)])
def test_route_ties_go_to_lower_index(score, dtype, d, T, E):
    """Duplicated router rows give bitwise-equal scores; the lower expert index
    takes the earlier slot.  An all-zero router ties every expert."""
    k = 6
    g = torch.Generator().manual_seed(3)
    wr = (torch.randn(E, d, generator=g) * 0.05)
    for a, b in ((3, 70), (10, 11), (40, 95)):
        wr[b] = wr[a]
    x = torch.randn(T, d, generator=g)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    wr, x = wr.to(tdt), x.to(tdt)
    bias = torch.zeros(E) if score != "softmax" else None
    desc = M.layer_desc(d, E, k, 64, score=score, dtype=dtype, max_tokens=T)
    w = {"w_router": wr.to(DEV), "router_bias": None if bias is None else bias.to(DEV)}
    g_ids, g_w, g_sel = run_route(desc, x.to(DEV), w, T)
    for a, b in ((3, 70), (10, 11), (40, 95)):
        assert np.array_equal(g_sel[:, a], g_sel[:, b])
    assert np.array_equal(O.topk_select(g_sel, k), g_ids)
    for t in range(T):
        ids = list(g_ids[t])
        for a, b in ((3, 70), (10, 11), (40, 95)):
            if b in ids:
                assert a in ids and ids.index(a) < ids.index(b)
    # all-zero router: experts 0..k-1, equal weights
    w0 = {"w_router": torch.zeros(E, d, dtype=tdt, device=DEV), "router_bias": w["router_bias"]}
    g_ids, g_w, _ = run_route(desc, x.to(DEV), w0, T)
    assert g_ids.tolist() == [list(range(k))] * T
    np.testing.assert_allclose(g_w, 1.0 / k, atol=1e-6)
    if score != "softmax":
        # zero logits: selection follows the bias alone
        bias2 = torch.zeros(E)
        bias2[[5, 17, 33, 60, 61, 90]] = torch.tensor([0.3, 0.9, 0.1, 0.5, 0.7, 0.2])
        w0["router_bias"] = bias2.to(DEV)
        g_ids, g_w, _ = run_route(desc, x.to(DEV), w0, T)
        assert g_ids.tolist() == [[17, 61, 60, 5, 90, 33]] * T
        np.testing.assert_allclose(g_w, 1.0 / k, atol=1e-6)


@pytest.mark.parametrize("score,dtype,d,T,E,m,k,kd", [
    ("softmax", "f32", 264, 5, 96, 8, 6, 2), ("sigmoid", "f32", 264, 7, 96, 4, 6, 1),
    ("softmax_bias", "bf16", 1032, 20, 96, 12, 6, 3),
    # one expert per department: department and expert ranking coincide
    ("softmax", "bf16", 264, 5, 64, 64, 4, 5),
    # k fills the chosen departments exactly
    ("sigmoid", "bf16", 2056, 20, 330, 22, 30, 2),
    ("softmax", "bf16", 7168, 16, 864, 8, 10, 5)])
def test_route_grouped_parity(score, dtype, d, T, E, m, k, kd):
    """Department-limited top-k: the ids are the oracle's grouped selection of
    the GPU's own scores (bit-exact, slot order included); every token's
    experts lie in at most k_dept departments; the weights are those of the
    selected logits."""
    g = torch.Generator().manual_seed(11)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    wr = (torch.randn(E, d, generator=g) * 0.05).to(tdt)
    x = torch.randn(T, d, generator=g).to(tdt)
    bias = (torch.rand(E, generator=g) * 0.2 - 0.1) if score != "softmax" else None
    desc = M.layer_desc(d, E, k, 64, score=score, dtype=dtype, max_tokens=T, n_depts=m,
                        d_ff_dept=64, k_dept=kd)
    w = {"w_router": wr.to(DEV), "router_bias": None if bias is None else bias.to(DEV)}
    g_ids, g_w, g_sel = run_route(desc, x.to(DEV), w, T)
    assert np.array_equal(O.topk_select_grouped(g_sel, k, m, kd), g_ids)
    G = E // m
    assert all(len({int(e) // G for e in row}) <= kd for row in g_ids)
    o_ids, _, o_sel, o_l32 = O.route(x, wr, k, score, bias, True, 1.0, m, kd)
    tol = TAU * np.maximum(1.0, np.abs(o_sel))
    assert np.all(np.abs(g_sel.astype(np.float64) - o_sel) <= tol)
    ids, _ = reference_ids(o_ids, o_sel, g_ids, k, m, kd, allow_near=True)
    np.testing.assert_allclose(g_w, O.routing_weights(o_l32, g_ids, score), atol=1e-5)


@pytest.mark.parametrize("score,dtype,d,T,E,m,k,kd", [
    ("softmax", "f32", 264, 9, 96, 4, 6, 3), ("sigmoid", "bf16", 1032, 20, 96, 4, 6, 4),
    ("softmax_bias", "bf16", 264, 20, 128, 8, 5, 5),
    # many departments: the paper's shape, and one expert per department
    ("softmax", "bf16", 7168, 16, 864, 8, 10, 5), ("softmax", "bf16", 264, 5, 64, 64, 6, 6)])
def test_route_strict_parity(score, dtype, d, T, E, m, k, kd):
    """Strict department coverage: the ids are the oracle's strict selection
    of the GPU's own scores (bit-exact, slot order included), every token
    covers exactly k_dept departments, and the weights are those of the
    final selection's logits."""
    g = torch.Generator().manual_seed(13)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    wr = (torch.randn(E, d, generator=g) * 0.05).to(tdt)
    x = torch.randn(T, d, generator=g).to(tdt)
    bias = (torch.rand(E, generator=g) * 0.2 - 0.1) if score != "softmax" else None
    desc = M.layer_desc(d, E, k, 64, score=score, dtype=dtype, max_tokens=T, n_depts=m,
                        d_ff_dept=64, k_dept=kd, dept_strict=True)
    w = {"w_router": wr.to(DEV), "router_bias": None if bias is None else bias.to(DEV)}
    g_ids, g_w, g_sel = run_route(desc, x.to(DEV), w, T)
    assert np.array_equal(O.topk_select_strict(g_sel, k, m, kd), g_ids)
    G = E // m
    assert all(len({int(e) // G for e in row}) == kd for row in g_ids)
    swaps = int((O.topk_select_grouped(g_sel, k, m, kd) != g_ids).any(axis=1).sum())
    o_ids, _, o_sel, o_l32 = O.route(x, wr, k, score, bias, True, 1.0, m, kd, strict=True)
    tol = TAU * np.maximum(1.0, np.abs(o_sel))
    assert np.all(np.abs(g_sel.astype(np.float64) - o_sel) <= tol)
    np.testing.assert_allclose(g_w, O.routing_weights(o_l32, g_ids, score), atol=1e-5)
    print(f"strict E={E} m={m} k={k} k_dept={kd}: {swaps} of {T} tokens swapped")


def test_route_strict_all_ties():
    """An all-zero router ties everything: departments 0..2 are chosen, the
    top 6 are experts 0..5 of department 0 alone, and the strict swaps bring
    in experts 24 and 48 in place of 5 and 4."""
    E, m, d, T, k, kd = 96, 4, 264, 3, 6, 3
    desc = M.layer_desc(d, E, k, 64, dtype="bf16", max_tokens=T, n_depts=m, d_ff_dept=64,
                        k_dept=kd, dept_strict=True)
    x = torch.randn(T, d, generator=torch.Generator().manual_seed(2)).to(torch.bfloat16)
    w0 = {"w_router": torch.zeros(E, d, dtype=torch.bfloat16, device=DEV)}
    g_ids, g_w, _ = run_route(desc, x.to(DEV), w0, T)
    assert g_ids.tolist() == [[0, 1, 2, 3, 24, 48]] * T
    np.testing.assert_allclose(g_w, 1.0 / k, atol=1e-6)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_route_grouped_ties(dtype):
    """Equal department scores go to the lower department; an all-zero router
    ties everything and gives experts 0..k-1; a bias alone picks departments
    by their best biased expert."""
    E, m, d, T, k, kd = 96, 8, 264, 4, 5, 2
    G = E // m
    g = torch.Generator().manual_seed(5)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    wr = torch.randn(E, d, generator=g) * 0.05
    x = torch.randn(T, d, generator=g)
    # department 6's best expert copies each token's overall best expert
    # row set: copy a whole department, so both tie on their best score
    wr[6 * G:7 * G] = wr[1 * G:2 * G]
    wr, x = wr.to(tdt), x.to(tdt)
    desc = M.layer_desc(d, E, k, 64, score="softmax_bias", dtype=dtype, max_tokens=T,
                        n_depts=m, d_ff_dept=64, k_dept=kd)
    w = {"w_router": wr.to(DEV), "router_bias": torch.zeros(E, device=DEV)}
    g_ids, _, g_sel = run_route(desc, x.to(DEV), w, T)
    assert np.array_equal(g_sel[:, G:2 * G], g_sel[:, 6 * G:7 * G])
    assert np.array_equal(O.topk_select_grouped(g_sel, k, m, kd), g_ids)
    for row in g_ids:
        assert not any(6 * G <= e < 7 * G for e in row) or any(G <= e < 2 * G for e in row)
    w0 = {"w_router": torch.zeros(E, d, dtype=tdt, device=DEV),
          "router_bias": torch.zeros(E, device=DEV)}
    g_ids, g_w, _ = run_route(desc, x.to(DEV), w0, T)
    assert g_ids.tolist() == [list(range(k))] * T
    np.testing.assert_allclose(g_w, 1.0 / k, atol=1e-6)
    # zero logits, bias on experts of departments 7 (0.9), 3 (0.8, 0.1), 5 (0.85):
    # departments 7 and 5 win; then their experts by bias, then the lowest index
    b = torch.zeros(E)
    b[7 * G + 4], b[3 * G], b[3 * G + 1], b[5 * G + 2] = 0.9, 0.8, 0.1, 0.85
    w0["router_bias"] = b.to(DEV)
    g_ids, _, _ = run_route(desc, x.to(DEV), w0, T)
    assert g_ids.tolist() == [[7 * G + 4, 5 * G + 2, 5 * G, 5 * G + 1, 5 * G + 3]] * T


def test_route_k_equals_E_and_not_renormalised():
    E, d, T = 8, 256, 4
    g = torch.Generator().manual_seed(4)
    wr, x = torch.randn(E, d, generator=g) * 0.05, torch.randn(T, d, generator=g)
    for k, renorm, score in ((8, True, "softmax"), (3, False, "softmax"), (3, False, "sigmoid")):
        desc = M.layer_desc(d, E, k, 64, dtype="f32", max_tokens=T, renormalize=renorm,
                            score=score)
        g_ids, g_w, _ = run_route(desc, x.to(DEV), {"w_router": wr.to(DEV)}, T)
        o_ids, o_w, _, _ = O.route(x, wr, k, score, None, renorm)
        assert np.array_equal(g_ids, o_ids)
        np.testing.assert_allclose(g_w, o_w, atol=1e-6)


# ---------------------------------------------------------------------------
# Dispatch: bit-exact plan
# ---------------------------------------------------------------------------

def run_dispatch(desc, ids, tw):
    ws = M.alloc_workspace(desc, DEV)
    plan = M.moe_dispatch(desc, torch.as_tensor(ids, dtype=torch.int32).to(DEV).contiguous(),
                          torch.as_tensor(tw, dtype=torch.float32).to(DEV).contiguous(), ws)
    return plan, ws, M.plan_to_host(desc, plan, ws)


def assert_plan_equal(g, o, m):
    for key in ("counts", "offsets", "row_token", "row_slot", "row_expert", "inv_perm", "active"):
        assert np.array_equal(g[key], np.asarray(o[key])), key
    assert g["n_rows"] == o["n_rows"] and g["n_invalid"] == o["n_invalid"]
    np.testing.assert_array_equal(g["row_weight"], np.asarray(o["row_weight"], np.float32))
    if m:
        for key in ("dept_counts", "dept_offsets", "dept_row_token", "dept_row_dept", "dept_inv",
                    "active_depts"):
            assert np.array_equal(g[key], np.asarray(o[key])), key
        np.testing.assert_allclose(g["dept_row_scale"], o["dept_row_scale"], rtol=1e-6, atol=1e-7)
    if "row_pair" in g:
        # factorised form: each row's (token, department) pair
        G = len(o["counts"]) // m
        want = [o["dept_inv"][t * m + e // G] for t, e in zip(o["row_token"], o["row_expert"])]
        assert np.array_equal(g["row_pair"], np.asarray(want, np.int32)), "row_pair"


def test_dispatch_worked_example():
    with open(GOLDEN) as f:
        gd = json.load(f)
    desc = M.layer_desc(8, gd["n_experts"], gd["top_k"], 8, dtype="f32", max_tokens=4)
    ids, tw = np.array(gd["topk_ids"]), np.array(gd["topk_w"])
    plan, ws, g = run_dispatch(desc, ids, tw)
    ex = gd["expected"]
    assert g["offsets"].tolist() == ex["expert_offsets"]
    assert g["row_token"].tolist() == ex["row_token"]
    assert g["inv_perm"].tolist() == ex["inv_perm"]
    assert g["counts"].tolist() == ex["group_rows"]
    # combine with expert n's row output = n * ones gives the page's sums
    d = 8
    row_out = torch.tensor(np.repeat((g["row_expert"] + 1.0)[:, None], d, 1), dtype=torch.float32, device=DEV)
    y = torch.empty(4, d, dtype=torch.float32, device=DEV)
    M.moe_combine(desc, plan, row_out, None, None, y)
    want = ex["combine_constant_rows"]["y"]
    np.testing.assert_allclose(y.cpu().numpy(), np.repeat(np.array(want)[:, None], d, 1), atol=1e-6)


@pytest.mark.parametrize("seed", range(6))
def test_dispatch_random_plans(seed):
    rng = np.random.default_rng(seed)
    E, k, T, m = [(8, 2, 4, 0), (128, 8, 16, 0), (64, 8, 16, 8), (256, 8, 32, 32),
                  (16, 4, 7, 4), (2048, 8, 32, 0)][seed]
    ids = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
    tw = rng.random((T, k)).astype(np.float32)
    desc = M.layer_desc(8, E, k, 8, n_depts=m, d_ff_dept=8 if m else 0, dtype="f32", max_tokens=T)
    _, _, g = run_dispatch(desc, ids, tw)
    assert_plan_equal(g, O.dispatch(ids, E, tw.astype(np.float64), m), m)


def test_dispatch_duplicates_and_invalid_ids():
    """Caller-given ids: a repeated expert inside a token keeps slot order;
    ids outside [0, E) are dropped and counted."""
    E, k, T = 6, 3, 4
    ids = np.array([[1, 1, 4], [5, -1, 0], [2, 6, 2], [0, 1, 2]], np.int32)
    tw = np.arange(12, dtype=np.float32).reshape(T, k) / 10
    desc = M.layer_desc(8, E, k, 8, n_depts=3, d_ff_dept=8, dtype="f32", max_tokens=T)
    _, _, g = run_dispatch(desc, ids, tw)
    o = O.dispatch(ids, E, tw.astype(np.float64), 3)
    assert o["n_invalid"] == 2
    assert_plan_equal(g, o, 3)


def test_dispatch_max_assignments():
    E, k, T = 256, 8, 512  # 4096 assignments, the limit
    rng = np.random.default_rng(9)
    ids = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
    tw = rng.random((T, k)).astype(np.float32)
    desc = M.layer_desc(8, E, k, 8, dtype="f32", max_tokens=T)
    _, _, g = run_dispatch(desc, ids, tw)
    assert_plan_equal(g, O.dispatch(ids, E, tw.astype(np.float64)), 0)


# ---------------------------------------------------------------------------
# Expert FFN and combine as separate calls
# ---------------------------------------------------------------------------

def _rand_weights(seed, d, E, I, m=0, S=0, Is=0, dtype=torch.float32, scale=0.05):
    g = torch.Generator().manual_seed(seed)
    r = lambda *s: (torch.randn(*s, generator=g) * scale).to(dtype).to(DEV)  # noqa: E731
    w = {"w_router": r(E, d), "w_gate": r(E, I, d), "w_up": r(E, I, d), "w_down": r(E, d, I)}
    if m:
        w.update(wd_gate=r(m, S, d), wd_up=r(m, S, d), wd_down=r(m, d, S))
    if Is:
        w.update(ws_gate=r(Is, d), ws_up=r(Is, d), ws_down=r(d, Is))
    return w


@pytest.mark.parametrize("case", [
    # (d, E, k, I, m, S, Is, T, dtype): several tiles, ragged tails, groups of >4, >8, >16 rows
    (256, 8, 2, 128, 0, 0, 0, 4, "f32"),
    (264, 6, 3, 40, 0, 0, 24, 5, "f32"),
    (520, 4, 2, 136, 2, 72, 0, 20, "f32"),
    (1024, 16, 4, 96, 4, 160, 64, 9, "bf16"),
    (776, 3, 3, 24, 0, 0, 16, 33, "bf16"),
])
def test_expert_ffn_and_combine_parity(case):
    d, E, k, I, m, S, Is, T, dt = case
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    w = _rand_weights(sum(case[:8]), d, E, I, m, S, Is, tdt)
    g = torch.Generator().manual_seed(7)
    x = torch.randn(T, d, generator=g).to(tdt).to(DEV)
    desc = M.layer_desc(d, E, k, I, n_depts=m, d_ff_dept=S, d_ff_shared=Is, dtype=dt,
                        max_tokens=T + 3)
    rng = np.random.default_rng(case[0])
    ids = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
    if T > 16:
        ids[:, 0] = 0  # one expert with > 16 rows
    tw = rng.random((T, k)).astype(np.float32)
    plan, ws, gp = run_dispatch(desc, ids, tw)
    op = O.dispatch(ids, E, tw.astype(np.float64), m)
    assert_plan_equal(gp, op, m)
    row_out = torch.full((T * k, d), float("nan"), device=DEV)
    dept_out = torch.full((max(1, op.get("n_dept_rows", 0)), d), float("nan"), device=DEV) if m else None
    shared_out = torch.full((T, d), float("nan"), device=DEV) if Is else None
    M.moe_expert_ffn(desc, w, x, plan, ws, row_out, dept_out, shared_out)
    wc = {kk: v.cpu() for kk, v in w.items()}
    o_row, o_dept, o_sh = O.expert_outputs(x.cpu(), wc, op, E, m, dept_split=bool(m))
    # row outputs are fp32; bf16 layers keep the intermediate h in bf16, so
    # they get the bf16 layer tolerance
    assert_close(to_np(row_out[:op["n_rows"]]), o_row, dt, "row_out")
    if m:
        assert_close(to_np(dept_out[:op["n_dept_rows"]]), o_dept, dt, "dept_out")
    if Is:
        assert_close(to_np(shared_out), o_sh, dt, "shared_out")
    y = torch.empty(T, d, dtype=tdt, device=DEV)
    M.moe_combine(desc, plan, row_out, dept_out, shared_out, y)
    # combine checked against the oracle combine of the GPU's own row outputs
    y_ref = O.combine(op, to_np(row_out[:op["n_rows"]]), T, k,
                      None if not m else to_np(dept_out[:op["n_dept_rows"]]),
                      None if not Is else to_np(shared_out), m, d)
    floor = 1e-6 * np.abs(y_ref).max()
    if dt == "bf16":  # one bf16 ulp where the fp32 sum straddles a rounding boundary
        np.testing.assert_allclose(to_np(y), O.cast_output(y_ref, "bf16"), rtol=2 ** -7, atol=floor)
    else:
        np.testing.assert_allclose(to_np(y), y_ref, rtol=1e-6, atol=floor)


# ---------------------------------------------------------------------------
# The fused decode step on every layer shape
# ---------------------------------------------------------------------------

def run_layer(desc, w, x):
    layer = M.MoeLayer(desc, w, DEV)
    y = torch.full_like(x, float("nan"))
    layer(x, y)
    torch.cuda.synchronize()
    return y, layer


def check_layer(name, seed, T, sample_tokens=None, max_tokens=None, allow_near=False):
    shape = SH[name]
    w = gpu_layer(name, seed)
    desc = desc_of(shape, max_tokens)
    x = moe_synth.make_tokens(shape, seed, T, DEV)
    y, layer = run_layer(desc, w, x)
    g_plan = layer.plan(T)
    g_ids, g_w = gpu_ids_from_plan(g_plan, T, shape.top_k)
    xc = x.cpu()
    o_ids, _, o_sel, o_l32 = oracle_route(shape, xc, {k: v.cpu() for k, v in w.items()})
    ids, near = reference_ids(o_ids, o_sel, g_ids, shape.top_k, shape.n_depts, shape.k_dept,
                              allow_near)
    o_w = O.routing_weights(o_l32, ids, shape.score, shape.renormalize, shape.route_scale)
    np.testing.assert_allclose(g_w, o_w, atol=1e-5)
    # the plan is the oracle's dispatch of the selected ids
    op = O.dispatch(g_ids, shape.n_experts, g_w.astype(np.float64), shape.n_depts)
    assert_plan_equal(g_plan, op, shape.n_depts)
    toks = range(T) if sample_tokens is None else sorted(set(t for t in sample_tokens if t < T))
    yg = to_np(y)
    assert np.isfinite(yg).all()
    token_output = (O.deamoe_token_output if shape.dept_form == "factorised"
                    else O.layer_token_output)
    wref = O.dequantize_layer({k: v.cpu() for k, v in w.items()}) \
        if shape.expert_dtype == "fp8" else w
    ref = np.stack([token_output(xc[t], ids[t], o_w[t], wref, shape.n_experts, shape.n_depts)
                    for t in toks])
    emax, rmax = assert_close(yg[list(toks)], ref, shape.dtype, f"{name} T={T}",
                              TOL_FACTORISED if shape.dept_form == "factorised" else None)
    print(f"{name} seed={seed} T={T}: max|err| {emax:.3e} (max|ref| {rmax:.3e}), "
          f"active {g_plan['active'].size}, near-ties {int(near.sum())}")
    return y


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_layer_tiny(seed):
    check_layer(TINY, seed, 4)


@pytest.mark.parametrize("T", [1, 4, 16])
@pytest.mark.parametrize("seed", [0, 1])
def test_layer_qwen3_shape(seed, T):
    check_layer(QWEN, seed, T)


@pytest.mark.parametrize("T", [1, 4, 16])
@pytest.mark.parametrize("seed", [0, 1])
def test_layer_deamoe_7b(seed, T):
    check_layer(DEA7, seed, T)


@pytest.mark.parametrize("name", [QWEN, DEA7])
def test_layer_two_token_tiles(name):
    """Batches of 17-32 tokens at d = 2048: the K-split gate/up tiles pass two
    16-token tiles (groups of up to 32 rows); 8 spread tokens checked."""
    check_layer(name, 0, 32, sample_tokens=spread_tokens(32), max_tokens=32)


@pytest.mark.parametrize("name,T", [(QWEN, 128), (QWEN, 512), (DEA7, 100), (DSV3, 128),
                                    (DEAV3, 128), (PAPER, 128),
                                    ("deepseek_v3_d7168_e256_i2048_s2048_top8_fp8", 128)])
def test_layer_large_batch(name, T):
    """Batches past 64 tokens: the plan ranks an assignment by popcounts over
    its expert's token bits spread across several 64-bit words (eight at
    T = 512, the assignment limit at top-8; the 864-expert layer's 1728 words
    at T = 128 sit in the plan launch's staging area), a pair by its
    department's token bits (two words at T = 100 and 128), one wave writes
    the plan when there are no departments, the combine lists each token's
    active departments (32 of them on the DeepSeek-V3 geometry), and groups
    span several 16-token chunks.  The whole plan is compared; outputs on a
    sample of tokens."""
    stride = 7 if SH[name].d <= 2048 else 31
    check_layer(name, 0, T, sample_tokens=list(range(0, T, stride)) + [T - 1], max_tokens=T,
                allow_near=True)


@pytest.mark.parametrize("T", [1, 2, 4, 8, 16, 32])
def test_layer_deepseek_v3_shape(T):
    """The DeepSeek-V3-shaped layer at every listed batch: every token up to
    four tokens, eight spread tokens (first and last included) above."""
    check_layer(DSV3, 0, T, sample_tokens=spread_tokens(T))


@pytest.mark.parametrize("T", [1, 2, 4, 8, 16])
def test_layer_deamoe_dsv3(T):
    """The department transform of the DeepSeek-V3-shaped layer at every
    listed batch (department reuse starts at four tokens): every token up to
    four tokens, eight spread tokens above."""
    check_layer(DEAV3, 0, T, sample_tokens=spread_tokens(T))


@pytest.mark.parametrize("name,T", [(n, T) for n in FACT for T in FACT[n].batches])
def test_layer_factorised_small(name, T):
    """Factorised DeaMoE experts end to end against the oracle's per-expert
    definition, every token."""
    check_layer(name, 0, T)


@pytest.mark.parametrize("T", [1, 4, 16])
def test_layer_factorised_paper_shape(T):
    """DeaMoE's DeepSeek-V3-matched layer (864 experts in 8 departments,
    hffn = 2048, k = 10), sampled tokens against the oracle."""
    check_layer(PAPER, 0, T, sample_tokens=spread_tokens(T, 4))


@pytest.mark.parametrize("name,T", [(n, T) for n in FP8 for T in FP8[n].batches])
def test_layer_fp8_small(name, T):
    """FP8 expert layers end to end against the oracle on the dequantized
    weights, every token."""
    check_layer(name, 0, T)


@pytest.mark.parametrize("T", [1, 4, 16])
def test_layer_fp8_qwen3_shape(T):
    check_layer("qwen3_30b_a3b_d2048_e128_i768_top8_fp8", 0, T)


@pytest.mark.parametrize("T", [1, 8, 32])
def test_layer_fp8_deepseek_v3_shape(T):
    check_layer("deepseek_v3_d7168_e256_i2048_s2048_top8_fp8", 0, T,
                sample_tokens=[0, T // 2, T - 1])


def test_fp8_every_code():
    """Codes drawn over every E4M3 value (subnormals, both zeros, +-448; no
    NaN) with per-row scales over six binades: moe_expert_ffn's per-row
    outputs and the combined y against the oracle's dequantized weights, so
    that each code's widening on the GPU is checked against the format's
    definition."""
    d, E, k, I, m, S, Is, T = 528, 5, 2, 64, 0, 0, 48, 6
    g = torch.Generator().manual_seed(11)
    finite = torch.tensor([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=torch.uint8)

    def codes(*shape):
        return finite[torch.randint(0, finite.numel(), shape, generator=g)].to(DEV)

    def scales(*shape):
        return (2.0 ** torch.randint(-14, -8, shape, generator=g).float()).to(DEV)
    w = {"w_router": (torch.randn(E, d, generator=g) * 0.05).to(torch.bfloat16).to(DEV),
         "w_gate": codes(E, I, d), "w_up": codes(E, I, d), "w_down": codes(E, d, I),
         "w_gate_scale": scales(E, I), "w_up_scale": scales(E, I), "w_down_scale": scales(E, d),
         "ws_gate": codes(Is, d), "ws_up": codes(Is, d), "ws_down": codes(d, Is),
         "ws_gate_scale": scales(Is), "ws_up_scale": scales(Is), "ws_down_scale": scales(d)}
    x = torch.randn(T, d, generator=g).to(torch.bfloat16).to(DEV)
    desc = M.layer_desc(d, E, k, I, d_ff_shared=Is, dtype="bf16", expert_dtype="fp8",
                        max_tokens=T)
    rng = np.random.default_rng(2)
    ids = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
    ids[:, 0] = 1  # one group of six rows: two token chunks
    tw = rng.random((T, k)).astype(np.float32)
    plan, ws, gp = run_dispatch(desc, ids, tw)
    op = O.dispatch(ids, E, tw.astype(np.float64), 0)
    row_out = torch.full((T * k, d), float("nan"), device=DEV)
    shared_out = torch.full((T, d), float("nan"), device=DEV)
    M.moe_expert_ffn(desc, w, x, plan, ws, row_out, None, shared_out)
    wref = O.dequantize_layer({kk: v.cpu() for kk, v in w.items()})
    o_row, _, o_sh = O.expert_outputs(x.cpu(), wref, op, E, 0)
    assert_close(to_np(row_out[:op["n_rows"]]), o_row, "bf16", "fp8 row_out")
    assert_close(to_np(shared_out), o_sh, "bf16", "fp8 shared_out")


def test_factorised_expert_ffn_and_combine_match_the_fused_step():
    """moe_dispatch + moe_expert_ffn + moe_combine give the fused step's y bit
    for bit, and row_out holds each row's private output
    SiLU((A_d)^T (SiLU(A_g x_g) * (A_u x_u))) (checked against the oracle on
    sampled rows)."""
    name = "fact_bf16_d1024_e32_m4_h256_top6"
    shape, T = SH[name], 5
    w = gpu_layer(name, 0)
    desc = desc_of(shape)
    x = moe_synth.make_tokens(shape, 0, T, DEV)
    y_fused, layer = run_layer(desc, w, x)
    k, E, m, S = shape.top_k, shape.n_experts, shape.n_depts, shape.d_ff_dept
    ws = M.alloc_workspace(desc, DEV)
    g_ids = torch.empty(T, k, dtype=torch.int32, device=DEV)
    g_w = torch.empty(T, k, dtype=torch.float32, device=DEV)
    M.moe_route(desc, x, w["w_router"], w.get("router_bias"), g_ids, g_w, ws)
    plan = M.moe_dispatch(desc, g_ids, g_w, ws)
    row_out = torch.full((T * k, S), float("nan"), device=DEV)
    dept_out = torch.full((T * min(m, k), shape.d), float("nan"), device=DEV)
    shared_out = torch.full((T, shape.d), float("nan"), device=DEV)
    M.moe_expert_ffn(desc, w, x, plan, ws, row_out, dept_out, shared_out)
    y = torch.full_like(x, float("nan"))
    M.moe_combine(desc, plan, None, dept_out, shared_out, y)
    torch.cuda.synchronize()
    assert torch.equal(y, y_fused)
    hp = M.plan_to_host(desc, plan, ws)

    def f64(t):
        return t.detach().to("cpu", torch.float64).numpy()
    G = E // m
    for r in range(0, hp["n_rows"], 3):
        e, t = int(hp["row_expert"][r]), int(hp["row_token"][r])
        j = e // G
        xg = O.silu(f64(w["wd_gate"][j]) @ f64(x[t]))
        xu = O.silu(f64(w["wd_up"][j]) @ f64(x[t]))
        yv = O.silu(f64(w["w_gate"][e]) @ xg) * (f64(w["w_up"][e]) @ xu)
        z = O.silu(f64(w["w_down"][e]) @ yv)   # stored (A_d)^T, applied as is
        # Z sits behind three bf16 roundings (x_g, x_u and Y, each about 2^-9
        # relative) where the layer output y sits behind one (h), so the rms
        # bound is widened from 4e-3 to 1e-2; the max bound is the same.
        got = row_out[r].cpu().numpy().astype(np.float64)
        err = np.abs(got - z)
        assert err.max() <= 2e-2 * np.abs(z).max(), f"row {r}: max|err| {err.max():.3e}"
        assert np.sqrt((err ** 2).mean()) <= 1e-2 * np.sqrt((z ** 2).mean()), f"row {r} rms"


def test_layer_department_equals_expanded_vanilla():
    """The department layer equals a vanilla layer whose experts carry the
    concatenated [department ; private] matrices (computed on the GPU by the
    vanilla path), on the same tokens."""
    shape = SH[DEA7]
    w = gpu_layer(DEA7, 0)
    T = 16
    x = moe_synth.make_tokens(shape, 0, T, DEV)
    yd, _ = run_layer(desc_of(shape), w, x)
    G = shape.n_experts // shape.n_depts
    dept = torch.arange(shape.n_experts, device=DEV) // G
    wv = {"w_router": w["w_router"],
          "w_gate": torch.cat([w["wd_gate"][dept], w["w_gate"]], 1).contiguous(),
          "w_up": torch.cat([w["wd_up"][dept], w["w_up"]], 1).contiguous(),
          "w_down": torch.cat([w["wd_down"][dept], w["w_down"]], 2).contiguous()}
    dv = M.layer_desc(shape.d, shape.n_experts, shape.top_k, shape.d_ff_dept + shape.d_ff,
                      dtype="bf16", max_tokens=T)
    yv, _ = run_layer(dv, wv, x)
    assert_close(to_np(yd), to_np(yv), "bf16", "department vs expanded")


# ---------------------------------------------------------------------------
# Edge cases, errors, determinism
# ---------------------------------------------------------------------------

def test_layer_edge_shapes():
    """k = 1, k = E, one expert per department, T = max_tokens, ragged d/I."""
    cases = [dict(d=264, E=4, k=1, I=40, T=3), dict(d=256, E=8, k=8, I=128, T=4),
             dict(d=128, E=4, k=2, I=16, m=4, S=24, T=6), dict(d=1032, E=5, k=2, I=72, Is=40, T=17)]
    for i, c in enumerate(cases):
        m, S, Is = c.get("m", 0), c.get("S", 0), c.get("Is", 0)
        w = _rand_weights(50 + i, c["d"], c["E"], c["I"], m, S, Is)
        g = torch.Generator().manual_seed(i)
        x = torch.randn(c["T"], c["d"], generator=g).to(DEV)
        desc = M.layer_desc(c["d"], c["E"], c["k"], c["I"], n_depts=m, d_ff_dept=S,
                            d_ff_shared=Is, dtype="f32", max_tokens=c["T"])
        y, layer = run_layer(desc, w, x)
        wc = {kk: v.cpu() for kk, v in w.items()}
        o_ids, o_w, o_sel, _ = O.route(x.cpu(), wc["w_router"], c["k"])
        g_ids, _ = gpu_ids_from_plan(layer.plan(c["T"]), c["T"], c["k"])
        ids, _ = reference_ids(o_ids, o_sel, g_ids, c["k"], allow_near=True)
        ref = O.layer_bruteforce(x.cpu(), wc, ids, o_w, c["E"], m)
        assert_close(to_np(y), ref, "f32", f"edge case {c}")


@pytest.mark.parametrize("case", [
    # (d, E, k, I, m, S, Is): rows of one step with idle lanes (I = 40, Is = 24),
    # rows of several steps with a ragged last one (I = 1096: 137 chunks of 16
    # bytes over 64 lanes), department slices with and without the shared
    # expert; rows of 128 and 256 elements, whose groups share a wave load
    # four or two at a time (a ragged last load when the group count is not
    # a multiple), in every family
    (776, 6, 3, 40, 0, 0, 24),
    (264, 8, 2, 1096, 0, 0, 0),
    (1024, 16, 4, 96, 4, 160, 64),
    (520, 12, 6, 56, 3, 200, 0),
    (512, 16, 4, 128, 4, 256, 128),
    (640, 10, 3, 256, 0, 0, 256),
    (384, 24, 7, 128, 0, 0, 0),
])
@pytest.mark.parametrize("T", [1, 2, 3, 4])
def test_layer_down_with_combine_epilogue(case, T):
    """bf16 layers at batches of at most four tokens take the down projection
    that writes y itself (each wave one output column over every group of
    every family); against the oracle's per-token evaluation of the GPU's
    selection, every token."""
    d, E, k, I, m, S, Is = case
    w = _rand_weights(sum(case) + T, d, E, I, m, S, Is, torch.bfloat16)
    g = torch.Generator().manual_seed(T)
    x = torch.randn(T, d, generator=g).to(torch.bfloat16).to(DEV)
    desc = M.layer_desc(d, E, k, I, n_depts=m, d_ff_dept=S, d_ff_shared=Is, dtype="bf16",
                        max_tokens=4)
    y, layer = run_layer(desc, w, x)
    wc = {kk: v.cpu() for kk, v in w.items()}
    o_ids, o_w, o_sel, _ = O.route(x.cpu(), wc["w_router"], k)
    g_ids, _ = gpu_ids_from_plan(layer.plan(T), T, k)
    ids, _ = reference_ids(o_ids, o_sel, g_ids, k, allow_near=True)
    ref = O.layer_bruteforce(x.cpu(), wc, ids, o_w, E, m)
    assert_close(to_np(y), ref, "bf16", f"fused down+combine {case} T={T}")
    # the same step without the fused epilogue: per-row outputs, then the
    # combine (summation orders differ, so bf16-rounding agreement)
    ws = M.alloc_workspace(desc, DEV)
    g_ids_t = torch.empty(T, k, dtype=torch.int32, device=DEV)
    g_w_t = torch.empty(T, k, dtype=torch.float32, device=DEV)
    M.moe_route(desc, x, w["w_router"], None, g_ids_t, g_w_t, ws)
    plan = M.moe_dispatch(desc, g_ids_t, g_w_t, ws)
    row_out = torch.empty(T * k, d, device=DEV)
    dept_out = torch.empty(T * min(m, k), d, device=DEV) if m else None
    shared_out = torch.empty(T, d, device=DEV) if Is else None
    M.moe_expert_ffn(desc, w, x, plan, ws, row_out, dept_out, shared_out)
    y2 = torch.empty_like(y)
    M.moe_combine(desc, plan, row_out, dept_out, shared_out, y2)
    torch.cuda.synchronize()
    a, b = to_np(y), to_np(y2)
    np.testing.assert_allclose(a, b, rtol=2 ** -7, atol=1e-6 * np.abs(b).max())


def _to_fp8(w):
    """The bf16 expert matrices of `w` as E4M3 codes with per-row scales
    (torch's float8_e4m3fn rounding of row / (row max / 448))."""
    out = {"w_router": w["w_router"]}
    for k, v in w.items():
        if k == "w_router":
            continue
        f = v.float()
        sc = f.abs().amax(dim=-1).clamp_min(1e-30) / 448.0
        out[k] = (f / sc[..., None]).clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8)
        out[k + "_scale"] = sc.contiguous()
    return out


@pytest.mark.parametrize("case", [
    # (d, E, k, I, m, S, Is): FP8 widths are multiples of 16
    (1040, 6, 3, 48, 0, 0, 32),
    (528, 12, 6, 64, 3, 208, 0),
    (272, 5, 2, 2048, 0, 0, 0),
])
@pytest.mark.parametrize("T", [1, 3, 4])
def test_layer_fp8_down_with_combine_epilogue(case, T):
    """FP8 layers at batches of at most four tokens take the down launch
    that writes y; against the oracle on the dequantized weights, and
    against the separate down and combine launches."""
    d, E, k, I, m, S, Is = case
    w = _to_fp8(_rand_weights(sum(case) + 7 * T, d, E, I, m, S, Is, torch.bfloat16))
    g = torch.Generator().manual_seed(T + 100)
    x = torch.randn(T, d, generator=g).to(torch.bfloat16).to(DEV)
    desc = M.layer_desc(d, E, k, I, n_depts=m, d_ff_dept=S, d_ff_shared=Is, dtype="bf16",
                        expert_dtype="fp8", max_tokens=4)
    assert M.moe_layer_kernel_count(desc, T) == 4
    y, layer = run_layer(desc, w, x)
    wc = {kk: v.cpu() for kk, v in w.items()}
    o_ids, o_w, o_sel, _ = O.route(x.cpu(), wc["w_router"], k)
    g_ids, _ = gpu_ids_from_plan(layer.plan(T), T, k)
    ids, _ = reference_ids(o_ids, o_sel, g_ids, k, allow_near=True)
    ref = O.layer_bruteforce(x.cpu(), O.dequantize_layer(wc), ids, o_w, E, m)
    assert_close(to_np(y), ref, "bf16", f"fp8 fused down+combine {case} T={T}")
    ws = M.alloc_workspace(desc, DEV)
    ti = torch.empty(T, k, dtype=torch.int32, device=DEV)
    tw = torch.empty(T, k, dtype=torch.float32, device=DEV)
    M.moe_route(desc, x, w["w_router"], None, ti, tw, ws)
    plan = M.moe_dispatch(desc, ti, tw, ws)
    row_out = torch.empty(T * k, d, device=DEV)
    dept_out = torch.empty(T * min(m, k), d, device=DEV) if m else None
    shared_out = torch.empty(T, d, device=DEV) if Is else None
    M.moe_expert_ffn(desc, w, x, plan, ws, row_out, dept_out, shared_out)
    y2 = torch.empty_like(y)
    M.moe_combine(desc, plan, row_out, dept_out, shared_out, y2)
    torch.cuda.synchronize()
    a, b = to_np(y), to_np(y2)
    np.testing.assert_allclose(a, b, rtol=2 ** -7, atol=1e-6 * np.abs(b).max())


def test_layer_zero_tokens_and_errors():
    shape = SH[TINY]
    w = gpu_layer(TINY, 0)
    desc = desc_of(shape)
    layer = M.MoeLayer(desc, w, DEV)
    x0 = torch.empty(0, shape.d, device=DEV)
    assert layer(x0).shape == (0, shape.d)
    x = moe_synth.make_tokens(shape, 0, 5, DEV)  # max_tokens is 4
    with pytest.raises(M.MoeError) as e:
        layer(x)
    assert e.value.status == M.MOE_ERR_INVALID_ARG
    small = torch.empty(64, dtype=torch.uint8, device=DEV)
    y = torch.full((4, shape.d), 3.0, device=DEV)
    with pytest.raises(M.MoeError) as e:
        M.moe_layer_decode(desc, w, x[:4].contiguous(), y, small)
    assert e.value.status == M.MOE_ERR_WORKSPACE
    assert torch.all(y == 3.0)  # nothing written
    # misaligned activation pointer
    buf = torch.zeros(4 * shape.d + 1, device=DEV)
    xm = buf[1:].view(4, shape.d)
    with pytest.raises(M.MoeError) as e:
        M.moe_layer_decode(desc, w, xm, y, layer.workspace)
    assert e.value.status == M.MOE_ERR_INVALID_ARG


def test_layer_is_deterministic():
    shape = SH[QWEN]
    w = gpu_layer(QWEN, 0)
    x = moe_synth.make_tokens(shape, 0, 16, DEV)
    layer = M.MoeLayer(desc_of(shape), w, DEV)
    ys = [layer(x).clone() for _ in range(3)]
    torch.cuda.synchronize()
    assert all(torch.equal(ys[0], y) for y in ys[1:])


@pytest.mark.parametrize("name,T", [(TINY, 4), (QWEN, 1), (QWEN, 16), (DEA7, 4), (DEA7, 16),
                                    ("fact_bf16_d1024_e32_m4_h256_top6", 5),
                                    ("fp8_d1040_e12_m3_s208_i48_sh32_top4", 9)])
def test_step_stats(name, T):
    """The step's routing statistics, written on the device by the plan
    kernel, against the oracle's load count of the same ids (DeepSeekMoE
    Guide's balance metric: max expert count over the mean of the E routed
    experts) and its byte count; y is the same with and without them."""
    shape = SH[name]
    w = gpu_layer(name, 0)
    desc = desc_of(shape)
    x = moe_synth.make_tokens(shape, 0, T, DEV)
    layer = M.MoeLayer(desc, w, DEV)
    y0 = layer(x).clone()
    stats = M.alloc_step_stats(DEV)
    stats.fill_(-1)
    y1 = layer(x, stats=stats)
    torch.cuda.synchronize()
    assert torch.equal(y0, y1)
    g = M.step_stats_to_host(stats, shape.n_experts)
    g_ids, _ = gpu_ids_from_plan(layer.plan(T), T, shape.top_k)
    o = O.expert_load_stats(g_ids, shape.n_experts, shape.n_depts)
    assert g["n_tokens"] == T and g["n_invalid"] == 0
    assert g["expert_rows"] == o["counts"]
    assert g["n_assignments"] == o["n_assignments"] == T * shape.top_k
    assert g["max_expert_rows"] == o["max"]
    assert g["n_active_experts"] == o["n_active_experts"]
    assert g["n_active_depts"] == o["n_active_depts"]
    assert g["mean_expert_rows"] == pytest.approx(o["mean"], rel=1e-6)
    assert g["imbalance_ratio"] == pytest.approx(o["imbalance_ratio"], rel=1e-6)
    if shape.expert_dtype == "fp8":
        want = O.loaded_weight_bytes_fp8(g_ids, shape.n_experts, shape.d, shape.d_ff, 2,
                                         shape.n_depts, shape.d_ff_dept, shape.d_ff_shared)
    else:
        want = O.loaded_weight_bytes(g_ids, shape.n_experts, shape.d, shape.d_ff,
                                     4 if shape.dtype == "f32" else 2, shape.n_depts,
                                     shape.d_ff_dept, shape.d_ff_shared,
                                     factorised=shape.dept_form == "factorised")
    assert g["loaded_weight_bytes"] == want
    # entries past E are left alone
    if shape.n_experts < M.MAX_EXPERTS:
        raw = stats.cpu().numpy().view(np.int32)
        off = (M.StepStats.expert_rows.offset // 4) + shape.n_experts
        assert raw[off] == -1


def test_stage_events_time_each_kernel():
    """With stage events the step gives the same y, and every stage's
    start/stop pair brackets a kernel of positive duration."""
    shape = SH[QWEN]
    w = gpu_layer(QWEN, 0)
    x = moe_synth.make_tokens(shape, 0, 4, DEV)
    layer = M.MoeLayer(desc_of(shape), w, DEV)
    y0 = layer(x).clone()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(2 * M.N_STAGES)]
    for e in evs:
        e.record()
    torch.cuda.synchronize()
    y1 = layer(x, stage_events=evs)
    torch.cuda.synchronize()
    assert torch.equal(y0, y1)
    for s in range(M.N_STAGES):
        ms = evs[2 * s].elapsed_time(evs[2 * s + 1])
        # at four tokens the down launch writes y itself: the combine stage is
        # an empty interval
        lo = 0.0 if M.STAGE_NAMES[s] == "combine" else 1e-6
        assert lo <= ms < 50.0, (M.STAGE_NAMES[s], ms)


def test_stream_read_sums_each_16k_block():
    """The measurement helper reads every byte once: block sums of a known
    bf16 pattern (small integers, exact in fp32)."""
    n_blocks = 300
    vals = (torch.arange(n_blocks * 8192, dtype=torch.int64) % 7 - 3).to(torch.bfloat16)
    src = vals.to(DEV)
    sink = torch.full((n_blocks,), -1.0, dtype=torch.float32, device=DEV)
    M.moe_stream_read(src, sink)
    torch.cuda.synchronize()
    ref = vals.float().view(n_blocks, 8192).sum(1)
    assert torch.equal(sink.cpu(), ref)

