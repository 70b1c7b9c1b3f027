"""Shared helpers of the GPU parity tests: build a layer on the device from the
seeded generator, run the oracle on the same inputs, compare."""
from __future__ import annotations

import numpy as np
import torch

import moe_layer_decode_amd as M
import moe_synth
import oracle as O

# Selection-score agreement bound between the HIP path (fp32 sums in its own
# order) and the oracle (fp64 sums rounded once): the logits of these layers
# differ by ~1e-6 absolute; 2e-5 * max(1, |s|) leaves a wide margin.  Tokens
# whose k-th/(k+1)-th oracle margin is within 2 tau are near-ties where either
# selection is correct to fp32 precision.
TAU = 2e-5

# Output tolerances: bf16 layers max|err| <= 2e-2 * max|ref| (the contract),
# plus an RMS bound well above bf16 output rounding (2^-9 relative per
# element); fp32 layers 1e-4 * max|ref|.
TOL = {"bf16": (2e-2, 4e-3), "f32": (1e-4, 1e-5)}


def desc_of(shape: moe_synth.LayerShape, max_tokens: int = None, **over) -> M.LayerDesc:
    kw = dict(n_depts=shape.n_depts, d_ff_dept=shape.d_ff_dept, d_ff_shared=shape.d_ff_shared,
              score=shape.score, renormalize=shape.renormalize, route_scale=shape.route_scale,
              dtype=shape.dtype, max_tokens=max_tokens or max(shape.batches),
              dept_form=shape.dept_form, k_dept=shape.k_dept,
              dept_strict=shape.dept_strict, expert_dtype=shape.expert_dtype)
    kw.update(over)
    return M.layer_desc(shape.d, shape.n_experts, shape.top_k, shape.d_ff, **kw)


def to_np(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float64).numpy()


def oracle_route(shape, x, w, k=None):
    return O.route(x, w["w_router"], k or shape.top_k, shape.score, w.get("router_bias"),
                   shape.renormalize, shape.route_scale, shape.n_depts, shape.k_dept,
                   shape.dept_strict)


def select(sel: np.ndarray, shape, k=None) -> np.ndarray:
    """The oracle's selection rule of this layer shape applied to given scores."""
    k = k or shape.top_k
    if shape.dept_strict:
        return O.topk_select_strict(sel, k, shape.n_depts, shape.k_dept)
    if shape.k_dept:
        return O.topk_select_grouped(sel, k, shape.n_depts, shape.k_dept)
    return O.topk_select(sel, k)


def _gap(s: np.ndarray, k: int) -> np.ndarray:
    s = -np.sort(-s.astype(np.float64), axis=1)
    if s.shape[1] <= k:
        return np.full(s.shape[0], np.inf)
    return s[:, k - 1] - s[:, k]


def margins(sel: np.ndarray, k: int, n_depts: int = 0, k_dept: int = 0) -> np.ndarray:
    """Per token: k-th minus (k+1)-th largest selection score (inf if k = E).
    Department-limited: the smaller of the k_dept-th/(k_dept+1)-th gap of the
    department scores and the expert gap inside the chosen departments."""
    if not k_dept:
        return _gap(sel, k)
    T, E = sel.shape
    g = E // n_depts
    dscore = sel.reshape(T, n_depts, g).max(axis=2)
    out = _gap(dscore, k_dept)
    for t in range(T):
        # every chosen department counts, also those left without experts
        chosen = sorted(range(n_depts), key=lambda j: (-dscore[t, j], j))[:k_dept]
        pool = np.concatenate([sel[t, j * g:(j + 1) * g] for j in chosen])
        out[t] = min(out[t], _gap(pool[None], k)[0])
    return out


def reference_ids(o_ids, o_sel, g_ids, k, n_depts: int = 0, k_dept: int = 0,
                  allow_near: bool = False):
    """Oracle ids, except that on near-tie tokens (margin within 2 tau) the
    HIP path's choice stands.  Returns (ids, near_tie_mask); asserts that
    every other token agrees exactly.  Unless allow_near, asserts that there
    is no near-tie token at all, so the ids are the oracle's bit for bit (the
    committed seeds of the listed layer shapes have none up to 32 tokens)."""
    tau = TAU * np.maximum(1.0, np.abs(o_sel).max(axis=1))
    near = margins(o_sel, k, n_depts, k_dept) <= 2 * tau
    assert allow_near or not near.any(), \
        f"near-tie tokens {np.nonzero(near)[0].tolist()} where none is expected"
    mism = np.any(o_ids != g_ids, axis=1)
    bad = mism & ~near
    assert not bad.any(), f"top-k ids differ on tokens {np.nonzero(bad)[0].tolist()} outside near-ties"
    ids = np.where(near[:, None], g_ids, o_ids)
    return ids, near


def gpu_ids_from_plan(plan, T, k):
    inv = plan["inv_perm"].reshape(T, k)
    return plan["row_expert"][inv], plan["row_weight"][inv]


# Factorised DeaMoE layers (section 3.1) in bf16 round to bf16 six times on
# the way to y (x_g, x_u, Y, Z, the department sum z, then y), each about
# 2^-9 relative, against once (h) for the plain layer: the rms bound widens
# from 4e-3 to 1e-2; the max bound, the contract, stays.
TOL_FACTORISED = {"bf16": (2e-2, 1e-2), "f32": TOL["f32"]}


def assert_close(y_gpu: np.ndarray, y_ref: np.ndarray, dtype: str, what: str = "y",
                 tol=None):
    mx_tol, rms_tol = (tol or TOL)[dtype]
    ref_max = np.abs(y_ref).max() if y_ref.size else 0.0
    err = np.abs(y_gpu - y_ref)
    emax = err.max() if err.size else 0.0
    assert emax <= mx_tol * ref_max + 1e-30, f"{what}: max|err| {emax:.3e} > {mx_tol} * max|ref| {ref_max:.3e}"
    if y_ref.size:
        rms_ref = np.sqrt(np.mean(y_ref ** 2))
        rms_err = np.sqrt(np.mean(err ** 2))
        assert rms_err <= rms_tol * rms_ref + 1e-30, f"{what}: rms err {rms_err:.3e} > {rms_tol} * rms ref {rms_ref:.3e}"
    return emax, ref_max


def spread_tokens(T: int, n: int = 8):
    """Every token when T <= 4, else n tokens spread evenly over [0, T)
    with the first and the last among them."""
    if T <= 4:
        return list(range(T))
    return sorted({int(round(v)) for v in np.linspace(0, T - 1, min(n, T))})
