"""Python binding of the MI355X MoE decode-layer library (libmoe_decode.so).

Argument marshalling only: every step of the layer runs in the library's HIP
kernels.  torch supplies device memory (tensors) and streams; tensors are
passed to the C ABI as raw device pointers.  If the shared library is not
built, importing works but every call raises -- there is no CPU fallback.

The functions keep the C names: moe_workspace_bytes, moe_route, moe_dispatch,
moe_expert_ffn, moe_combine, moe_layer_decode (see include/moe_decode.h for the
exact contract of each).
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional, Sequence

import torch

__all__ = [
    "MoeError", "LayerDesc", "Weights", "Plan", "layer_desc", "lib", "lib_path",
    "moe_workspace_bytes", "moe_workspace_init", "moe_validate_desc", "moe_route", "moe_dispatch",
    "moe_expert_ffn", "moe_combine", "moe_layer_decode", "moe_layer_decode_timed",
    "moe_layer_decode_noalloc", "NOALLOC_SCRATCH_BYTES", "moe_status_string", "StepStats", "STEP_STATS_BYTES", "alloc_step_stats", "step_stats_to_host",
    "moe_loaded_weight_bytes", "moe_stream_read", "moe_layer_kernel_count",
    "moe_layer_launch_workitems", "alloc_workspace",
    "plan_to_host", "MoeLayer",
    "MOE_OK", "MOE_ERR_INVALID_ARG", "MOE_ERR_UNSUPPORTED", "MOE_ERR_WORKSPACE",
    "MOE_ERR_HIP", "SCORE_FNS", "DEPT_FORMS", "MOE_DEPT_SLICE", "MOE_DEPT_FACTORISED",
    "MOE_F32", "MOE_BF16", "MOE_FP8_E4M3",
    "N_STAGES", "STAGE_NAMES", "STAGE_ROUTE", "STAGE_DISPATCH", "STAGE_GATEUP", "STAGE_DOWN",
    "STAGE_COMBINE", "EXPORTED_SYMBOLS",
]

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = range(5)
MOE_F32, MOE_BF16, MOE_FP8_E4M3 = 0, 1, 2
MOE_DEPT_SLICE, MOE_DEPT_FACTORISED = 0, 1
DEPT_FORMS = {"slice": MOE_DEPT_SLICE, "factorised": MOE_DEPT_FACTORISED}
SCORE_FNS = {"softmax": 0, "sigmoid": 1, "softmax_bias": 2}
PLAN_HEADER_LEN = 16
PLAN_N_ROWS, PLAN_N_ACTIVE, PLAN_N_DEPT_ROWS, PLAN_N_ACTIVE_DEPTS, PLAN_N_INVALID = range(5)
N_STAGES = 5
STAGE_NAMES = ("route", "dispatch", "gateup", "down", "combine")
STAGE_ROUTE, STAGE_DISPATCH, STAGE_GATEUP, STAGE_DOWN, STAGE_COMBINE = range(N_STAGES)
EXPORTED_SYMBOLS = (
    "moe_workspace_bytes", "moe_workspace_init", "moe_validate_desc", "moe_plan_from_workspace", "moe_route",
    "moe_dispatch", "moe_expert_ffn", "moe_combine", "moe_layer_decode", "moe_layer_decode_timed",
    "moe_layer_decode_noalloc", "moe_status_string", "moe_loaded_weight_bytes", "moe_stream_read", "moe_layer_kernel_count",
    "moe_layer_launch_workitems",
)

_i32, _f32, _vp, _sz = ctypes.c_int32, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t


class LayerDesc(ctypes.Structure):
    _fields_ = [("d_model", _i32), ("n_experts", _i32), ("top_k", _i32), ("d_ff", _i32),
                ("n_depts", _i32), ("d_ff_dept", _i32), ("d_ff_shared", _i32),
                ("score_fn", _i32), ("renormalize", _i32), ("route_scale", _f32),
                ("w_dtype", _i32), ("act_dtype", _i32), ("max_tokens", _i32),
                ("dept_form", _i32), ("k_dept", _i32), ("dept_strict", _i32)]

    @property
    def torch_dtype(self):
        return torch.bfloat16 if self.act_dtype == MOE_BF16 else torch.float32


_MATS = ("w_gate", "w_up", "w_down", "wd_gate", "wd_up", "wd_down", "ws_gate", "ws_up",
         "ws_down")


class Weights(ctypes.Structure):
    _fields_ = [(n, _vp) for n in ("w_router", "router_bias", *_MATS,
                                   *(m + "_scale" for m in _MATS))]


_PLAN_ARRAYS = ("header", "counts", "offsets", "row_token", "row_slot", "row_expert",
                "row_weight", "inv_perm", "active", "dept_counts", "dept_offsets",
                "dept_row_token", "dept_row_dept", "dept_row_scale", "dept_inv", "active_depts",
                "row_pair")


class Plan(ctypes.Structure):
    _fields_ = [(n, _vp) for n in _PLAN_ARRAYS] + [("n_tokens", _i32)]


MAX_EXPERTS = 2048


class StepStats(ctypes.Structure):
    """moe_step_stats: the step's routing statistics, filled on the device."""
    _fields_ = [("n_tokens", _i32), ("n_assignments", _i32), ("n_active_experts", _i32),
                ("n_active_depts", _i32), ("max_expert_rows", _i32), ("n_invalid", _i32),
                ("mean_expert_rows", _f32), ("imbalance_ratio", _f32),
                ("loaded_weight_bytes", ctypes.c_uint64),
                ("expert_rows", _i32 * MAX_EXPERTS)]


STEP_STATS_BYTES = ctypes.sizeof(StepStats)
NOALLOC_SCRATCH_BYTES = 32 << 20   # MOE_NOALLOC_SCRATCH_BYTES


class MoeError(RuntimeError):
    def __init__(self, status: int, call: str):
        self.status = status
        super().__init__(f"{call}: {moe_status_string(status)} (status {status})")


_LIB = None


def lib_path() -> str:
    return os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoe_decode.so")


def lib() -> ctypes.CDLL:
    """The loaded C library; raises if it has not been built."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = lib_path()
    if not os.path.exists(path):
        raise ImportError(
            f"{path} is missing: build the HIP library first "
            "(python -m moe_layer_decode_amd.build); there is no CPU fallback")
    L = ctypes.CDLL(path)
    P = ctypes.POINTER
    L.moe_workspace_bytes.argtypes = [P(LayerDesc)]
    L.moe_workspace_bytes.restype = _sz
    L.moe_workspace_init.argtypes = [P(LayerDesc), _vp, _sz, _vp]
    L.moe_workspace_init.restype = _i32
    L.moe_validate_desc.argtypes = [P(LayerDesc)]
    L.moe_validate_desc.restype = _i32
    L.moe_plan_from_workspace.argtypes = [P(LayerDesc), _vp, _sz, _i32, P(Plan)]
    L.moe_plan_from_workspace.restype = _i32
    L.moe_route.argtypes = [P(LayerDesc), _vp, _vp, _vp, _i32, _vp, _vp, _vp, _vp, _sz, _vp]
    L.moe_route.restype = _i32
    L.moe_dispatch.argtypes = [P(LayerDesc), _vp, _vp, _i32, _vp, _sz, P(Plan), _vp]
    L.moe_dispatch.restype = _i32
    L.moe_expert_ffn.argtypes = [P(LayerDesc), P(Weights), _vp, _i32, P(Plan), _vp, _sz,
                                 _vp, _vp, _vp, _vp]
    L.moe_expert_ffn.restype = _i32
    L.moe_combine.argtypes = [P(LayerDesc), P(Plan), _vp, _vp, _vp, _i32, _vp, _vp]
    L.moe_combine.restype = _i32
    L.moe_layer_decode.argtypes = [P(LayerDesc), P(Weights), _vp, _i32, _vp, _vp, _sz, _vp, _vp]
    L.moe_layer_decode.restype = _i32
    L.moe_layer_decode_timed.argtypes = [P(LayerDesc), P(Weights), _vp, _i32, _vp, _vp, _sz, _vp,
                                         _vp, _vp]
    L.moe_layer_decode_timed.restype = _i32
    L.moe_layer_decode_noalloc.argtypes = [P(LayerDesc), P(Weights), _vp, _i32, _vp, _vp, _vp]
    L.moe_layer_decode_noalloc.restype = _i32
    L.moe_status_string.argtypes = [_i32]
    L.moe_status_string.restype = ctypes.c_char_p
    L.moe_loaded_weight_bytes.argtypes = [P(LayerDesc), _i32, _i32]
    L.moe_loaded_weight_bytes.restype = ctypes.c_uint64
    L.moe_stream_read.argtypes = [_vp, _sz, _vp, _vp]
    L.moe_stream_read.restype = _i32
    L.moe_layer_kernel_count.argtypes = [P(LayerDesc), _i32]
    L.moe_layer_kernel_count.restype = _i32
    L.moe_layer_launch_workitems.argtypes = [P(LayerDesc), _i32, _i32]
    L.moe_layer_launch_workitems.restype = ctypes.c_int64
    _LIB = L
    return L


def moe_stream_read(src: torch.Tensor, sink: torch.Tensor):
    """Measurement helper: read `src` (bf16, a multiple of 16 KiB) once;
    sink[b] = sum of the bf16 values of its 16 KiB block b."""
    nbytes = src.numel() * src.element_size()
    if src.dtype != torch.bfloat16 or not src.is_contiguous():
        raise ValueError("src must be a contiguous bf16 tensor")
    if sink.dtype != torch.float32 or sink.numel() < nbytes // 16384:
        raise ValueError("sink needs one float per 16 KiB of src")
    _check(lib().moe_stream_read(src.data_ptr(), nbytes, sink.data_ptr(), _stream(src.device)),
           "moe_stream_read")


def moe_status_string(status: int) -> str:
    return lib().moe_status_string(int(status)).decode()


def _check(status: int, call: str):
    if status != MOE_OK:
        raise MoeError(status, call)


def layer_desc(d_model: int, n_experts: int, top_k: int, d_ff: int, *, n_depts: int = 0,
               d_ff_dept: int = 0, d_ff_shared: int = 0, score: str = "softmax",
               renormalize: bool = True, route_scale: float = 1.0, dtype: str = "bf16",
               max_tokens: int = 32, dept_form: str = "slice", k_dept: int = 0,
               dept_strict: bool = False, expert_dtype: str = "") -> LayerDesc:
    """dtype: weights and activations ("bf16" | "f32"); expert_dtype "fp8":
    the expert matrices are E4M3 codes with per-row scales (bf16 only)."""
    dt = MOE_BF16 if dtype == "bf16" else MOE_F32
    wdt = MOE_FP8_E4M3 if expert_dtype == "fp8" else dt
    return LayerDesc(d_model, n_experts, top_k, d_ff, n_depts, d_ff_dept, d_ff_shared,
                     SCORE_FNS[score], int(bool(renormalize)), float(route_scale), wdt, dt,
                     max_tokens, DEPT_FORMS[dept_form], k_dept, int(dept_strict))


def moe_validate_desc(desc: LayerDesc) -> int:
    return lib().moe_validate_desc(ctypes.byref(desc))


def moe_workspace_bytes(desc: LayerDesc) -> int:
    n = lib().moe_workspace_bytes(ctypes.byref(desc))
    if n == 0:
        _check(moe_validate_desc(desc) or MOE_ERR_INVALID_ARG, "moe_workspace_bytes")
    return n


def moe_loaded_weight_bytes(desc: LayerDesc, n_active: int, n_active_depts: int = 0) -> int:
    return int(lib().moe_loaded_weight_bytes(ctypes.byref(desc), n_active, n_active_depts))


def moe_layer_kernel_count(desc: LayerDesc, T: int) -> int:
    """Kernels moe_layer_decode launches for T tokens (4: the down launch
    writes y itself and the combine stage is empty)."""
    return int(lib().moe_layer_kernel_count(ctypes.byref(desc), T))


def moe_layer_launch_workitems(desc: LayerDesc, T: int, stage: int) -> int:
    """Work-items of the gate/up (STAGE_GATEUP) or down (STAGE_DOWN) launch of
    a decode step of T tokens, as a profiler's kernel trace reports its grid
    (0 where not reported: FP8 weights, the factorised form)."""
    return int(lib().moe_layer_launch_workitems(ctypes.byref(desc), T, stage))


def moe_workspace_init(desc: LayerDesc, workspace: torch.Tensor):
    st = lib().moe_workspace_init(ctypes.byref(desc), _ptr(workspace, "workspace", torch.uint8),
                                  workspace.numel(), _stream(workspace.device))
    _check(st, "moe_workspace_init")


def alloc_workspace(desc: LayerDesc, device="cuda") -> torch.Tensor:
    """A device workspace of moe_workspace_bytes(desc) bytes (torch-owned),
    initialised with moe_workspace_init."""
    ws = torch.empty(moe_workspace_bytes(desc), dtype=torch.uint8, device=device)
    moe_workspace_init(desc, ws)
    return ws


# ---------------------------------------------------------------------------
# tensor -> pointer marshalling
# ---------------------------------------------------------------------------

def _ptr(t: Optional[torch.Tensor], name: str, dtype=None, shape: Optional[Sequence[int]] = None,
         device=None):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor (got {t.device})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype} (got {t.dtype})")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)} (got {tuple(t.shape)})")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    return t.data_ptr()


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _wdt(desc):
    """torch dtype of the expert matrices (FP8: their raw E4M3 codes)."""
    if desc.w_dtype == MOE_FP8_E4M3:
        return torch.uint8
    return torch.bfloat16 if desc.w_dtype == MOE_BF16 else torch.float32


def _rdt(desc):
    """torch dtype of the router (the activation dtype next to FP8 experts)."""
    return desc.torch_dtype if desc.w_dtype == MOE_FP8_E4M3 else _wdt(desc)


def _weights_struct(desc: LayerDesc, w: Dict[str, torch.Tensor]) -> Weights:
    E, d, I = desc.n_experts, desc.d_model, desc.d_ff
    wdt = _wdt(desc)
    s = Weights()
    shapes = {"w_gate": (E, I, d), "w_up": (E, I, d), "w_down": (E, d, I)}
    if w.get("w_router") is not None:
        s.w_router = _ptr(w["w_router"], "w_router", _rdt(desc), (E, d))
    if desc.n_depts and desc.dept_form == MOE_DEPT_FACTORISED:
        # private transforms A_g, A_u and (A_d)^T are S x S (I == S)
        shapes.update(w_gate=(E, I, I), w_up=(E, I, I), w_down=(E, I, I))
    if desc.n_depts:
        m, S = desc.n_depts, desc.d_ff_dept
        shapes.update(wd_gate=(m, S, d), wd_up=(m, S, d), wd_down=(m, d, S))
    if desc.d_ff_shared:
        Is = desc.d_ff_shared
        shapes.update(ws_gate=(Is, d), ws_up=(Is, d), ws_down=(d, Is))
    for name, shp in shapes.items():
        if name in w and w[name] is not None:
            setattr(s, name, _ptr(w[name], name, wdt, shp))
            if desc.w_dtype == MOE_FP8_E4M3:  # one fp32 scale per output row
                sc = w.get(name + "_scale")
                setattr(s, name + "_scale",
                        _ptr(sc, name + "_scale", torch.float32, shp[:-1]) if sc is not None
                        else None)
    if w.get("router_bias") is not None:
        s.router_bias = _ptr(w["router_bias"], "router_bias", torch.float32, (E,))
    return s


def _ws(desc, workspace):
    return _ptr(workspace, "workspace", torch.uint8), workspace.numel()


def moe_route(desc: LayerDesc, x: torch.Tensor, w_router: torch.Tensor,
              router_bias: Optional[torch.Tensor], topk_ids: torch.Tensor, topk_w: torch.Tensor,
              workspace: torch.Tensor, sel_scores: Optional[torch.Tensor] = None):
    T = x.shape[0]
    E, k, d = desc.n_experts, desc.top_k, desc.d_model
    wsp, wsn = _ws(desc, workspace)
    st = lib().moe_route(
        ctypes.byref(desc), _ptr(x, "x", desc.torch_dtype, (T, d)),
        _ptr(w_router, "w_router", _rdt(desc), (E, d)),
        _ptr(router_bias, "router_bias", torch.float32, (E,)), T,
        _ptr(topk_ids, "topk_ids", torch.int32, (T, k)),
        _ptr(topk_w, "topk_w", torch.float32, (T, k)),
        _ptr(sel_scores, "sel_scores", torch.float32, (T, E)), wsp, wsn, _stream(x.device))
    _check(st, "moe_route")


def moe_dispatch(desc: LayerDesc, topk_ids: torch.Tensor, topk_w: torch.Tensor,
                 workspace: torch.Tensor) -> Plan:
    T, k = topk_ids.shape[0], desc.top_k
    plan = Plan()
    wsp, wsn = _ws(desc, workspace)
    st = lib().moe_dispatch(ctypes.byref(desc), _ptr(topk_ids, "topk_ids", torch.int32, (T, k)),
                            _ptr(topk_w, "topk_w", torch.float32, (T, k)), T, wsp, wsn,
                            ctypes.byref(plan), _stream(topk_ids.device))
    _check(st, "moe_dispatch")
    return plan


def moe_expert_ffn(desc: LayerDesc, weights: Dict[str, torch.Tensor], x: torch.Tensor,
                   plan: Plan, workspace: torch.Tensor, row_out: torch.Tensor,
                   dept_out: Optional[torch.Tensor] = None,
                   shared_out: Optional[torch.Tensor] = None):
    T, d = x.shape[0], desc.d_model
    ws = _weights_struct(desc, weights)
    wsp, wsn = _ws(desc, workspace)
    st = lib().moe_expert_ffn(
        ctypes.byref(desc), ctypes.byref(ws), _ptr(x, "x", desc.torch_dtype, (T, d)), T,
        ctypes.byref(plan), wsp, wsn, _ptr(row_out, "row_out", torch.float32),
        _ptr(dept_out, "dept_out", torch.float32),
        _ptr(shared_out, "shared_out", torch.float32, (T, d) if shared_out is not None else None),
        _stream(x.device))
    _check(st, "moe_expert_ffn")


def moe_combine(desc: LayerDesc, plan: Plan, row_out: torch.Tensor,
                dept_out: Optional[torch.Tensor], shared_out: Optional[torch.Tensor],
                y: torch.Tensor):
    T, d = y.shape[0], desc.d_model
    st = lib().moe_combine(
        ctypes.byref(desc), ctypes.byref(plan), _ptr(row_out, "row_out", torch.float32),
        _ptr(dept_out, "dept_out", torch.float32),
        _ptr(shared_out, "shared_out", torch.float32), T,
        _ptr(y, "y", desc.torch_dtype, (T, d)), _stream(y.device))
    _check(st, "moe_combine")


def alloc_step_stats(device="cuda") -> torch.Tensor:
    """Device storage for one moe_step_stats (8-byte aligned, torch-owned)."""
    return torch.zeros(STEP_STATS_BYTES // 8, dtype=torch.int64, device=device)


def step_stats_to_host(stats: torch.Tensor, n_experts: int) -> Dict[str, "object"]:
    """Copy a moe_step_stats from the device (synchronising) into a dict;
    expert_rows trimmed to the first n_experts entries."""
    raw = stats.cpu().numpy().tobytes()
    st = StepStats.from_buffer_copy(raw[:STEP_STATS_BYTES])
    out = {name: getattr(st, name) for name, _ in StepStats._fields_ if name != "expert_rows"}
    out["expert_rows"] = list(st.expert_rows[:n_experts])
    return out


def _stats_ptr(stats: Optional[torch.Tensor], device):
    if stats is None:
        return None
    if stats.numel() * stats.element_size() < STEP_STATS_BYTES:
        raise ValueError(f"stats needs {STEP_STATS_BYTES} bytes")
    return _ptr(stats, "stats", device=device)


def moe_layer_decode(desc: LayerDesc, weights: Dict[str, torch.Tensor], x: torch.Tensor,
                     y: torch.Tensor, workspace: torch.Tensor, stats: Optional[torch.Tensor] = None):
    """y[T][d] = the layer on x[T][d]; `stats` (alloc_step_stats()) receives
    the step's routing statistics on the device when given."""
    T, d = x.shape[0], desc.d_model
    ws = _weights_struct(desc, weights)
    wsp, wsn = _ws(desc, workspace)
    st = lib().moe_layer_decode(
        ctypes.byref(desc), ctypes.byref(ws), _ptr(x, "x", desc.torch_dtype, (T, d)), T,
        _ptr(y, "y", desc.torch_dtype, (T, d)), wsp, wsn, _stats_ptr(stats, x.device),
        _stream(x.device))
    _check(st, "moe_layer_decode")


def moe_layer_decode_timed(desc: LayerDesc, weights: Dict[str, torch.Tensor], x: torch.Tensor,
                           y: torch.Tensor, workspace: torch.Tensor, stage_events=None,
                           stats: Optional[torch.Tensor] = None):
    """moe_layer_decode with kernel timing.  stage_events: None or a sequence
    of 2 * N_STAGES torch.cuda.Event(enable_timing=True), each recorded once
    beforehand (so it exists); pairs (start, stop) bracket each stage's
    kernel exactly."""
    T, d = x.shape[0], desc.d_model
    ws = _weights_struct(desc, weights)
    wsp, wsn = _ws(desc, workspace)
    ev = None
    if stage_events is not None:
        if len(stage_events) != 2 * N_STAGES:
            raise ValueError(f"stage_events needs {2 * N_STAGES} events")
        ev = (_vp * (2 * N_STAGES))(*[e.cuda_event for e in stage_events])
    st = lib().moe_layer_decode_timed(
        ctypes.byref(desc), ctypes.byref(ws), _ptr(x, "x", desc.torch_dtype, (T, d)), T,
        _ptr(y, "y", desc.torch_dtype, (T, d)), wsp, wsn, _stats_ptr(stats, x.device), ev,
        _stream(x.device))
    _check(st, "moe_layer_decode_timed")


def moe_layer_decode_noalloc(desc: LayerDesc, weights: Dict[str, torch.Tensor], x: torch.Tensor,
                             y: torch.Tensor, stats: Optional[torch.Tensor] = None):
    """moe_layer_decode without a workspace: the library's fixed per-GPU
    scratch holds the intermediates (no device allocation in the call).
    Calls that overlap on one GPU race; order them on one stream."""
    T, d = x.shape[0], desc.d_model
    ws = _weights_struct(desc, weights)
    st = lib().moe_layer_decode_noalloc(
        ctypes.byref(desc), ctypes.byref(ws), _ptr(x, "x", desc.torch_dtype, (T, d)), T,
        _ptr(y, "y", desc.torch_dtype, (T, d)), _stats_ptr(stats, x.device), _stream(x.device))
    _check(st, "moe_layer_decode_noalloc")


def plan_to_host(desc: LayerDesc, plan: Plan, workspace: torch.Tensor) -> Dict[str, "object"]:
    """Copy the plan arrays a dispatch wrote into `workspace` to host numpy
    arrays, trimmed to their valid lengths (synchronising copy)."""
    import numpy as np
    T, k, E, m = plan.n_tokens, desc.top_k, desc.n_experts, desc.n_depts
    base = workspace.data_ptr()

    def rd(name, n, dt):
        off = getattr(plan, name) - base
        if off < 0 or off + 4 * n > workspace.numel():
            raise ValueError(f"plan array {name} lies outside the workspace")
        raw = workspace[off:off + 4 * n].view(torch.int32 if dt == "i" else torch.float32)
        return raw.cpu().numpy().astype(np.int32 if dt == "i" else np.float32)

    hdr = rd("header", PLAN_HEADER_LEN, "i")
    n_rows, n_act = int(hdr[PLAN_N_ROWS]), int(hdr[PLAN_N_ACTIVE])
    out = dict(header=hdr, n_rows=n_rows, n_invalid=int(hdr[PLAN_N_INVALID]),
               counts=rd("counts", E, "i"), offsets=rd("offsets", E + 1, "i"),
               row_token=rd("row_token", n_rows, "i"), row_slot=rd("row_slot", n_rows, "i"),
               row_expert=rd("row_expert", n_rows, "i"), row_weight=rd("row_weight", n_rows, "f"),
               inv_perm=rd("inv_perm", T * k, "i"), active=rd("active", n_act, "i"))
    if m:
        nd, nad = int(hdr[PLAN_N_DEPT_ROWS]), int(hdr[PLAN_N_ACTIVE_DEPTS])
        out.update(n_dept_rows=nd, dept_counts=rd("dept_counts", m, "i"),
                   dept_offsets=rd("dept_offsets", m + 1, "i"),
                   dept_row_token=rd("dept_row_token", nd, "i"),
                   dept_row_dept=rd("dept_row_dept", nd, "i"),
                   dept_row_scale=rd("dept_row_scale", nd, "f"),
                   dept_inv=rd("dept_inv", T * m, "i"),
                   active_depts=rd("active_depts", nad, "i"))
        if desc.dept_form == MOE_DEPT_FACTORISED:
            out["row_pair"] = rd("row_pair", n_rows, "i")
    return out


class MoeLayer:
    """One layer's descriptor, weights and workspace on one device."""

    def __init__(self, desc: LayerDesc, weights: Dict[str, torch.Tensor], device="cuda"):
        self.desc = desc
        self.weights = weights
        self.device = torch.device(device)
        self.workspace = alloc_workspace(desc, self.device)

    def __call__(self, x: torch.Tensor, y: Optional[torch.Tensor] = None, stage_events=None,
                 stats: Optional[torch.Tensor] = None):
        if y is None:
            y = torch.empty_like(x)
        if stage_events is None:
            moe_layer_decode(self.desc, self.weights, x, y, self.workspace, stats)
        else:
            moe_layer_decode_timed(self.desc, self.weights, x, y, self.workspace, stage_events,
                                   stats)
        return y

    def plan(self, T: int) -> Dict[str, "object"]:
        """The plan the last call wrote (host copy)."""
        p = Plan()
        _check(lib().moe_plan_from_workspace(ctypes.byref(self.desc),
                                             _vp(self.workspace.data_ptr()),
                                             self.workspace.numel(), T, ctypes.byref(p)),
               "moe_plan_from_workspace")
        return plan_to_host(self.desc, p, self.workspace)
