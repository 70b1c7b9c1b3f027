"""Seeded synthetic inputs for the MoE decode layer.

This module only draws numbers: it holds none of the layer's arithmetic, so
both the HIP path and the CPU oracle can take their inputs from it without
sharing any computation.

Every value is a pure function of (seed, tensor id, flat element index): a
counter-based hash (Chris Wellons' "lowbias32" integer mixer) turns the
counter into two 32-bit words, and the Box-Muller transform turns them into a
standard normal.  The same call therefore gives the same tensor in any chunking
and on any device, up to the last bit of the fp64 transcendental functions
(which the final rounding to fp32/bf16 almost always absorbs).  Rounding to
bf16 is round-to-nearest-even (torch's own conversion).

Layer shapes
------------
The layer shapes follow the workloads the pages name (Qwen3-30B-A3B,
DeepSeek-V3, the DeaMoE department layer in slice form, and DeaMoE's own
factorised experts at its DeepSeek-V3-matched configuration); the value
distributions follow the pages' own routers: router and expert weights
N(0, 0.02) (the router initialisation in the DeepSeekMoE guide's PyTorch
layer), activations N(0, 1) except the tiny layer (N(0, 0.02)), selection bias
U(-0.1, 0.1); factorised private transforms are the identity DeaMoE starts
them from plus N(0, 0.02).

FP8 expert weights (shapes with expert_dtype "fp8") are the same fp32 draws
stored as OCP E4M3 codes with one fp32 scale per output row: the scale is the
row's largest magnitude over 448 (the largest E4M3 value), and the codes are
torch's float8_e4m3fn rounding of the row divided by its scale.  This is
input preparation (an offline weight format), not the layer's arithmetic.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional

import torch

__all__ = [
    "LayerShape", "SHAPES", "normal", "uniform", "make_layer", "make_tokens",
    "clone_weights", "E4M3_MAX",
]

_MASK32 = 0xFFFFFFFF


@dataclasses.dataclass(frozen=True)
class LayerShape:
    """Sizes and routing rule of one MoE FFN layer.

    d: hidden width; n_experts: routed experts; top_k: experts per token;
    d_ff: SwiGLU intermediate of a routed expert (the private slice width in the
    department variant); n_depts: departments (0 = vanilla); d_ff_dept: width
    of the department-shared slice; d_ff_shared: width of the always-on shared
    expert (0 = none); score: "softmax" | "sigmoid" | "softmax_bias".
    """
    name: str
    d: int
    n_experts: int
    top_k: int
    d_ff: int
    n_depts: int = 0
    d_ff_dept: int = 0
    d_ff_shared: int = 0
    score: str = "softmax"
    renormalize: bool = True
    route_scale: float = 1.0
    dtype: str = "bf16"            # weights and activations
    dept_form: str = "slice"       # "slice" | "factorised" (private S x S transforms)
    a_std: float = 0.02            # factorised: private transforms = I + N(0, a_std)
    k_dept: int = 0                # department-limited top-k cap (0 = none)
    dept_strict: bool = False      # exactly k_dept departments per token
    x_std: float = 1.0
    w_std: float = 0.02
    bias_range: float = 0.0        # U(-r, r) selection bias when > 0
    batches: tuple = (1, 4, 16)
    data_seed_of: Optional[str] = None  # reuse x / router / bias of this shape
    expert_dtype: str = ""         # "" = dtype; "fp8": E4M3 codes + per-row fp32 scales

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16


SHAPES: Dict[str, LayerShape] = {
    # Tiny fp32 layer: d=256, 8 experts, I=128, top-2 softmax, 4 tokens.
    "tiny_d256_e8_i128_top2": LayerShape(
        name="tiny_d256_e8_i128_top2", d=256, n_experts=8, top_k=2, d_ff=128,
        dtype="f32", x_std=0.02, batches=(4,)),
    # Qwen3-30B-A3B-shaped: d=2048, 128 experts, I=768, top-8 softmax.
    "qwen3_30b_a3b_d2048_e128_i768_top8": LayerShape(
        name="qwen3_30b_a3b_d2048_e128_i768_top8", d=2048, n_experts=128,
        top_k=8, d_ff=768, batches=(1, 4, 16)),
    # DeepSeek-V3-shaped: d=7168, 256 experts, I=2048, shared 2048,
    # sigmoid scores with selection bias, top-8.
    "deepseek_v3_d7168_e256_i2048_s2048_top8": LayerShape(
        name="deepseek_v3_d7168_e256_i2048_s2048_top8", d=7168,
        n_experts=256, top_k=8, d_ff=2048, d_ff_shared=2048, score="sigmoid",
        bias_range=0.1, batches=(1, 2, 4, 8, 16, 32, 64, 128)),
    # DeaMoE department layer at 7.3B scale: 64 experts in 8 departments,
    # intermediate [shared 1024 ; private 128], top-8 softmax.
    "deamoe_7b_d2048_e64_m8_s1024_p128_top8": LayerShape(
        name="deamoe_7b_d2048_e64_m8_s1024_p128_top8", d=2048, n_experts=64,
        top_k=8, d_ff=128, n_depts=8, d_ff_dept=1024, batches=(1, 4, 16)),
    # DeaMoE transform of the DeepSeek-V3-shaped layer: 256 experts in 32
    # departments, intermediate [shared 1792 ; private 256], shared expert 2048,
    # sigmoid + bias top-8; same tokens, router and bias as that layer.
    "deamoe_dsv3_d7168_e256_m32_s1792_p256_top8": LayerShape(
        name="deamoe_dsv3_d7168_e256_m32_s1792_p256_top8", d=7168,
        n_experts=256, top_k=8, d_ff=256, n_depts=32, d_ff_dept=1792,
        d_ff_shared=2048, score="sigmoid", bias_range=0.1,
        batches=(1, 2, 4, 8, 16, 32, 64, 128),
        data_seed_of="deepseek_v3_d7168_e256_i2048_s2048_top8"),
    # DeaMoE's own factorised experts at the DeepSeek-V3-matched configuration
    # of its Table 1 (8 departments x 108 experts, h = 7168, hffn = 2048,
    # k = 10 within k_dept = 5 departments), softmax routing (Eq. (2)-(3));
    # DeepSeek-V3's tokens and shared expert.
    "deamoe_paper_dsv3_d7168_e864_m8_h2048_top10": LayerShape(
        name="deamoe_paper_dsv3_d7168_e864_m8_h2048_top10", d=7168,
        n_experts=864, top_k=10, d_ff=2048, n_depts=8, d_ff_dept=2048,
        d_ff_shared=2048, dept_form="factorised", k_dept=5, batches=(1, 2, 4, 8, 16, 32, 64, 128),
        data_seed_of="deepseek_v3_d7168_e256_i2048_s2048_top8"),
    # The Qwen3-30B-A3B- and DeepSeek-V3-shaped layers with FP8 expert weights
    # (same draws, quantized per output row; router and activations bf16).
    "qwen3_30b_a3b_d2048_e128_i768_top8_fp8": LayerShape(
        name="qwen3_30b_a3b_d2048_e128_i768_top8_fp8", d=2048, n_experts=128,
        top_k=8, d_ff=768, batches=(1, 4, 16), expert_dtype="fp8"),
    "deepseek_v3_d7168_e256_i2048_s2048_top8_fp8": LayerShape(
        name="deepseek_v3_d7168_e256_i2048_s2048_top8_fp8", d=7168,
        n_experts=256, top_k=8, d_ff=2048, d_ff_shared=2048, score="sigmoid",
        bias_range=0.1, batches=(1, 2, 4, 8, 16, 32, 64, 128), expert_dtype="fp8"),
}

# Tensor ids: part of the counter, so every tensor of a layer draws its own
# stream.  Shapes that share tokens/router/bias use the same ids for them.
_TID = {"x": 1, "w_router": 2, "router_bias": 3, "w_gate": 10, "w_up": 11,
        "w_down": 12, "wd_gate": 20, "wd_up": 21, "wd_down": 22,
        "ws_gate": 30, "ws_up": 31, "ws_down": 32}


def _mul32(x: torch.Tensor, c: int) -> torch.Tensor:
    """(x * c) mod 2**32 for int64 tensors holding values < 2**32, without
    signed overflow: split c into 16-bit halves."""
    lo, hi = c & 0xFFFF, c >> 16
    return (x * lo + (((x * hi) & 0xFFFF) << 16)) & _MASK32


def _lowbias32(x: torch.Tensor) -> torch.Tensor:
    x = x ^ (x >> 16)
    x = _mul32(x, 0x7FEB352D)
    x = x ^ (x >> 15)
    x = _mul32(x, 0x846CA68B)
    x = x ^ (x >> 16)
    return x


def _key(seed: int, tid: int, stream: int) -> int:
    """Scalar key of one (seed, tensor, stream) triple, mixed on the host."""
    v = torch.tensor([(seed * 0x9E3779B1 + tid * 0x85EBCA77 + stream * 0xC2B2AE3D)
                      & _MASK32], dtype=torch.int64)
    return int(_lowbias32(_lowbias32(v) ^ 0x27D4EB2F)[0])


def _words(idx: torch.Tensor, key: int) -> torch.Tensor:
    """One 32-bit word per 64-bit counter value."""
    hi = _lowbias32((idx >> 32) ^ key)
    return _lowbias32((idx & _MASK32) ^ hi)


def _chunk_elems(device) -> int:
    return (1 << 26) if torch.device(device).type == "cuda" else (1 << 22)


def _fill(out: torch.Tensor, seed: int, tid: int, fn, offset: int = 0) -> torch.Tensor:
    """Fill `out` with elements [offset, offset + out.numel()) of the
    tensor's stream."""
    flat = out.view(-1)
    n = flat.numel()
    step = _chunk_elems(out.device)
    ka, kb = _key(seed, tid, 1), _key(seed, tid, 2)
    for s in range(0, n, step):
        e = min(n, s + step)
        idx = torch.arange(s + offset, e + offset, dtype=torch.int64, device=out.device)
        ua = (_words(idx, ka).to(torch.float64) + 0.5) * (1.0 / 4294967296.0)
        ub = (_words(idx, kb).to(torch.float64) + 0.5) * (1.0 / 4294967296.0)
        flat[s:e] = fn(ua, ub).to(out.dtype)
    return out


def normal(seed: int, tid: int, shape, std: float, dtype=torch.float32,
           device="cpu", mean: float = 0.0, offset: int = 0) -> torch.Tensor:
    """N(mean, std^2) samples, rounded once to `dtype`; `offset` starts at
    that flat element of the stream (a slice of a larger tensor)."""
    out = torch.empty(shape, dtype=dtype, device=device)

    def bm(ua, ub):
        return torch.sqrt(-2.0 * torch.log(ua)) * torch.cos(2.0 * math.pi * ub) * std + mean
    return _fill(out, seed, tid, bm, offset)


E4M3_MAX = 448.0  # largest finite OCP E4M3 value


def _normal_fp8(seed: int, tid: int, shape, std: float, device):
    """The fp32 N(0, std^2) draws of `shape` as E4M3 codes (uint8) and one
    fp32 scale per row of the last dimension, generated one leading slice at
    a time so no full fp32 copy is held."""
    shape = tuple(shape)
    codes = torch.empty(shape, dtype=torch.uint8, device=device)
    scales = torch.empty(shape[:-1], dtype=torch.float32, device=device)
    lead = shape[0] if len(shape) == 3 else 1
    per = int(math.prod(shape[1:])) if len(shape) == 3 else int(math.prod(shape))
    cv = codes.view(lead, *shape[-2:])
    sv = scales.view(lead, shape[-2])
    for i in range(lead):
        w = normal(seed, tid, shape[-2:], std, torch.float32, device, offset=i * per)
        amax = w.abs().amax(dim=-1)
        sc = torch.where(amax > 0, amax / E4M3_MAX, torch.ones_like(amax))
        q = (w / sc[:, None]).clamp(-E4M3_MAX, E4M3_MAX).to(torch.float8_e4m3fn)
        cv[i] = q.view(torch.uint8)
        sv[i] = sc
    return codes, scales


def uniform(seed: int, tid: int, shape, lo: float, hi: float,
            dtype=torch.float32, device="cpu") -> torch.Tensor:
    """U(lo, hi) samples, rounded once to `dtype`."""
    out = torch.empty(shape, dtype=dtype, device=device)
    return _fill(out, seed, tid, lambda ua, ub: lo + (hi - lo) * ua)


def make_tokens(shape: LayerShape, seed: int, T: int, device="cpu") -> torch.Tensor:
    """Decode-step activations x[T][d] (the first T rows of one long stream,
    so batch T is a prefix of batch T' > T)."""
    src = SHAPES[shape.data_seed_of] if shape.data_seed_of else shape
    return normal(seed, _TID["x"], (T, src.d), src.x_std, shape.torch_dtype, device)


def make_layer(shape: LayerShape, seed: int, device="cpu",
               router_only: bool = False) -> Dict[str, torch.Tensor]:
    """All weights of one layer, in the layout the library takes:
    router [E][d]; gate/up [E][I][d]; down [E][d][I] (nn.Linear out x in);
    department gate/up [m][S][d], down [m][d][S]; shared gate/up [Is][d],
    down [d][Is]; bias fp32 [E].  router_only: just router and bias."""
    dt = shape.torch_dtype
    src = SHAPES[shape.data_seed_of] if shape.data_seed_of else shape
    E, d, I = shape.n_experts, shape.d, shape.d_ff
    w = {}
    w["w_router"] = normal(seed, _TID["w_router"], (E, d), src.w_std, dt, device)
    if shape.bias_range > 0:
        w["router_bias"] = uniform(seed, _TID["router_bias"], (E,),
                                   -src.bias_range, src.bias_range,
                                   torch.float32, device)
    if router_only:
        return w
    # Expert tensors of a transformed layer draw from their own seed space so
    # they are not a slice of the source layer's experts.
    eseed = seed if not shape.data_seed_of else seed + 7919
    if shape.dept_form == "factorised":
        # private transforms A_g, A_u and (A_d)^T, [E][S][S]: the identity the
        # pages start them from, plus N(0, a_std); rounded once to dtype
        for name in ("w_gate", "w_up", "w_down"):
            a = normal(eseed, _TID[name], (E, I, I), shape.a_std, torch.float32, device)
            a.diagonal(dim1=1, dim2=2).add_(1.0)
            w[name] = a.to(dt)
            del a
    else:
        mat(w, "w_gate", eseed, (E, I, d), shape, dt, device)
        mat(w, "w_up", eseed, (E, I, d), shape, dt, device)
        mat(w, "w_down", eseed, (E, d, I), shape, dt, device)
    if shape.n_depts:
        m, S = shape.n_depts, shape.d_ff_dept
        mat(w, "wd_gate", eseed, (m, S, d), shape, dt, device)
        mat(w, "wd_up", eseed, (m, S, d), shape, dt, device)
        mat(w, "wd_down", eseed, (m, d, S), shape, dt, device)
    if shape.d_ff_shared:
        Is = shape.d_ff_shared
        # The shared expert is the source layer's own (same seed space), so a
        # transformed layer keeps its shared expert.
        mat(w, "ws_gate", seed, (Is, d), shape, dt, device)
        mat(w, "ws_up", seed, (Is, d), shape, dt, device)
        mat(w, "ws_down", seed, (d, Is), shape, dt, device)
    return w


def mat(w: Dict[str, torch.Tensor], name: str, seed: int, shape, layer: LayerShape, dt,
        device) -> None:
    """One expert matrix into w: in the layer dtype, or (FP8 layers) as E4M3
    codes under `name` and per-row fp32 scales under name + "_scale"."""
    if layer.expert_dtype == "fp8":
        w[name], w[name + "_scale"] = _normal_fp8(seed, _TID[name], shape, layer.w_std, device)
    else:
        w[name] = normal(seed, _TID[name], shape, layer.w_std, dt, device)


def clone_weights(w: Dict[str, torch.Tensor]) -> Dict[str, torch.Tensor]:
    """A replica of a layer at fresh addresses (same values)."""
    return {k: v.clone() for k, v in w.items()}
