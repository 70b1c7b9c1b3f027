"""The allocation-free decode entry point (for callers that cannot allocate
device memory) against moe_layer_decode with a caller workspace: the same
kernels on the same inputs, so y and the step statistics must agree bit for
bit, on two calls in a row, the second with fewer tokens (the scratch keeps
the first call's contents)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import moe_layer_decode_amd as M
import moe_synth

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def _desc(shape, max_tokens):
    return M.layer_desc(shape.d, shape.n_experts, shape.top_k, shape.d_ff, n_depts=shape.n_depts,
                        d_ff_dept=shape.d_ff_dept, d_ff_shared=shape.d_ff_shared,
                        score=shape.score, renormalize=shape.renormalize,
                        route_scale=shape.route_scale, dtype=shape.dtype, max_tokens=max_tokens,
                        dept_form=shape.dept_form, k_dept=shape.k_dept,
                        dept_strict=shape.dept_strict, expert_dtype=shape.expert_dtype)


@pytest.mark.parametrize("name,T1,T2", [
    ("qwen3_30b_a3b_d2048_e128_i768_top8", 16, 3),
    ("deamoe_7b_d2048_e64_m8_s1024_p128_top8", 16, 1),
    ("tiny_d256_e8_i128_top2", 4, 2),
])
def test_noalloc_matches_workspace_call(name, T1, T2):
    M.lib()
    shape = moe_synth.SHAPES[name]
    w = moe_synth.make_layer(shape, 0, DEV)
    desc = _desc(shape, T1)
    ws = M.alloc_workspace(desc, DEV)
    for T in (T1, T2):
        x = moe_synth.make_tokens(shape, 1, T, DEV)
        y_ref = torch.full_like(x, float("nan"))
        s_ref = M.alloc_step_stats(DEV)
        M.moe_layer_decode(desc, w, x, y_ref, ws, s_ref)
        y = torch.full_like(x, float("nan"))
        s = M.alloc_step_stats(DEV)
        M.moe_layer_decode_noalloc(desc, w, x, y, s)
        torch.cuda.synchronize()
        print(f"{name} T={T}: noalloc vs workspace call", flush=True)
        assert torch.isfinite(y.float()).all()
        assert torch.equal(y, y_ref), f"{name} T={T}: y differs"
        a = M.step_stats_to_host(s, shape.n_experts)
        b = M.step_stats_to_host(s_ref, shape.n_experts)
        assert a == b, f"{name} T={T}: stats differ"
