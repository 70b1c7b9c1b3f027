"""Host-side checks of the C ABI: the library loads, exports every declared
symbol, and validates descriptors without touching a GPU."""
import ctypes
import os
import re

import pytest

import moe_layer_decode_amd as M

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    with open(os.path.join(ROOT, "include", "moe_decode.h")) as f:
        src = f.read()
    return sorted(set(re.findall(
        r"^(?:const char\*|size_t|moe_status|uint64_t|int64_t|int32_t)\s+(moe_\w+)\(", src, re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(M.lib_path()):
        import moe_layer_decode_amd.build as B
        B.build()
    return M.lib()


def test_header_declares_the_calls():
    decl = _declared_functions()
    for name in ("moe_route", "moe_dispatch", "moe_expert_ffn", "moe_combine",
                 "moe_layer_decode", "moe_workspace_bytes", "moe_workspace_init",
                 "moe_status_string"):
        assert name in decl
    assert sorted(M.EXPORTED_SYMBOLS) == decl


def test_library_exports_every_declared_symbol(lib):
    for name in _declared_functions():
        assert hasattr(lib, name), name
        assert ctypes.cast(getattr(lib, name), ctypes.c_void_p).value


def test_status_strings(lib):
    for s in range(5):
        assert M.moe_status_string(s)
    assert M.moe_status_string(99) == "unknown status"


def _desc(**kw):
    base = dict(d_model=2048, n_experts=128, top_k=8, d_ff=768)
    base.update(kw)
    d, E, k, I = base.pop("d_model"), base.pop("n_experts"), base.pop("top_k"), base.pop("d_ff")
    return M.layer_desc(d, E, k, I, **base)


@pytest.mark.parametrize("kw,status", [
    (dict(), M.MOE_OK),
    (dict(d_model=2047), M.MOE_ERR_INVALID_ARG),
    (dict(d_model=0), M.MOE_ERR_INVALID_ARG),
    (dict(top_k=0), M.MOE_ERR_INVALID_ARG),
    (dict(top_k=129), M.MOE_ERR_INVALID_ARG),
    (dict(d_ff=100), M.MOE_ERR_INVALID_ARG),
    (dict(n_depts=3, d_ff_dept=64), M.MOE_ERR_INVALID_ARG),       # 128 % 3 != 0
    (dict(n_depts=8, d_ff_dept=0), M.MOE_ERR_INVALID_ARG),
    (dict(n_depts=8, d_ff_dept=1024), M.MOE_OK),
    (dict(d_ff_shared=12), M.MOE_ERR_INVALID_ARG),
    (dict(max_tokens=0), M.MOE_ERR_INVALID_ARG),
    (dict(max_tokens=513), M.MOE_ERR_UNSUPPORTED),               # T*k > 4096
    (dict(n_experts=4096, top_k=8), M.MOE_ERR_UNSUPPORTED),
    (dict(top_k=33), M.MOE_ERR_UNSUPPORTED),
    (dict(score="sigmoid", route_scale=float("inf")), M.MOE_ERR_INVALID_ARG),
    # factorised department form: S x S private transforms need d_ff == d_ff_dept
    (dict(n_depts=8, d_ff=1024, d_ff_dept=1024, dept_form="factorised"), M.MOE_OK),
    (dict(n_depts=8, d_ff_dept=1024, dept_form="factorised"), M.MOE_ERR_INVALID_ARG),
    (dict(dept_form="factorised"), M.MOE_ERR_INVALID_ARG),                # needs departments
    # department-limited top-k
    (dict(n_depts=8, d_ff_dept=1024, k_dept=3), M.MOE_OK),
    (dict(n_depts=8, d_ff_dept=1024, k_dept=8), M.MOE_OK),                 # no cap in effect
    (dict(k_dept=1), M.MOE_ERR_INVALID_ARG),                               # needs departments
    (dict(n_depts=8, d_ff_dept=1024, k_dept=9), M.MOE_ERR_INVALID_ARG),    # > n_depts
    (dict(n_depts=8, d_ff_dept=1024, k_dept=-1), M.MOE_ERR_INVALID_ARG),
    (dict(n_depts=64, d_ff_dept=128, top_k=2, k_dept=1), M.MOE_OK),      # k = 1 * (E / m)
    (dict(n_depts=64, d_ff_dept=128, top_k=3, k_dept=1), M.MOE_ERR_INVALID_ARG),  # 3 > 1 * 2
    (dict(n_experts=256, n_depts=128, d_ff_dept=128, top_k=2, k_dept=2),
     M.MOE_ERR_UNSUPPORTED),                                               # > 64 departments
    # strict department coverage
    (dict(n_depts=8, d_ff_dept=1024, k_dept=3, dept_strict=True), M.MOE_OK),
    (dict(n_depts=8, d_ff_dept=1024, k_dept=8, dept_strict=True), M.MOE_OK),  # k = k_dept
    (dict(n_depts=8, d_ff_dept=1024, dept_strict=True), M.MOE_ERR_INVALID_ARG),  # no cap
    (dict(n_depts=8, d_ff_dept=1024, top_k=2, k_dept=3, dept_strict=True),
     M.MOE_ERR_INVALID_ARG),                                               # k < k_dept
])
def test_descriptor_validation(lib, kw, status):
    assert M.moe_validate_desc(_desc(**kw)) == status
    if status != M.MOE_OK:
        assert lib.moe_workspace_bytes(ctypes.byref(_desc(**kw))) == 0


def test_mixed_dtypes_unsupported(lib):
    d = _desc()
    d.w_dtype, d.act_dtype = M.MOE_BF16, M.MOE_F32
    assert M.moe_validate_desc(d) == M.MOE_ERR_UNSUPPORTED


def test_workspace_grows_with_tokens_and_features(lib):
    small = M.moe_workspace_bytes(_desc(max_tokens=1))
    big = M.moe_workspace_bytes(_desc(max_tokens=32))
    assert 0 < small < big
    assert M.moe_workspace_bytes(_desc(d_ff_shared=2048)) > M.moe_workspace_bytes(_desc())
    assert M.moe_workspace_bytes(_desc(n_depts=8, d_ff_dept=1024)) > M.moe_workspace_bytes(_desc())
    assert big % 256 == 0


def test_calls_reject_bad_arguments_before_any_launch(lib):
    """Errors found on the host return before any HIP call: these run on a
    machine without a GPU."""
    d = _desc()
    P = M.Plan()
    nul = None
    # T out of range
    assert lib.moe_dispatch(ctypes.byref(d), 256, 256, 33, 4096, 1 << 30, ctypes.byref(P), nul) \
        == M.MOE_ERR_INVALID_ARG
    # misaligned ids pointer
    assert lib.moe_dispatch(ctypes.byref(d), 258, 256, 1, 4096, 1 << 30, ctypes.byref(P), nul) \
        == M.MOE_ERR_INVALID_ARG
    # workspace too small / misaligned
    assert lib.moe_dispatch(ctypes.byref(d), 256, 256, 1, 4096, 16, ctypes.byref(P), nul) \
        == M.MOE_ERR_WORKSPACE
    assert lib.moe_dispatch(ctypes.byref(d), 256, 256, 1, 4097, 1 << 30, ctypes.byref(P), nul) \
        == M.MOE_ERR_WORKSPACE
    # invalid descriptor wins over everything
    bad = _desc(d_model=7)
    assert lib.moe_route(ctypes.byref(bad), 256, 256, None, 1, 256, 256, None, 4096, 1 << 30,
                         nul) == M.MOE_ERR_INVALID_ARG
    # softmax mode takes no selection bias
    assert lib.moe_route(ctypes.byref(d), 256, 256, 512, 1, 256, 256, None, 4096, 1 << 30,
                         nul) == M.MOE_ERR_INVALID_ARG
    # missing expert weights
    W = M.Weights(w_router=256)
    assert lib.moe_layer_decode(ctypes.byref(d), ctypes.byref(W), 256, 1, 512, 4096, 1 << 30,
                                None, nul) == M.MOE_ERR_INVALID_ARG
    # department layer without department weights
    dd = _desc(n_depts=8, d_ff_dept=1024)
    W = M.Weights(w_router=256, w_gate=256, w_up=256, w_down=256)
    assert lib.moe_layer_decode(ctypes.byref(dd), ctypes.byref(W), 256, 1, 512, 4096, 1 << 30,
                                None, nul) == M.MOE_ERR_INVALID_ARG


def test_stream_read_rejects_bad_arguments(lib):
    assert lib.moe_stream_read(256, 16384 + 16, 256, None) == M.MOE_ERR_INVALID_ARG
    assert lib.moe_stream_read(256, 0, 256, None) == M.MOE_ERR_INVALID_ARG
    assert lib.moe_stream_read(None, 16384, 256, None) == M.MOE_ERR_INVALID_ARG
    assert lib.moe_stream_read(258, 16384, 256, None) == M.MOE_ERR_INVALID_ARG
    assert lib.moe_stream_read(256, 16384, None, None) == M.MOE_ERR_INVALID_ARG


def test_zero_tokens_is_a_noop(lib):
    d = _desc()
    P = M.Plan()
    ws = M.moe_workspace_bytes(d)
    assert lib.moe_dispatch(ctypes.byref(d), 256, 256, 0, 4096, ws, ctypes.byref(P), None) == M.MOE_OK
    assert P.n_tokens == 0
    W = M.Weights(w_router=256, w_gate=256, w_up=256, w_down=256)
    assert lib.moe_layer_decode(ctypes.byref(d), ctypes.byref(W), 256, 0, 512, 4096, ws,
                                None, None) == M.MOE_OK


def test_plan_addresses_inside_workspace(lib):
    d = _desc(n_depts=8, d_ff_dept=1024)
    ws = M.moe_workspace_bytes(d)
    P = M.Plan()
    base = 1 << 20
    assert lib.moe_plan_from_workspace(ctypes.byref(d), base, ws, 4, ctypes.byref(P)) == M.MOE_OK
    addrs = [getattr(P, n) for n in M._PLAN_ARRAYS]
    assert all(base <= a < base + ws for a in addrs)
    assert len(set(addrs)) == len(addrs)


def test_dept_form_field_is_checked(lib):
    d = _desc()
    d.dept_form = 7
    assert M.moe_validate_desc(d) == M.MOE_ERR_INVALID_ARG


def test_factorised_workspace_and_bytes(lib):
    fac = _desc(n_experts=32, top_k=6, d_ff=256, n_depts=4, d_ff_dept=256, dept_form="factorised")
    sl = _desc(n_experts=32, top_k=6, d_ff=256, n_depts=4, d_ff_dept=256)
    assert M.moe_workspace_bytes(fac) > M.moe_workspace_bytes(sl)  # backbone outputs per pair
    # router + 10 private S x S triples + 3 department S x d triples, bf16
    assert M.moe_loaded_weight_bytes(fac, 10, 3) == 2 * (32 * 2048 + 10 * 3 * 256 * 256
                                                         + 3 * 3 * 2048 * 256)


def test_loaded_weight_bytes(lib):
    d = _desc()
    per_expert = 3 * 2048 * 768 * 2
    router = 128 * 2048 * 2
    assert M.moe_loaded_weight_bytes(d, 8) == router + 8 * per_expert
    dd = _desc(n_experts=64, d_ff=128, n_depts=8, d_ff_dept=1024)
    assert M.moe_loaded_weight_bytes(dd, 10, 3) == 2 * (64 * 2048 + 10 * 3 * 2048 * 128
                                                         + 3 * 3 * 2048 * 1024)


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(M, "_LIB", None)
    monkeypatch.setattr(M, "lib_path", lambda: str(tmp_path / "missing.so"))
    with pytest.raises(ImportError, match="no CPU fallback"):
        M.moe_validate_desc(_desc())


@pytest.mark.parametrize("kw,status", [
    (dict(expert_dtype="fp8"), M.MOE_OK),
    (dict(expert_dtype="fp8", d_ff=776), M.MOE_ERR_INVALID_ARG),           # 776 % 16 != 0
    (dict(expert_dtype="fp8", d_model=2056), M.MOE_ERR_INVALID_ARG),
    (dict(expert_dtype="fp8", d_ff_shared=24), M.MOE_ERR_INVALID_ARG),
    (dict(expert_dtype="fp8", n_depts=8, d_ff_dept=1032), M.MOE_ERR_INVALID_ARG),
    (dict(expert_dtype="fp8", n_depts=8, d_ff_dept=1024, d_ff_shared=2048), M.MOE_OK),
    (dict(expert_dtype="fp8", d_model=8192 + 16), M.MOE_ERR_UNSUPPORTED),  # > MOE_FP8_MAX_WIDTH
    (dict(expert_dtype="fp8", d_ff=8192), M.MOE_OK),
    (dict(expert_dtype="fp8", dtype="f32"), M.MOE_ERR_UNSUPPORTED),       # bf16 activations only
    (dict(expert_dtype="fp8", n_depts=8, d_ff=1024, d_ff_dept=1024, dept_form="factorised"),
     M.MOE_ERR_UNSUPPORTED),
])
def test_fp8_descriptor_validation(lib, kw, status):
    assert M.moe_validate_desc(_desc(**kw)) == status


def test_fp8_calls_need_row_scales(lib):
    """An FP8 layer without the per-row scales of a matrix it has is refused
    on the host (no GPU needed)."""
    d = _desc(expert_dtype="fp8", d_ff_shared=2048)
    full = dict(w_router=256, w_gate=256, w_up=256, w_down=256, ws_gate=256, ws_up=256,
                ws_down=256, w_gate_scale=512, w_up_scale=512, w_down_scale=512,
                ws_gate_scale=512, ws_up_scale=512, ws_down_scale=512)
    ws = M.moe_workspace_bytes(d)
    assert lib.moe_layer_decode(ctypes.byref(d), ctypes.byref(M.Weights(**full)), 256, 0, 512,
                                4096, ws, None, None) == M.MOE_OK  # T = 0: valid no-op
    for missing in ("w_down_scale", "ws_gate_scale"):
        W = M.Weights(**{k: v for k, v in full.items() if k != missing})
        assert lib.moe_layer_decode(ctypes.byref(d), ctypes.byref(W), 256, 1, 512, 4096, ws,
                                    None, None) == M.MOE_ERR_INVALID_ARG, missing


def test_fp8_loaded_weight_bytes_match_the_oracle(lib):
    """The library's FP8 byte count equals the oracle's (one byte per expert
    weight, 4 per row scale, the router in bf16) for the plain layer, the
    shared expert and department slices."""
    import numpy as np
    import oracle as O
    for kw, n_act, n_dep in ((dict(), 8, 0), (dict(d_ff_shared=2048), 5, 0),
                             (dict(n_experts=64, d_ff=128, n_depts=8, d_ff_dept=1024), 10, 3)):
        d = _desc(expert_dtype="fp8", **kw)
        E = d.n_experts
        G = E // d.n_depts if d.n_depts else E
        # n_act distinct experts spread over exactly n_dep departments (or any)
        ids = [(i % max(n_dep, 1)) * G + i // max(n_dep, 1) for i in range(n_act)]
        want = O.loaded_weight_bytes_fp8(np.array(ids), E, d.d_model, d.d_ff, router_bytes=2,
                                         n_depts=d.n_depts, d_ff_dept=d.d_ff_dept,
                                         d_ff_shared=d.d_ff_shared)
        assert M.moe_loaded_weight_bytes(d, n_act, n_dep) == want


def test_layer_kernel_count(lib):
    """Four launches where the down projection writes y (bf16 activations, T <= 4, rows
    of h within the LDS budget), five otherwise, eight in the factorised
    form; 0 at T = 0, -1 for an invalid descriptor or T."""
    q = _desc(max_tokens=16)
    assert [M.moe_layer_kernel_count(q, T) for T in (0, 1, 4, 5, 16)] == [0, 4, 4, 5, 5]
    assert M.moe_layer_kernel_count(q, 17) == -1
    assert M.moe_layer_kernel_count(_desc(d_model=7), 1) == -1
    # rows of h over the LDS budget: 4 tokens x 8 experts x 2048 bf16 = 128 KiB
    assert M.moe_layer_kernel_count(_desc(d_ff=2048, max_tokens=4), 4) == 5
    assert M.moe_layer_kernel_count(_desc(d_ff=2048, max_tokens=4), 1) == 4
    assert M.moe_layer_kernel_count(_desc(dtype="f32"), 1) == 5
    assert M.moe_layer_kernel_count(_desc(expert_dtype="fp8"), 1) == 4
    assert M.moe_layer_kernel_count(_desc(expert_dtype="fp8", max_tokens=8), 5) == 5
    fac = _desc(n_experts=32, top_k=6, d_ff=256, n_depts=4, d_ff_dept=256,
                dept_form="factorised")
    assert M.moe_layer_kernel_count(fac, 3) == 8
    # the selection per token ahead of a separate plan launch: past 16 tokens,
    # or past 256 experts
    big = _desc(max_tokens=64)
    assert [M.moe_layer_kernel_count(big, T) for T in (16, 17, 64)] == [5, 6, 6]
    wide = _desc(n_experts=512, max_tokens=4)
    assert [M.moe_layer_kernel_count(wide, T) for T in (1, 4)] == [5, 5]
    assert M.moe_layer_kernel_count(_desc(n_experts=256, max_tokens=4), 1) == 4
    fac_wide = _desc(n_experts=864, top_k=10, d_ff=2048, n_depts=8, d_ff_dept=2048,
                     dept_form="factorised", k_dept=5, max_tokens=16)
    assert M.moe_layer_kernel_count(fac_wide, 1) == 9


def test_layer_launch_workitems(lib):
    """Grids of the gate/up and down launches as a kernel trace reports them:
    whole 256-thread blocks; the down launch that writes y
    has one 512-thread block per 8 output columns; not reported for FP8 or
    the factorised form; -1 for a stage that is no grouped launch."""
    q = _desc(max_tokens=32)
    G, D = M.STAGE_GATEUP, M.STAGE_DOWN
    gu = [M.moe_layer_launch_workitems(q, T, G) for T in (1, 4, 16, 32)]
    assert all(g > 0 and g % 256 == 0 for g in gu)
    assert M.moe_layer_launch_workitems(q, 1, D) == 2048 // 8 * 512
    assert M.moe_layer_launch_workitems(q, 16, D) % 256 == 0
    assert M.moe_layer_launch_workitems(q, 16, D) != 2048 // 8 * 512
    # gate/up at T = 1: each active-expert slot (at most 8) streams 768 rows, a
    # row per wave of one 4-wave block
    assert gu[0] == 8 * (768 // 4) * 256
    assert M.moe_layer_launch_workitems(q, 0, G) == 0
    assert M.moe_layer_launch_workitems(_desc(expert_dtype="fp8"), 1, G) == 0
    fac = _desc(n_experts=32, top_k=6, d_ff=256, n_depts=4, d_ff_dept=256,
                dept_form="factorised")
    assert M.moe_layer_launch_workitems(fac, 1, G) == 0
    assert M.moe_layer_launch_workitems(q, 1, M.STAGE_ROUTE) == -1
    assert M.moe_layer_launch_workitems(q, 33, G) == -1


def test_step_stats_layout_matches_the_header(tmp_path):
    """The binding's StepStats has the C struct's size and field offsets
    (compiled from include/moe_decode.h with the host C compiler)."""
    import shutil
    import subprocess
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no host C compiler")
    fields = [f for f, _ in M.StepStats._fields_]
    src = tmp_path / "layout.c"
    src.write_text("#include <stdio.h>\n#include <stddef.h>\n#include \"moe_decode.h\"\n"
                   "int main(void) {\n  printf(\"%zu\\n\", sizeof(moe_step_stats));\n"
                   + "".join(f"  printf(\"%zu\\n\", offsetof(moe_step_stats, {f}));\n"
                             for f in fields)
                   + "  return 0;\n}\n")
    exe = tmp_path / "layout"
    subprocess.run([cc, "-std=c99", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)],
                   check=True)
    out = [int(v) for v in subprocess.run([str(exe)], capture_output=True, text=True,
                                          check=True).stdout.split()]
    assert out[0] == M.STEP_STATS_BYTES
    assert out[1:] == [getattr(M.StepStats, f).offset for f in fields]


def test_decode_rejects_a_misaligned_stats_pointer(lib):
    d = _desc()
    W = M.Weights(w_router=256, w_gate=256, w_up=256, w_down=256)
    ws = M.moe_workspace_bytes(d)
    assert lib.moe_layer_decode(ctypes.byref(d), ctypes.byref(W), 256, 1, 512, 4096, ws,
                                4100, None) == M.MOE_ERR_INVALID_ARG
    assert lib.moe_layer_decode_timed(ctypes.byref(d), ctypes.byref(W), 256, 1, 512, 4096, ws,
                                      4100, None, None) == M.MOE_ERR_INVALID_ARG


def test_noalloc_refuses_steps_beyond_its_scratch(lib):
    """The allocation-free entry point lays its scratch out for exactly T
    tokens and refuses, on the host before any HIP call, a step that does
    not fit MOE_NOALLOC_SCRATCH_BYTES (DeepSeek-V3 geometry at 128 tokens
    needs about 42 MiB); invalid descriptors and T are refused first."""
    big = _desc(d_model=7168, n_experts=256, d_ff=2048, d_ff_shared=2048, score="sigmoid",
                max_tokens=128)
    assert M.moe_workspace_bytes(big) > M.NOALLOC_SCRATCH_BYTES
    fits = _desc(d_model=7168, n_experts=256, d_ff=2048, d_ff_shared=2048, score="sigmoid",
                 max_tokens=32)
    assert M.moe_workspace_bytes(fits) <= M.NOALLOC_SCRATCH_BYTES
    W = M.Weights(w_router=256, w_gate=256, w_up=256, w_down=256, ws_gate=256, ws_up=256,
                  ws_down=256)
    assert lib.moe_layer_decode_noalloc(ctypes.byref(big), ctypes.byref(W), 256, 128, 512, None,
                                        None) == M.MOE_ERR_UNSUPPORTED
    assert lib.moe_layer_decode_noalloc(ctypes.byref(big), ctypes.byref(W), 256, 129, 512, None,
                                        None) == M.MOE_ERR_INVALID_ARG
    assert lib.moe_layer_decode_noalloc(ctypes.byref(_desc(d_model=7)), ctypes.byref(W), 256, 1,
                                        512, None, None) == M.MOE_ERR_INVALID_ARG
    assert lib.moe_layer_decode_noalloc(ctypes.byref(big), ctypes.byref(W), 256, 0, 512, None,
                                        None) == M.MOE_OK
