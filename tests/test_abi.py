"""The C ABI without a GPU: the library loads, exports every entry point that
include/moe.h declares, and its host-side checks follow the documented error
conventions (they run before any HIP call)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")


def declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def M():
    from mixture_experts_layer_sparse_amd import moe
    if not os.path.exists(moe.LIB_PATH):
        pytest.skip("libmoe.so not built")
    moe.lib()
    return moe


def test_every_declared_symbol_is_exported(M):
    names = declared()
    assert {"moe_route", "moe_dispatch", "moe_experts", "moe_combine"} <= set(names)
    h = ctypes.CDLL(M.LIB_PATH)
    for n in names:
        assert hasattr(h, n), n


def test_binding_covers_every_symbol(M):
    assert set(declared()) == set(M._SIGS)


def test_struct_layout_matches_c(M, tmp_path):
    """The ctypes mirror has the C compiler's layout of moe_shape."""
    import subprocess
    src = tmp_path / "layout.c"
    src.write_text('#include <stdio.h>\n#include <stddef.h>\n#include "moe.h"\n'
                   'int main(void){printf("%zu %zu %zu %zu %zu %zu\\n", sizeof(moe_shape),'
                   ' offsetof(moe_shape, d), offsetof(moe_shape, drop), offsetof(moe_shape, alpha),'
                   ' offsetof(moe_shape, gate), offsetof(moe_shape, wfmt));'
                   'return 0;}\n')
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)], check=True)
    size, off_d, off_drop, off_alpha, off_gate, off_wfmt = map(
        int, subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split())
    assert ctypes.sizeof(M.Shape) == size == 72
    assert (M.Shape.d.offset, M.Shape.drop.offset, M.Shape.alpha.offset, M.Shape.gate.offset,
            M.Shape.wfmt.offset) == (off_d, off_drop, off_alpha, off_gate, off_wfmt)


def _s(M, **kw):
    base = dict(T=64, d=64, N=8, k=2, F=128, act="silu", dtype="f32")
    base.update(kw)
    return M.make_shape(**base)


def test_shape_checks(M):
    ok = _s(M)
    assert M.check_shape(ok) == M.MOE_OK
    assert M.workspace_bytes(ok) > 0
    bad = [dict(k=9, N=8), dict(k=0), dict(N=0), dict(N=300), dict(d=60), dict(T=-1),
           dict(n_groups=3), dict(n_groups=4, topk_groups=0), dict(n_groups=4, topk_groups=5),
           dict(n_groups=8, topk_groups=1, k=2), dict(n_groups=4, topk_groups=2, group_score_k=3)]
    for kw in bad:
        st = M.check_shape(_s(M, **kw))
        assert st in (M.MOE_ERR_ARG, M.MOE_ERR_UNSUPPORTED), kw
        assert M.workspace_bytes(_s(M, **kw)) == 0
    assert M.check_shape(_s(M, dtype="f32", buf="fp8")) == M.MOE_ERR_UNSUPPORTED
    assert M.check_shape(_s(M, dtype="bf16", d=72)) == M.MOE_ERR_UNSUPPORTED
    assert M.check_shape(_s(M, N=16, k=9)) == M.MOE_ERR_UNSUPPORTED
    # one bf16 expert matrix beyond the 32-bit byte range of a buffer resource
    assert M.check_shape(_s(M, dtype="bf16", d=32768, F=65536)) == M.MOE_ERR_UNSUPPORTED
    assert M.check_shape(_s(M, dtype="bf16", d=16384, F=65536)) == M.MOE_OK
    # the fallback drop mode needs the shared expert; the gate is one of two values
    assert M.check_shape(_s(M, drop="fallback")) == M.MOE_ERR_ARG
    assert M.check_shape(_s(M, drop="fallback", shared=True)) == M.MOE_OK
    assert M.check_shape(_s(M, gate="full")) == M.MOE_OK
    assert M.check_shape(_s(M).replace(gate=2)) == M.MOE_ERR_ARG
    assert M.check_shape(_s(M).replace(drop=3)) == M.MOE_ERR_ARG
    # MXFP4 expert weights need bf16 layers
    assert M.check_shape(_s(M, dtype="bf16", wfmt="mxfp4")) == M.MOE_OK
    assert M.check_shape(_s(M, wfmt="mxfp4")) == M.MOE_ERR_UNSUPPORTED
    assert M.check_shape(_s(M).replace(wfmt=2)) == M.MOE_ERR_ARG


def test_null_pointers_and_workspace_rejected_on_host(M):
    s = _s(M)
    L = M.lib()
    p = ctypes.c_void_p(16)  # never dereferenced: the checks run first
    # missing x
    st = L.moe_route(ctypes.byref(s), None, p, None, p, p, p, p, None, None, None, None, p,
                     M.workspace_bytes(s), None)
    assert st == M.MOE_ERR_ARG
    # workspace too small
    st = L.moe_route(ctypes.byref(s), p, p, None, p, p, p, p, None, None, None, None, p, 8, None)
    assert st == M.MOE_ERR_WORKSPACE
    st = L.moe_experts(ctypes.byref(s), p, None, p, p, None, p, None, None, None, None, p, None,
                       p, 16, None)
    assert st == M.MOE_ERR_WORKSPACE
    # route + dispatch in one call: missing x_perm, then too small a workspace
    st = L.moe_route_dispatch(ctypes.byref(s), p, p, None, p, p, p, p, None, None, None, p, p, p,
                              p, None, None, p, M.workspace_bytes(s), None)
    assert st == M.MOE_ERR_ARG
    st = L.moe_route_dispatch(ctypes.byref(s), p, p, None, p, p, p, p, None, None, None, p, p, p,
                              p, p, None, p, 8, None)
    assert st == M.MOE_ERR_WORKSPACE
    # SwiGLU without W3
    s2 = _s(M, act="swiglu")
    st = L.moe_expert_up(ctypes.byref(s2), p, None, p, p, None, p, None, 0, None)
    assert st == M.MOE_ERR_ARG
    # the shared expert's split entry points: no shared expert, a missing buffer, SwiGLU without Ws3
    st = L.moe_expert_down_shared(ctypes.byref(s), p, p, p, p, p, p, p, None, 0, None)
    assert st == M.MOE_ERR_ARG
    ssh = _s(M, shared=True)
    st = L.moe_expert_down_shared(ctypes.byref(ssh), p, p, p, p, None, p, p, None, 0, None)
    assert st == M.MOE_ERR_ARG
    st = L.moe_shared_expert_up(ctypes.byref(s2), p, p, None, p, None, 0, None)
    assert st == M.MOE_ERR_ARG
    # routed + shared up in one call: no shared expert, then a missing h_shared
    st = L.moe_expert_up_gather_shared(ctypes.byref(s), p, None, p, p, p, None, p, p, p, None, p, None, 0,
                                       None)
    assert st == M.MOE_ERR_ARG
    st = L.moe_expert_up_gather_shared(ctypes.byref(ssh), p, None, p, p, p, None, p, p, p, None, None, None,
                                       0, None)
    assert st == M.MOE_ERR_ARG
    # the combining down GEMM: missing src, missing y, shared expert without its buffers, small workspace
    st = L.moe_expert_down_combine(ctypes.byref(s), p, p, None, p, p, None, None, None, p, p, p, p, p,
                                   M.workspace_bytes(s), None)
    assert st == M.MOE_ERR_ARG
    st = L.moe_expert_down_combine(ctypes.byref(s), p, p, p, p, p, None, None, None, p, p, p, None, p,
                                   M.workspace_bytes(s), None)
    assert st == M.MOE_ERR_ARG
    st = L.moe_expert_down_combine(ctypes.byref(ssh), p, p, p, p, p, None, p, p, p, p, p, p, p,
                                   M.workspace_bytes(ssh), None)
    assert st == M.MOE_ERR_ARG
    st = L.moe_expert_down_combine(ctypes.byref(s), p, p, p, p, p, None, None, None, p, p, p, p, p, 8, None)
    assert st == M.MOE_ERR_WORKSPACE
    # the scatter layer: missing y, then too small a workspace
    st = L.moe_forward_scatter(ctypes.byref(s), p, p, None, p, p, p, None, None, None, p, p, p, p, None,
                               None, None, p, p, p, p, None, p, None, None, p, M.workspace_bytes(s), None)
    assert st == M.MOE_ERR_ARG
    st = L.moe_forward_scatter(ctypes.byref(s), p, p, None, p, p, p, None, None, None, p, p, p, p, None,
                               None, None, p, p, p, p, None, p, None, p, p, 8, None)
    assert st == M.MOE_ERR_WORKSPACE
    # T == 0 is a no-op even with null buffers
    s0 = _s(M, T=0)
    st = L.moe_route(ctypes.byref(s0), None, None, None, None, None, None, None, None, None, None,
                     None, None, 0, None)
    assert st == M.MOE_OK
    assert M.status_string(M.MOE_ERR_WORKSPACE) == "workspace too small"


def test_workspace_grows_with_h(M):
    for dt, es in (("f32", 4), ("bf16", 2)):
        a = M.workspace_bytes(_s(M, T=64, dtype=dt))
        b = M.workspace_bytes(_s(M, T=128, dtype=dt))
        assert b > a
        s = _s(M, T=128, dtype=dt)
        assert b >= s.T * s.k * s.F * es          # the expert intermediate h lives there


def test_bench_roofline_kernel_is_in_the_counter_summary():
    """bench.py fills roofline.traffic from the committed counter summary by the
    gate/up kernel's name: that name (all template arguments, as the trace
    prints them) must be one of the summary's kernels, so that the field is not
    silently null."""
    import json
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    sys.path.insert(0, root)
    import bench
    with open(bench.COUNTER_FILE) as f:
        text = f.read()
    data = json.loads(text.split("```json", 1)[1].split("```", 1)[0])
    assert bench.UP_KERNEL["mixtral"] in data["kernels"]
