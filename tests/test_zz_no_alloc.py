"""moe_route_dispatch_noalloc (scratch in the library's static device array, no
workspace argument) against moe_route_dispatch (a caller's workspace): the
same kernels on the same inputs, so every output must be bit for bit the same.
Three calls in a row on one device, each with a smaller input than the one
before, so that each call finds the previous call's contents in the shared
scratch: a wide router (logits through the split-K GEMM, 8-token tiles, fp8
buffer, groups, capacity), split logits below 512 tokens, and a single router
tile (statistics in the router kernel)."""
import ctypes

import numpy as np
import pytest
import torch

import synthetic_inputs as si
from mixture_experts_layer_sparse_amd import moe as M

pytestmark = pytest.mark.gpu

SEQUENCE = [
    si.Workload("na_wide", T=1003, d=8192, N=64, k=8, F=64, act="swiglu", dtype="bf16", buf="fp8",
                n_groups=8, topk_groups=4, capacity=120),
    si.small("mixtral", T=300, capacity=70),
    si.Workload("na_tile", T=5, d=512, N=32, k=3, F=64, act="relu", dtype="bf16", buf="bf16",
                bias="zipf2"),
]


def test_noalloc_matches_workspace_call():
    from moe_gpu_util import upload
    for wl in SEQUENCE:
        s = M.shape_of(wl)
        need = M.workspace_bytes(s)
        print(f"case {wl.name}: T={wl.T} d={wl.d} N={wl.N} k={wl.k} workspace {need >> 20} MiB", flush=True)
        g = upload(wl, si.generate(wl, experts=False))
        ref = M.route_dispatch(s, g["x"], g["wg"], g.get("bias"))
        got = M.route_dispatch(s, g["x"], g["wg"], g.get("bias"), noalloc=True)
        torch.cuda.synchronize()
        R = int(ref["offsets"][-1].item())
        for key, want in ref.items():
            if want is None:
                continue
            have = got[key]
            if key in ("src", "x_perm", "row_scale"):
                want, have = want[:R], have[:R]
            assert torch.equal(have, want), (wl.name, key)
        if wl.capacity:
            assert int(ref["drop"].sum().item()) > 0


def test_noalloc_rejects_too_large_before_launching():
    s = M.make_shape(T=1 << 20, d=64, N=256, k=8, F=64, act="relu", dtype="bf16")
    p = ctypes.c_void_p(16)            # never dereferenced: the size check comes first
    L = M.lib()
    st = L.moe_route_dispatch_noalloc(ctypes.byref(s), p, p, None, p, p, p, p, None, None, None, p,
                                      p, p, p, p, None, None)
    assert st == M.MOE_ERR_TOO_LARGE
    assert "static" in M.status_string(st)
