"""Python binding of the C ABI in include/moe.h (ctypes over libmoe.so).

Argument marshalling only: tensors are checked (device, dtype, shape,
contiguity) and their device pointers are passed with the current HIP stream.
Every step of the layer runs in the library's HIP kernels; there is no other
code path.  The library must be built (``python -m
mixture_experts_layer_sparse_amd.build``); importing works without it, but the
first call raises if it is missing.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_float, c_int32, c_int64, c_size_t, c_void_p

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoe.so")

MOE_OK, MOE_ERR_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP, MOE_ERR_TOO_LARGE = range(6)
STATIC_SCRATCH_BYTES = 48 << 20      # MOE_STATIC_SCRATCH_BYTES
MOE_F32, MOE_BF16, MOE_FP8_E4M3 = range(3)
MOE_ACT_SILU, MOE_ACT_RELU, MOE_ACT_SWIGLU = range(3)
MOE_DROP_PASSTHROUGH, MOE_DROP_ZERO, MOE_DROP_FALLBACK = range(3)
MOE_GATE_SPARSE, MOE_GATE_FULL = range(2)
MOE_W_DEFAULT, MOE_W_MXFP4 = range(2)

_DT = {"f32": MOE_F32, "bf16": MOE_BF16, "fp8": MOE_FP8_E4M3}
_ACT = {"silu": MOE_ACT_SILU, "relu": MOE_ACT_RELU, "swiglu": MOE_ACT_SWIGLU}
_DROP = {"passthrough": MOE_DROP_PASSTHROUGH, "zero": MOE_DROP_ZERO, "fallback": MOE_DROP_FALLBACK}
_GATE = {"sparse": MOE_GATE_SPARSE, "full": MOE_GATE_FULL}
_WFMT = {"bf16": MOE_W_DEFAULT, "f32": MOE_W_DEFAULT, "default": MOE_W_DEFAULT, "mxfp4": MOE_W_MXFP4}


class MoeError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn}: {status_string(status)} (status {status})")


class Shape(ctypes.Structure):
    """Mirror of ``moe_shape``."""
    _fields_ = [("T", c_int64), ("d", c_int32), ("N", c_int32), ("k", c_int32), ("F", c_int32),
                ("capacity", c_int32), ("n_groups", c_int32), ("topk_groups", c_int32),
                ("group_score_k", c_int32), ("has_shared", c_int32), ("dtype", c_int32),
                ("buf_dtype", c_int32), ("act", c_int32), ("drop", c_int32), ("alpha", c_float),
                ("gate", c_int32), ("wfmt", c_int32)]

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.bfloat16 if self.dtype == MOE_BF16 else torch.float32

    @property
    def buf_torch_dtype(self) -> torch.dtype:
        if self.buf_dtype == MOE_FP8_E4M3:
            return torch.uint8
        return self.torch_dtype

    def replace(self, **kw) -> "Shape":
        s = Shape()
        ctypes.pointer(s)[0] = self
        for key, val in kw.items():
            setattr(s, key, val)
        return s


def make_shape(T, d, N, k, F, act="swiglu", dtype="bf16", buf=None, capacity=0,
               drop="passthrough", n_groups=0, topk_groups=0, group_score_k=2, shared=False,
               alpha=0.01, gate="sparse", wfmt="default") -> Shape:
    return Shape(T=T, d=d, N=N, k=k, F=F, capacity=capacity, n_groups=n_groups,
                 topk_groups=topk_groups, group_score_k=group_score_k,
                 has_shared=1 if shared else 0, dtype=_DT[dtype], buf_dtype=_DT[buf or dtype],
                 act=_ACT[act], drop=_DROP[drop], alpha=alpha, gate=_GATE[gate], wfmt=_WFMT[wfmt])


def mxfp4_bytes(rows: int, K: int) -> int:
    """Bytes of one MXFP4 matrix [rows][K] as the library takes it: codes, then scales."""
    return rows * K // 2 + rows * K // 32


def shape_of(wl) -> Shape:
    """Shape from any object with the workload attributes (T, d, N, k, F, act,
    dtype, buf, capacity, drop, n_groups, topk_groups, group_score_k, shared, alpha, and
    optionally gate)."""
    return make_shape(wl.T, wl.d, wl.N, wl.k, wl.F, act=wl.act, dtype=wl.dtype, buf=wl.buf,
                      capacity=wl.capacity, drop=wl.drop, n_groups=wl.n_groups,
                      topk_groups=wl.topk_groups, group_score_k=wl.group_score_k,
                      gate=getattr(wl, "gate", "sparse"), wfmt=getattr(wl, "wfmt", "default"),
                      shared=wl.shared, alpha=wl.alpha)


_lib = None
_P = c_void_p
_SIGS = {
    "moe_workspace_bytes": (c_size_t, [POINTER(Shape)]),
    "moe_check_shape": (c_int32, [POINTER(Shape)]),
    "moe_route": (c_int32, [POINTER(Shape)] + [_P] * 11 + [_P, c_size_t, _P]),
    "moe_dispatch": (c_int32, [POINTER(Shape)] + [_P] * 8 + [_P, c_size_t, _P]),
    "moe_route_dispatch": (c_int32, [POINTER(Shape)] + [_P] * 16 + [_P, c_size_t, _P]),
    "moe_route_dispatch_noalloc": (c_int32, [POINTER(Shape)] + [_P] * 16 + [_P]),
    "moe_route_plan": (c_int32, [POINTER(Shape)] + [_P] * 16 + [_P, c_size_t, _P]),
    "moe_expert_up": (c_int32, [POINTER(Shape)] + [_P] * 6 + [_P, c_size_t, _P]),
    "moe_expert_up_gather": (c_int32, [POINTER(Shape)] + [_P] * 7 + [_P, c_size_t, _P]),
    "moe_expert_down": (c_int32, [POINTER(Shape)] + [_P] * 4 + [_P, c_size_t, _P]),
    "moe_shared_expert": (c_int32, [POINTER(Shape)] + [_P] * 6 + [_P, c_size_t, _P]),
    "moe_shared_expert_up": (c_int32, [POINTER(Shape)] + [_P] * 4 + [_P, c_size_t, _P]),
    "moe_expert_down_shared": (c_int32, [POINTER(Shape)] + [_P] * 7 + [_P, c_size_t, _P]),
    "moe_expert_up_gather_shared": (c_int32, [POINTER(Shape)] + [_P] * 11 + [_P, c_size_t, _P]),
    "moe_experts": (c_int32, [POINTER(Shape)] + [_P] * 12 + [_P, c_size_t, _P]),
    "moe_combine": (c_int32, [POINTER(Shape)] + [_P] * 6 + [_P]),
    "moe_forward": (c_int32, [POINTER(Shape)] + [_P] * 25 + [_P, c_size_t, _P]),
    "moe_expert_down_combine": (c_int32, [POINTER(Shape)] + [_P] * 12 + [_P, c_size_t, _P]),
    "moe_forward_scatter": (c_int32, [POINTER(Shape)] + [_P] * 24 + [_P, c_size_t, _P]),
    "moe_status_string": (ctypes.c_char_p, [c_int32]),
}


def lib():
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m mixture_experts_layer_sparse_amd.build`")
        h = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(h, name)
            fn.restype = res
            fn.argtypes = args
        _lib = h
    return _lib


def status_string(st: int) -> str:
    return lib().moe_status_string(st).decode()


def _call(name: str, *args) -> None:
    st = getattr(lib(), name)(*args)
    if st != MOE_OK:
        raise MoeError(name, st)


def _ptr(t: torch.Tensor | None) -> int | None:
    return None if t is None else t.data_ptr()


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _check(t: torch.Tensor | None, name: str, shape: tuple, dtype: torch.dtype,
           required: bool = True) -> None:
    if t is None:
        if required:
            raise ValueError(f"{name} is required")
        return
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _check_w(t, name: str, s: Shape, n: int | None, rows: int, K: int, required: bool = True) -> None:
    """An expert weight tensor: [n][rows][K] (or [rows][K] when n is None) in the
    layer's type, or for MXFP4 weights [n][codes + scales] bytes."""
    if s.wfmt == MOE_W_MXFP4:
        shape = (mxfp4_bytes(rows, K),) if n is None else (n, mxfp4_bytes(rows, K))
        _check(t, name, shape, torch.uint8, required)
    else:
        shape = (rows, K) if n is None else (n, rows, K)
        _check(t, name, shape, s.torch_dtype, required)


def workspace_bytes(s: Shape) -> int:
    return int(lib().moe_workspace_bytes(ctypes.byref(s)))


def check_shape(s: Shape) -> int:
    return int(lib().moe_check_shape(ctypes.byref(s)))


def alloc_workspace(s: Shape, device="cuda") -> torch.Tensor:
    n = workspace_bytes(s)
    if n == 0:
        raise MoeError("moe_workspace_bytes", check_shape(s) or MOE_ERR_ARG)
    return torch.empty(n, dtype=torch.uint8, device=device)


# ------------------------------------------------------------------ calls --

def route(s: Shape, x, wg, bias=None, ws=None, logits=False, out=None) -> dict:
    T, N, k = s.T, s.N, s.k
    dev = x.device
    _check(x, "x", (T, s.d), s.torch_dtype)
    _check(wg, "wg", (N, s.d), s.torch_dtype)
    _check(bias, "bias", (N,), torch.float32, required=False)
    o = out if out is not None else {
        "idx": torch.empty((T, k), dtype=torch.int32, device=dev),
        "w": torch.empty((T, k), dtype=torch.float32, device=dev),
        "counts": torch.empty(N, dtype=torch.int32, device=dev),
        "kept_counts": torch.empty(N, dtype=torch.int32, device=dev),
        "p": torch.empty(N, dtype=torch.float32, device=dev),
        "f": torch.empty(N, dtype=torch.float32, device=dev),
        "l_aux": torch.empty(1, dtype=torch.float32, device=dev),
    }
    if logits and "logits" not in o:
        o["logits"] = torch.empty((T, N), dtype=torch.float32, device=dev)
    ws = ws if ws is not None else alloc_workspace(s, dev)
    _call("moe_route", ctypes.byref(s), _ptr(x), _ptr(wg), _ptr(bias), _ptr(o["idx"]),
          _ptr(o["w"]), _ptr(o["counts"]), _ptr(o["kept_counts"]), _ptr(o.get("p")),
          _ptr(o.get("f")), _ptr(o.get("l_aux")), _ptr(o.get("logits")), _ptr(ws), ws.numel(),
          _stream())
    return o


def dispatch(s: Shape, x, idx, ws=None, out=None) -> dict:
    T, N, k, d = s.T, s.N, s.k, s.d
    dev = x.device
    _check(x, "x", (T, d), s.torch_dtype)
    _check(idx, "idx", (T, k), torch.int32)
    fp8 = s.buf_dtype == MOE_FP8_E4M3
    o = out if out is not None else {
        "offsets": torch.empty(N + 1, dtype=torch.int32, device=dev),
        "pos": torch.empty((T, k), dtype=torch.int32, device=dev),
        "src": torch.empty(T * k, dtype=torch.int32, device=dev),
        "drop": torch.empty((T, k), dtype=torch.uint8, device=dev),
        "x_perm": torch.empty((T * k, d), dtype=s.buf_torch_dtype, device=dev),
        "row_scale": torch.empty(T * k, dtype=torch.float32, device=dev) if fp8 else None,
    }
    ws = ws if ws is not None else alloc_workspace(s, dev)
    _call("moe_dispatch", ctypes.byref(s), _ptr(x), _ptr(idx), _ptr(o["offsets"]), _ptr(o["pos"]),
          _ptr(o["src"]), _ptr(o["drop"]), _ptr(o["x_perm"]), _ptr(o.get("row_scale")), _ptr(ws),
          ws.numel(), _stream())
    return o


def route_dispatch(s: Shape, x, wg, bias=None, ws=None, noalloc=False, out=None) -> dict:
    """moe_route_dispatch: the outputs of route() and dispatch() (no logits)
    from one call, with the dispatch plan folded into the row copy.  With
    ``noalloc`` the call is moe_route_dispatch_noalloc (the library's static
    scratch, no workspace; ``ws`` is ignored).  ``out``: output tensors to
    fill (as returned by an earlier call), else allocated here."""
    T, N, k, d = s.T, s.N, s.k, s.d
    dev = x.device
    _check(x, "x", (T, d), s.torch_dtype)
    _check(wg, "wg", (N, d), s.torch_dtype)
    _check(bias, "bias", (N,), torch.float32, required=False)
    fp8 = s.buf_dtype == MOE_FP8_E4M3
    o = out if out is not None else {
        "idx": torch.empty((T, k), dtype=torch.int32, device=dev),
        "w": torch.empty((T, k), dtype=torch.float32, device=dev),
        "counts": torch.empty(N, dtype=torch.int32, device=dev),
        "kept_counts": torch.empty(N, dtype=torch.int32, device=dev),
        "p": torch.empty(N, dtype=torch.float32, device=dev),
        "f": torch.empty(N, dtype=torch.float32, device=dev),
        "l_aux": torch.empty(1, dtype=torch.float32, device=dev),
        "offsets": torch.empty(N + 1, dtype=torch.int32, device=dev),
        "pos": torch.empty((T, k), dtype=torch.int32, device=dev),
        "src": torch.empty(T * k, dtype=torch.int32, device=dev),
        "drop": torch.empty((T, k), dtype=torch.uint8, device=dev),
        "x_perm": torch.empty((T * k, d), dtype=s.buf_torch_dtype, device=dev),
        "row_scale": torch.empty(T * k, dtype=torch.float32, device=dev) if fp8 else None,
    }
    args = [ctypes.byref(s), _ptr(x), _ptr(wg), _ptr(bias), _ptr(o["idx"]), _ptr(o["w"]),
            _ptr(o["counts"]), _ptr(o["kept_counts"]), _ptr(o["p"]), _ptr(o["f"]), _ptr(o["l_aux"]),
            _ptr(o["offsets"]), _ptr(o["pos"]), _ptr(o["src"]), _ptr(o["drop"]), _ptr(o["x_perm"]),
            _ptr(o.get("row_scale"))]
    if noalloc:
        _call("moe_route_dispatch_noalloc", *args, _stream())
        return o
    ws = ws if ws is not None else alloc_workspace(s, dev)
    _call("moe_route_dispatch", *args, _ptr(ws), ws.numel(), _stream())
    return o


def route_plan(s: Shape, x, wg, bias=None, ws=None, out=None) -> dict:
    """moe_route_plan: route and plan without the expert-ordered copy (the
    fused layer's first phase); for an fp8 buffer also the token-order codes
    (``x_codes`` [T][d]) and the per-position row scales."""
    T, N, k, d = s.T, s.N, s.k, s.d
    dev = x.device
    _check(x, "x", (T, d), s.torch_dtype)
    _check(wg, "wg", (N, d), s.torch_dtype)
    _check(bias, "bias", (N,), torch.float32, required=False)
    fp8 = s.buf_dtype == MOE_FP8_E4M3
    i32 = dict(dtype=torch.int32, device=dev)
    f32 = dict(dtype=torch.float32, device=dev)
    o = out if out is not None else {
        "idx": torch.empty((T, k), **i32), "w": torch.empty((T, k), **f32),
        "counts": torch.empty(N, **i32), "kept_counts": torch.empty(N, **i32),
        "p": torch.empty(N, **f32), "f": torch.empty(N, **f32), "l_aux": torch.empty(1, **f32),
        "offsets": torch.empty(N + 1, **i32), "pos": torch.empty((T, k), **i32),
        "src": torch.empty(T * k, **i32), "drop": torch.empty((T, k), dtype=torch.uint8, device=dev),
        "x_codes": torch.empty((T, d), dtype=torch.uint8, device=dev) if fp8 else None,
        "row_scale": torch.empty(T * k, **f32) if fp8 else None,
    }
    ws = ws if ws is not None else alloc_workspace(s, dev)
    _call("moe_route_plan", ctypes.byref(s), _ptr(x), _ptr(wg), _ptr(bias), _ptr(o["idx"]),
          _ptr(o["w"]), _ptr(o["counts"]), _ptr(o["kept_counts"]), _ptr(o["p"]), _ptr(o["f"]),
          _ptr(o["l_aux"]), _ptr(o["offsets"]), _ptr(o["pos"]), _ptr(o["src"]), _ptr(o["drop"]),
          _ptr(o.get("x_codes")), _ptr(o.get("row_scale")), _ptr(ws), ws.numel(), _stream())
    return o


def expert_up_gather(s: Shape, a, row_scale, offsets, src, w1, w3, h=None, ws=None):
    """moe_expert_up_gather: the up GEMM reading row src[r] of ``a`` ([T][d]:
    x, or the token-order fp8 codes from route_plan) for dispatch row r."""
    R, F = s.T * s.k, s.F
    fp8 = s.buf_dtype == MOE_FP8_E4M3
    _check(a, "a", (s.T, s.d), torch.uint8 if fp8 else s.torch_dtype)
    _check(offsets, "offsets", (s.N + 1,), torch.int32)
    _check(src, "src", (R,), torch.int32)
    _check_w(w1, "w1", s, s.N, F, s.d)
    _check_w(w3, "w3", s, s.N, F, s.d, required=s.act == MOE_ACT_SWIGLU)
    if h is None:
        h = torch.empty((R, F), dtype=s.torch_dtype, device=a.device)
    _call("moe_expert_up_gather", ctypes.byref(s), _ptr(a), _ptr(row_scale), _ptr(offsets), _ptr(src),
          _ptr(w1), _ptr(w3), _ptr(h), _ptr(ws), 0 if ws is None else ws.numel(), _stream())
    return h


def expert_up_gather_shared(s: Shape, a, row_scale, offsets, src, w1, w3, x, ws1, ws3, h=None,
                            h_shared=None, ws=None):
    """moe_expert_up_gather_shared: expert_up_gather and shared_expert_up in one
    call (one launch for a call of at most four tokens).  Returns (h, h_shared)."""
    R, T, F = s.T * s.k, s.T, s.F
    fp8 = s.buf_dtype == MOE_FP8_E4M3
    _check(a, "a", (T, s.d), torch.uint8 if fp8 else s.torch_dtype)
    _check(offsets, "offsets", (s.N + 1,), torch.int32)
    _check(src, "src", (R,), torch.int32)
    _check(x, "x", (T, s.d), s.torch_dtype)
    _check_w(w1, "w1", s, s.N, F, s.d)
    _check_w(w3, "w3", s, s.N, F, s.d, required=s.act == MOE_ACT_SWIGLU)
    _check_w(ws1, "ws1", s, None, F, s.d)
    _check_w(ws3, "ws3", s, None, F, s.d, required=s.act == MOE_ACT_SWIGLU)
    if h is None:
        h = torch.empty((R, F), dtype=s.torch_dtype, device=a.device)
    if h_shared is None:
        h_shared = torch.empty((T, F), dtype=s.torch_dtype, device=a.device)
    _call("moe_expert_up_gather_shared", ctypes.byref(s), _ptr(a), _ptr(row_scale), _ptr(offsets),
          _ptr(src), _ptr(w1), _ptr(w3), _ptr(h), _ptr(x), _ptr(ws1), _ptr(ws3), _ptr(h_shared), _ptr(ws),
          0 if ws is None else ws.numel(), _stream())
    return h, h_shared


def expert_up(s: Shape, x_perm, row_scale, offsets, w1, w3, h=None, ws=None):
    """ws: None (a mostly idle last tile round runs as quarter tiles) or a
    workspace from alloc_workspace (that round is split along K instead)."""
    R, F = s.T * s.k, s.F
    _check(x_perm, "x_perm", (R, s.d), s.buf_torch_dtype)
    _check(offsets, "offsets", (s.N + 1,), torch.int32)
    _check_w(w1, "w1", s, s.N, F, s.d)
    _check_w(w3, "w3", s, s.N, F, s.d, required=s.act == MOE_ACT_SWIGLU)
    if h is None:
        h = torch.empty((R, F), dtype=s.torch_dtype, device=x_perm.device)
    _call("moe_expert_up", ctypes.byref(s), _ptr(x_perm), _ptr(row_scale), _ptr(offsets), _ptr(w1),
          _ptr(w3), _ptr(h), _ptr(ws), 0 if ws is None else ws.numel(), _stream())
    return h


def expert_down(s: Shape, h, offsets, w2, out=None, ws=None):
    """ws as for expert_up."""
    R = s.T * s.k
    _check(h, "h", (R, s.F), s.torch_dtype)
    _check_w(w2, "w2", s, s.N, s.d, s.F)
    if out is None:
        out = torch.empty((R, s.d), dtype=s.torch_dtype, device=h.device)
    _call("moe_expert_down", ctypes.byref(s), _ptr(h), _ptr(offsets), _ptr(w2), _ptr(out), _ptr(ws),
          0 if ws is None else ws.numel(), _stream())
    return out


def shared_expert(s: Shape, x, ws1, ws3, ws2, h_shared=None, out_shared=None, ws=None):
    T, d, F = s.T, s.d, s.F
    _check_w(ws1, "ws1", s, None, F, d)
    _check_w(ws3, "ws3", s, None, F, d, required=s.act == MOE_ACT_SWIGLU)
    _check_w(ws2, "ws2", s, None, d, F)
    if h_shared is None:
        h_shared = torch.empty((T, F), dtype=s.torch_dtype, device=x.device)
    if out_shared is None:
        out_shared = torch.empty((T, d), dtype=s.torch_dtype, device=x.device)
    _call("moe_shared_expert", ctypes.byref(s), _ptr(x), _ptr(ws1), _ptr(ws3), _ptr(ws2),
          _ptr(h_shared), _ptr(out_shared), _ptr(ws), 0 if ws is None else ws.numel(), _stream())
    return out_shared


def shared_expert_up(s: Shape, x, ws1, ws3, h_shared=None, ws=None):
    """moe_shared_expert_up: h_shared = act(Ws1 x, Ws3 x)."""
    T, d, F = s.T, s.d, s.F
    _check(x, "x", (T, d), s.torch_dtype)
    _check_w(ws1, "ws1", s, None, F, d)
    _check_w(ws3, "ws3", s, None, F, d, required=s.act == MOE_ACT_SWIGLU)
    if h_shared is None:
        h_shared = torch.empty((T, F), dtype=s.torch_dtype, device=x.device)
    _call("moe_shared_expert_up", ctypes.byref(s), _ptr(x), _ptr(ws1), _ptr(ws3), _ptr(h_shared),
          _ptr(ws), 0 if ws is None else ws.numel(), _stream())
    return h_shared


def expert_down_shared(s: Shape, h, offsets, w2, h_shared, ws2, out=None, out_shared=None, ws=None):
    """moe_expert_down_shared: the routed down GEMM and the shared expert's in
    one launch.  Returns (out, out_shared)."""
    T, d, F = s.T, s.d, s.F
    _check(h, "h", (T * s.k, F), s.torch_dtype)
    _check_w(w2, "w2", s, s.N, d, F)
    _check_w(ws2, "ws2", s, None, d, F)
    _check(h_shared, "h_shared", (T, F), s.torch_dtype)
    if out is None:
        out = torch.empty((T * s.k, d), dtype=s.torch_dtype, device=h.device)
    if out_shared is None:
        out_shared = torch.empty((T, d), dtype=s.torch_dtype, device=h.device)
    _call("moe_expert_down_shared", ctypes.byref(s), _ptr(h), _ptr(offsets), _ptr(w2), _ptr(out),
          _ptr(h_shared), _ptr(ws2), _ptr(out_shared), _ptr(ws), 0 if ws is None else ws.numel(),
          _stream())
    return out, out_shared


def experts(s: Shape, x_perm, row_scale, offsets, w1, w3, w2, x=None, ws1=None, ws3=None,
            ws2=None, ws=None, out=None, out_shared=None):
    R, d = s.T * s.k, s.d
    dev = x_perm.device
    if out is None:
        out = torch.empty((R, d), dtype=s.torch_dtype, device=dev)
    if s.has_shared and out_shared is None:
        out_shared = torch.empty((s.T, d), dtype=s.torch_dtype, device=dev)
    ws = ws if ws is not None else alloc_workspace(s, dev)
    _call("moe_experts", ctypes.byref(s), _ptr(x_perm), _ptr(row_scale), _ptr(offsets), _ptr(w1),
          _ptr(w3), _ptr(w2), _ptr(x), _ptr(ws1), _ptr(ws3), _ptr(ws2), _ptr(out),
          _ptr(out_shared), _ptr(ws), ws.numel(), _stream())
    return out, out_shared


def expert_down_combine(s: Shape, h, offsets, src, w2, x, pos, w, h_shared=None, ws2=None, out=None,
                        out_shared=None, y=None, ws=None):
    """moe_expert_down_combine: the down GEMM (with has_shared, the shared
    expert's too) whose tiles also write y.  Returns (out, out_shared, y)."""
    T, d, F = s.T, s.d, s.F
    dev = h.device
    _check(h, "h", (T * s.k, F), s.torch_dtype)
    _check_w(w2, "w2", s, s.N, d, F)
    _check(src, "src", (T * s.k,), torch.int32)
    _check(x, "x", (T, d), s.torch_dtype)
    _check(pos, "pos", (T, s.k), torch.int32)
    _check(w, "w", (T, s.k), torch.float32)
    if s.has_shared:
        _check(h_shared, "h_shared", (T, F), s.torch_dtype)
        _check_w(ws2, "ws2", s, None, d, F)
        if out_shared is None:
            out_shared = torch.empty((T, d), dtype=s.torch_dtype, device=dev)
    if out is None:
        out = torch.empty((T * s.k, d), dtype=s.torch_dtype, device=dev)
    if y is None:
        y = torch.empty((T, d), dtype=s.torch_dtype, device=dev)
    ws = ws if ws is not None else alloc_workspace(s, dev)
    _call("moe_expert_down_combine", ctypes.byref(s), _ptr(h), _ptr(offsets), _ptr(src), _ptr(w2),
          _ptr(out), _ptr(h_shared), _ptr(ws2), _ptr(out_shared), _ptr(x), _ptr(pos), _ptr(w), _ptr(y),
          _ptr(ws), ws.numel(), _stream())
    return out, out_shared, y


def combine(s: Shape, out, out_shared, x, pos, w, y=None):
    T, d = s.T, s.d
    _check(out, "out", (T * s.k, d), s.torch_dtype)
    _check(out_shared, "out_shared", (T, d), s.torch_dtype, required=bool(s.has_shared))
    _check(pos, "pos", (T, s.k), torch.int32)
    _check(w, "w", (T, s.k), torch.float32)
    if y is None:
        y = torch.empty((T, d), dtype=s.torch_dtype, device=x.device)
    _call("moe_combine", ctypes.byref(s), _ptr(out), _ptr(out_shared), _ptr(x), _ptr(pos), _ptr(w),
          _ptr(y), _stream())
    return y


class Layer:
    """One MoE layer with every output and scratch buffer allocated once, so
    that ``forward()`` only enqueues the library's kernels (what a timed loop or
    a captured graph needs).  Buffers are exposed as attributes."""

    def __init__(self, s: Shape, wg, w1, w3, w2, bias=None, ws1=None, ws3=None, ws2=None,
                 device="cuda", fused=False, scatter=False):
        st = check_shape(s)
        if st != MOE_OK:
            raise MoeError("moe_check_shape", st)
        self.s = s
        T, N, k, d, F = s.T, s.N, s.k, s.d, s.F
        dt = s.torch_dtype
        _check(wg, "wg", (N, d), dt)
        _check_w(w1, "w1", s, N, F, d)
        _check_w(w3, "w3", s, N, F, d, required=s.act == MOE_ACT_SWIGLU)
        _check_w(w2, "w2", s, N, d, F)
        _check(bias, "bias", (N,), torch.float32, required=False)
        if s.has_shared:
            _check_w(ws1, "ws1", s, None, F, d)
            _check_w(ws3, "ws3", s, None, F, d, required=s.act == MOE_ACT_SWIGLU)
            _check_w(ws2, "ws2", s, None, d, F)
        self.wg, self.w1, self.w3, self.w2, self.bias = wg, w1, w3, w2, bias
        self.ws1, self.ws3, self.ws2 = ws1, ws3, ws2
        e = dict(dtype=torch.int32, device=device)
        f = dict(dtype=torch.float32, device=device)
        self.idx = torch.empty((T, k), **e)
        self.w = torch.empty((T, k), **f)
        self.counts = torch.empty(N, **e)
        self.kept_counts = torch.empty(N, **e)
        self.p = torch.empty(N, **f)
        self.f = torch.empty(N, **f)
        self.l_aux = torch.empty(1, **f)
        self.offsets = torch.empty(N + 1, **e)
        self.pos = torch.empty((T, k), **e)
        self.src = torch.empty(T * k, **e)
        self.drop = torch.empty((T, k), dtype=torch.uint8, device=device)
        # fused: no dispatch buffer (the up GEMM gathers rows of x through src);
        # scatter (fused only): the down GEMM's tiles also write y (no combine launch)
        if scatter and not fused:
            raise ValueError("scatter needs fused=True")
        self.fused = fused
        self.scatter = scatter
        self.x_perm = None if fused else torch.empty((T * k, d), dtype=s.buf_torch_dtype, device=device)
        self.row_scale = torch.empty(T * k, **f) if s.buf_dtype == MOE_FP8_E4M3 else None
        self.x_codes = (torch.empty((T, d), dtype=torch.uint8, device=device)
                        if fused and s.buf_dtype == MOE_FP8_E4M3 else None)
        self.out = torch.empty((T * k, d), dtype=dt, device=device)
        self.out_shared = torch.empty((T, d), dtype=dt, device=device) if s.has_shared else None
        self.y = torch.empty((T, d), dtype=dt, device=device)
        self.ws = alloc_workspace(s, device)

    def forward(self, x) -> torch.Tensor:
        s = self.s
        _check(x, "x", (s.T, s.d), s.torch_dtype)
        if self.scatter:
            _call("moe_forward_scatter", ctypes.byref(s), _ptr(x), _ptr(self.wg), _ptr(self.bias),
                  _ptr(self.w1), _ptr(self.w3), _ptr(self.w2), _ptr(self.ws1), _ptr(self.ws3),
                  _ptr(self.ws2), _ptr(self.idx), _ptr(self.w), _ptr(self.counts),
                  _ptr(self.kept_counts), _ptr(self.p), _ptr(self.f), _ptr(self.l_aux),
                  _ptr(self.offsets), _ptr(self.pos), _ptr(self.src), _ptr(self.drop),
                  _ptr(self.row_scale), _ptr(self.out), _ptr(self.out_shared),
                  _ptr(self.y), _ptr(self.ws), self.ws.numel(), _stream())
            return self.y
        _call("moe_forward", ctypes.byref(s), _ptr(x), _ptr(self.wg), _ptr(self.bias),
              _ptr(self.w1), _ptr(self.w3), _ptr(self.w2), _ptr(self.ws1), _ptr(self.ws3),
              _ptr(self.ws2), _ptr(self.idx), _ptr(self.w), _ptr(self.counts),
              _ptr(self.kept_counts), _ptr(self.p), _ptr(self.f), _ptr(self.l_aux),
              _ptr(self.offsets), _ptr(self.pos), _ptr(self.src), _ptr(self.drop),
              _ptr(self.x_perm), _ptr(self.row_scale), _ptr(self.out), _ptr(self.out_shared),
              _ptr(self.y), _ptr(self.ws), self.ws.numel(), _stream())
        return self.y

    # the fused layer's phases (the same kernels as forward() with fused=True)
    def route_plan(self, x):
        s = self.s
        _call("moe_route_plan", ctypes.byref(s), _ptr(x), _ptr(self.wg), _ptr(self.bias),
              _ptr(self.idx), _ptr(self.w), _ptr(self.counts), _ptr(self.kept_counts),
              _ptr(self.p), _ptr(self.f), _ptr(self.l_aux), _ptr(self.offsets), _ptr(self.pos),
              _ptr(self.src), _ptr(self.drop), _ptr(self.x_codes), _ptr(self.row_scale),
              _ptr(self.ws), self.ws.numel(), _stream())

    def expert_up_gather(self, x, h):
        s = self.s
        a = self.x_codes if self.x_codes is not None else x
        _call("moe_expert_up_gather", ctypes.byref(s), _ptr(a), _ptr(self.row_scale),
              _ptr(self.offsets), _ptr(self.src), _ptr(self.w1), _ptr(self.w3), _ptr(h),
              _ptr(self.ws), self.ws.numel(), _stream())

    def expert_up_gather_shared(self, x, h, h_shared):
        s = self.s
        a = self.x_codes if self.x_codes is not None else x
        _call("moe_expert_up_gather_shared", ctypes.byref(s), _ptr(a), _ptr(self.row_scale),
              _ptr(self.offsets), _ptr(self.src), _ptr(self.w1), _ptr(self.w3), _ptr(h), _ptr(x),
              _ptr(self.ws1), _ptr(self.ws3), _ptr(h_shared), _ptr(self.ws), self.ws.numel(), _stream())

    def expert_down_combine(self, x, h, h_shared=None):
        """The scatter layer's last phase: down GEMM(s) writing out and y."""
        s = self.s
        _call("moe_expert_down_combine", ctypes.byref(s), _ptr(h), _ptr(self.offsets), _ptr(self.src),
              _ptr(self.w2), _ptr(self.out), _ptr(h_shared), _ptr(self.ws2), _ptr(self.out_shared), _ptr(x),
              _ptr(self.pos), _ptr(self.w), _ptr(self.y), _ptr(self.ws), self.ws.numel(), _stream())

    # forward in three calls (the same kernels): route + dispatch, experts, combine
    def route_dispatch(self, x):
        s = self.s
        _call("moe_route_dispatch", ctypes.byref(s), _ptr(x), _ptr(self.wg), _ptr(self.bias),
              _ptr(self.idx), _ptr(self.w), _ptr(self.counts), _ptr(self.kept_counts),
              _ptr(self.p), _ptr(self.f), _ptr(self.l_aux), _ptr(self.offsets), _ptr(self.pos),
              _ptr(self.src), _ptr(self.drop), _ptr(self.x_perm), _ptr(self.row_scale),
              _ptr(self.ws), self.ws.numel(), _stream())

    # the single phases (route and dispatch as separate calls)
    def route(self, x):
        s = self.s
        _call("moe_route", ctypes.byref(s), _ptr(x), _ptr(self.wg), _ptr(self.bias), _ptr(self.idx),
              _ptr(self.w), _ptr(self.counts), _ptr(self.kept_counts), _ptr(self.p), _ptr(self.f),
              _ptr(self.l_aux), None, _ptr(self.ws), self.ws.numel(), _stream())

    def dispatch(self, x):
        s = self.s
        _call("moe_dispatch", ctypes.byref(s), _ptr(x), _ptr(self.idx), _ptr(self.offsets),
              _ptr(self.pos), _ptr(self.src), _ptr(self.drop), _ptr(self.x_perm),
              _ptr(self.row_scale), _ptr(self.ws), self.ws.numel(), _stream())

    def experts(self, x):
        s = self.s
        _call("moe_experts", ctypes.byref(s), _ptr(self.x_perm), _ptr(self.row_scale),
              _ptr(self.offsets), _ptr(self.w1), _ptr(self.w3), _ptr(self.w2), _ptr(x),
              _ptr(self.ws1), _ptr(self.ws3), _ptr(self.ws2), _ptr(self.out),
              _ptr(self.out_shared), _ptr(self.ws), self.ws.numel(), _stream())

    def combine(self, x):
        s = self.s
        _call("moe_combine", ctypes.byref(s), _ptr(self.out), _ptr(self.out_shared), _ptr(x),
              _ptr(self.pos), _ptr(self.w), _ptr(self.y), _stream())
