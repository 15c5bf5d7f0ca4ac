"""Seeded synthetic inputs for the sparse MoE-layer forward.

This module is shared by the CPU oracle's tests, the GPU parity tests and
``bench.py``.  It holds the workload shapes and draws the random inputs; it
contains none of the layer's arithmetic (no routing, no softmax, no FFN).

Workloads (shapes of the architectures in the table of the glossary page
"moe communication costs", and DeepSeek-V3's sizes on "MoE: what it costs to
train and serve"):

    tiny         T=64    d=64   N=8   k=2  F=128    SiLU MLP, fp32 everywhere
    mixtral      T=4096  d=4096 N=8   k=2  F=14336  SwiGLU, bf16
    switch       T=8192  d=1024 N=128 k=1  F=4096   ReLU MLP, bf16, capacity 80,
                                                    dropped slots pass through
    deepseek_v3  T=4096  d=7168 N=256 k=8  F=2048   SwiGLU, bf16, 8 groups of 32
                                                    (keep 4 by top-2 sum), fp8
                                                    e4m3 dispatch buffer with a
                                                    per-token scale, +1 shared expert
    dbrx         T=16384 d=6144 N=16  k=4  F=10752  SwiGLU, bf16, router bias
                                                    b_e = 2 ln(1/(e+1))
    decode(B)    deepseek_v3 with T = B tokens (B = 1, 32, 128: a decode step)

Recipe (identical bytes go to the GPU and to the oracle):
  * every tensor is filled chunk by chunk; chunk ``c`` of tensor ``tag`` is
    drawn from ``numpy.random.default_rng(SeedSequence(seed, spawn_key=(tag, c)))``
    with ``standard_normal(dtype=float32)``; chunks are 2**22 elements;
  * x ~ N(0, 1); W_g, W1, W3 ~ N(0, 1/d); W2 ~ N(0, 1/F) (scale applied in fp32);
  * bf16 workloads round each fp32 draw to bf16 with round-to-nearest-even;
    bf16 tensors are returned as ``uint16`` bit patterns;
  * the router bias (dbrx) is computed in float64 and stored as float32;
  * MXFP4 expert weights (wfmt = "mxfp4"; the router stays in the layer's
    type) are drawn directly in the format, no rounding involved: each weight
    matrix [rows][K] is rows * K / 2 bytes of uniformly drawn code bytes (two
    FP4 E2M1 codes each, every code equally likely), then rows * K / 32 E8M0
    block scales drawn uniformly from e0 - 1, e0, e0 + 1, where e0 puts the
    weights' root mean square near 1 / sqrt(K) (the 16 codes' values have mean
    square 8.5625).
"""
from __future__ import annotations

import dataclasses
import math
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

CHUNK = 1 << 22

# tensor tags used in the seed spawn key
TAG_X, TAG_WG = 1, 2
TAG_W1, TAG_W3, TAG_W2 = 10, 11, 12          # + 16 * expert
TAG_WS1, TAG_WS3, TAG_WS2 = 5, 6, 7          # shared expert
TAG_SCALE = 1 << 20                          # + the weight tag: MXFP4 block scales
MX_BLOCK = 32                                # elements per MXFP4 scale block


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    T: int
    d: int
    N: int
    k: int
    F: int
    act: str = "swiglu"          # "silu" | "relu" | "swiglu"
    dtype: str = "bf16"          # storage of x, W_g, expert weights and y: "f32" | "bf16"
    buf: str = "bf16"            # dispatch buffer: "f32" | "bf16" | "fp8"
    capacity: int = 0            # <= 0: no limit
    drop: str = "passthrough"    # "passthrough" | "zero" | "fallback" (the shared expert)
    n_groups: int = 0            # 0: no group limit
    topk_groups: int = 0
    group_score_k: int = 2
    shared: bool = False
    bias: str | None = None      # None | "zipf2"
    alpha: float = 0.01
    gate: str = "sparse"         # "sparse" (softmax over the k selected) | "full" (full-softmax probability)
    wfmt: str = "bf16"           # expert weights: the layer's dtype ("bf16"/"f32") | "mxfp4"
    seed: int = 0

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)

    @property
    def swiglu(self) -> bool:
        return self.act == "swiglu"


WORKLOADS = {
    "tiny": Workload("tiny", T=64, d=64, N=8, k=2, F=128, act="silu",
                     dtype="f32", buf="f32"),
    "mixtral": Workload("mixtral", T=4096, d=4096, N=8, k=2, F=14336),
    "switch": Workload("switch", T=8192, d=1024, N=128, k=1, F=4096,
                       act="relu", capacity=80),
    "deepseek_v3": Workload("deepseek_v3", T=4096, d=7168, N=256, k=8, F=2048,
                            buf="fp8", n_groups=8, topk_groups=4, shared=True),
    "dbrx": Workload("dbrx", T=16384, d=6144, N=16, k=4, F=10752, bias="zipf2"),
}


def decode(B: int) -> Workload:
    """A decode step at the DeepSeek-V3 shape: B tokens, the same weights and
    router as ``deepseek_v3`` (the worked example "how many experts does one
    decode step touch?" of "MoE: what it costs to train and serve").  The
    token draws are the first B rows of the T = 4096 batch (each chunk's
    draws do not depend on how many are taken)."""
    return WORKLOADS["deepseek_v3"].replace(name=f"deepseek_v3_decode{B}", T=B)


def switch_capacity(T: int, N: int, factor: float = 1.25) -> int:
    """Capacity C = factor * T / N, rounded down to an integer slot count."""
    return int(math.floor(factor * T / N))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); returns uint16 bits.
    Inputs here are finite normal draws, so no NaN handling is needed."""
    b = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = (b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def _workers() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def _fill(tag: int, count: int, scale: float, seed: int, bf16: bool) -> np.ndarray:
    out = np.empty(count, dtype=np.uint16 if bf16 else np.float32)
    nchunks = (count + CHUNK - 1) // CHUNK

    def one(c: int) -> None:
        lo, hi = c * CHUNK, min(count, (c + 1) * CHUNK)
        rng = np.random.default_rng(np.random.SeedSequence(seed, spawn_key=(tag, c)))
        v = rng.standard_normal(hi - lo, dtype=np.float32)
        if scale != 1.0:
            v *= np.float32(scale)
        out[lo:hi] = f32_to_bf16_bits(v) if bf16 else v

    if nchunks <= 1:
        for c in range(nchunks):
            one(c)
    else:
        with ThreadPoolExecutor(_workers()) as ex:
            list(ex.map(one, range(nchunks)))
    return out


def _fill_ints(tag: int, count: int, lo: int, hi: int, seed: int) -> np.ndarray:
    """``count`` uint8 values drawn uniformly from lo..hi, chunk by chunk as _fill."""
    out = np.empty(count, dtype=np.uint8)
    for c in range((count + CHUNK - 1) // CHUNK):
        a, b = c * CHUNK, min(count, (c + 1) * CHUNK)
        rng = np.random.default_rng(np.random.SeedSequence(seed, spawn_key=(tag, c)))
        out[a:b] = rng.integers(lo, hi + 1, size=b - a, dtype=np.uint8)
    return out


def gen_mxfp4(wl: Workload, tag: int, rows: int, K: int) -> np.ndarray:
    """One MXFP4 weight matrix [rows][K] as the library stores it: the code
    bytes (row-major, element 2i in the low nibble of byte i), then the E8M0
    block scales (row-major, K / 32 per row)."""
    e0 = 127 + int(round(math.log2(1.0 / (math.sqrt(8.5625) * math.sqrt(K)))))
    codes = _fill_ints(tag, rows * K // 2, 0, 255, wl.seed)
    scales = _fill_ints(TAG_SCALE + tag, rows * K // MX_BLOCK, e0 - 1, e0 + 1, wl.seed)
    return np.concatenate([codes, scales])


def gen_tensor(wl: Workload, tag: int, shape: tuple, scale: float) -> np.ndarray:
    n = int(np.prod(shape)) if shape else 1
    return _fill(tag, n, scale, wl.seed, wl.dtype == "bf16").reshape(shape)


def router_bias(wl: Workload) -> np.ndarray | None:
    if wl.bias is None:
        return None
    if wl.bias == "zipf2":
        e = np.arange(wl.N, dtype=np.float64)
        return (2.0 * np.log(1.0 / (e + 1.0))).astype(np.float32)
    raise ValueError(f"unknown bias recipe {wl.bias!r}")


def generate(wl: Workload, experts: bool = True) -> dict:
    """All inputs of one workload as numpy arrays (uint16 bf16 bits or float32).

    Keys: x [T][d], wg [N][d], bias [N] or None, and when ``experts``:
    w1 [N][F][d], w3 [N][F][d] (SwiGLU only, else None), w2 [N][d][F],
    ws1/ws3/ws2 for the shared expert (None when absent)."""
    T, d, N, F = wl.T, wl.d, wl.N, wl.F
    out = {
        "x": gen_tensor(wl, TAG_X, (T, d), 1.0),
        "wg": gen_tensor(wl, TAG_WG, (N, d), 1.0 / math.sqrt(d)),
        "bias": router_bias(wl),
    }
    if experts:
        out.update(generate_experts(wl))
    return out


def generate_expert(wl: Workload, e: int) -> tuple:
    """(W1[e], W3[e] or None, W2[e]) for one routed expert."""
    d, F = wl.d, wl.F
    if wl.wfmt == "mxfp4":
        return (gen_mxfp4(wl, TAG_W1 + 16 * e, F, d),
                gen_mxfp4(wl, TAG_W3 + 16 * e, F, d) if wl.swiglu else None,
                gen_mxfp4(wl, TAG_W2 + 16 * e, d, F))
    w1 = gen_tensor(wl, TAG_W1 + 16 * e, (F, d), 1.0 / math.sqrt(d))
    w3 = gen_tensor(wl, TAG_W3 + 16 * e, (F, d), 1.0 / math.sqrt(d)) if wl.swiglu else None
    w2 = gen_tensor(wl, TAG_W2 + 16 * e, (d, F), 1.0 / math.sqrt(F))
    return w1, w3, w2


def mxfp4_bytes(rows: int, K: int) -> int:
    """Bytes of one MXFP4 matrix [rows][K]: codes and block scales."""
    return rows * K // 2 + rows * K // MX_BLOCK


def generate_experts(wl: Workload) -> dict:
    d, N, F = wl.d, wl.N, wl.F
    if wl.wfmt == "mxfp4":
        w1 = np.empty((N, mxfp4_bytes(F, d)), dtype=np.uint8)
        w3 = np.empty((N, mxfp4_bytes(F, d)), dtype=np.uint8) if wl.swiglu else None
        w2 = np.empty((N, mxfp4_bytes(d, F)), dtype=np.uint8)
    else:
        dt = np.uint16 if wl.dtype == "bf16" else np.float32
        w1 = np.empty((N, F, d), dtype=dt)
        w3 = np.empty((N, F, d), dtype=dt) if wl.swiglu else None
        w2 = np.empty((N, d, F), dtype=dt)
    for e in range(N):
        a, b, c = generate_expert(wl, e)
        w1[e] = a
        if w3 is not None:
            w3[e] = b
        w2[e] = c
    out = {"w1": w1, "w3": w3, "w2": w2, "ws1": None, "ws3": None, "ws2": None}
    if wl.shared and wl.wfmt == "mxfp4":
        out["ws1"] = gen_mxfp4(wl, TAG_WS1, F, d)
        out["ws3"] = gen_mxfp4(wl, TAG_WS3, F, d) if wl.swiglu else None
        out["ws2"] = gen_mxfp4(wl, TAG_WS2, d, F)
    elif wl.shared:
        out["ws1"] = gen_tensor(wl, TAG_WS1, (F, d), 1.0 / math.sqrt(d))
        out["ws3"] = gen_tensor(wl, TAG_WS3, (F, d), 1.0 / math.sqrt(d)) if wl.swiglu else None
        out["ws2"] = gen_tensor(wl, TAG_WS2, (d, F), 1.0 / math.sqrt(F))
    return out


def small(name: str, **kw) -> Workload:
    """Reduced versions of each workload family: the same structure (dtype,
    activation, groups, capacity, bias, shared expert, fp8 buffer) at sizes
    the oracle finishes in seconds, with a ragged token count so that the
    last tile of every kernel is partial."""
    base = {
        "tiny": dict(),
        "mixtral": dict(T=1000, d=512, F=768),
        "switch": dict(T=2000, d=256, N=32, F=512, capacity=switch_capacity(2000, 32)),
        "deepseek_v3": dict(T=700, d=512, N=64, k=8, F=256, n_groups=8, topk_groups=4),
        "dbrx": dict(T=1500, d=384, N=16, k=4, F=640),
    }[name]
    base.update(kw)
    return WORKLOADS[name].replace(name=name + "_small", **base)
