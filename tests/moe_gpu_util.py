"""Helpers shared by the GPU parity tests: upload the seeded inputs, run the
HIP path through the binding (C ABI), and compare every output with the
oracle under the acceptance rules:

  * routing (idx), counts, kept counts, offsets, pos, src, drop: bit-exact
    after tie-band adoption (tokens whose k-th/(k+1)-th logits differ by at most
    1e-5 * max|l| may be routed either way; see oracle.compare);
  * the dispatch buffer: bit-exact (a copy, or fp8 codes and scales that both
    sides compute with the same float32 operations);
  * w, p, f, L_aux (float32): relative L2 <= 1e-5;
  * y: relative L2 <= 1e-5 for float32 layers, <= 2e-2 for bf16 layers,
    against the float64 oracle.
"""
from __future__ import annotations

import numpy as np
import torch

import synthetic_inputs as si
from mixture_experts_layer_sparse_amd import moe as M
from oracle import compare, moe as om
from oracle.numerics import e4m3_decode

TOL_F32 = 1e-5
TOL_BF16 = 2e-2


def dev(arr, dtype: str | None = None):
    """numpy array -> device tensor (uint16 bf16 bits -> torch.bfloat16)."""
    if arr is None:
        return None
    if arr.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(arr)).cuda()


def host(t):
    if t is None:
        return None
    t = t.detach()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def bf16_bits_to_f64(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def as_values(arr, dtype):
    return bf16_bits_to_f64(arr) if dtype == "bf16" else np.asarray(arr, np.float64)


def upload(wl, inp):
    d = {k: dev(v) for k, v in inp.items() if v is not None}
    return d


def run_gpu(wl, inp, logits=True, g=None):
    """Run the four phases through the C ABI; returns host copies of everything.
    ``g``: the inputs already on the device (from upload), else uploaded here."""
    s = M.shape_of(wl)
    g = g if g is not None else upload(wl, inp)
    ws = M.alloc_workspace(s)
    r = M.route(s, g["x"], g["wg"], g.get("bias"), ws=ws, logits=logits)
    dsp = M.dispatch(s, g["x"], r["idx"], ws=ws)
    out, out_shared = M.experts(s, dsp["x_perm"], dsp["row_scale"], dsp["offsets"], g["w1"],
                                g.get("w3"), g["w2"], x=g["x"], ws1=g.get("ws1"),
                                ws3=g.get("ws3"), ws2=g.get("ws2"), ws=ws)
    y = M.combine(s, out, out_shared, g["x"], dsp["pos"], r["w"])
    torch.cuda.synchronize()
    res = {k: host(v) for k, v in r.items()}
    res.update({k: host(v) for k, v in dsp.items()})
    res["out"] = host(out)
    res["out_shared"] = host(out_shared)
    res["y"] = host(y)
    return res


def run_experts_no_workspace(wl, inp):
    """Route and dispatch as run_gpu, then the two grouped GEMMs called alone
    without a workspace (a mostly idle last tile round runs as quarter tiles
    instead of split-K); host copies of offsets and out."""
    s = M.shape_of(wl)
    g = upload(wl, inp)
    r = M.route(s, g["x"], g["wg"], g.get("bias"))
    dsp = M.dispatch(s, g["x"], r["idx"])
    h = M.expert_up(s, dsp["x_perm"], dsp["row_scale"], dsp["offsets"], g["w1"], g.get("w3"))
    out = M.expert_down(s, h, dsp["offsets"], g["w2"])
    torch.cuda.synchronize()
    return {"offsets": host(dsp["offsets"]), "out": host(out)}


def rows_rel_err(a, b):
    """Largest per-row relative L2 difference of two bf16/f32 row blocks."""
    a = as_values(a, "bf16") if a.dtype == np.uint16 else a.astype(np.float64)
    b = as_values(b, "bf16") if b.dtype == np.uint16 else b.astype(np.float64)
    num = np.sqrt(np.sum((a - b) ** 2, axis=1))
    den = np.maximum(np.sqrt(np.sum(b ** 2, axis=1)), 1e-30)
    return float(np.max(num / den)) if a.size else 0.0


def run_gpu_forward(wl, inp, g=None, fused=False, scatter=False):
    """The whole layer in one call (moe_forward); host copies of its outputs
    under the same names as run_gpu.  ``g`` as for run_gpu.  ``fused``: no
    dispatch buffer (x_perm is None), the up GEMM gathers x through src.
    ``scatter`` (fused): moe_forward_scatter, the down GEMM writing y; the result
    then also holds ``y_combine``, moe_combine run on the call's own expert
    outputs, which the down GEMM's y must equal bit for bit."""
    s = M.shape_of(wl)
    g = g if g is not None else upload(wl, inp)
    L = M.Layer(s, g["wg"], g["w1"], g.get("w3"), g["w2"], bias=g.get("bias"), ws1=g.get("ws1"),
                ws3=g.get("ws3"), ws2=g.get("ws2"), fused=fused or scatter, scatter=scatter)
    L.forward(g["x"])
    torch.cuda.synchronize()
    names = ["idx", "w", "counts", "kept_counts", "p", "f", "l_aux", "offsets", "pos", "src",
             "drop", "x_perm", "row_scale", "out", "out_shared", "y"]
    res = {n: host(getattr(L, n)) for n in names}
    if scatter:
        yc = M.combine(s, L.out, L.out_shared, g["x"], L.pos, L.w)
        torch.cuda.synchronize()
        res["y_combine"] = host(yc)
    return res


def check_layer(wl, inp, gpu, y_tokens=None, max_adopted=None):
    """Compare a GPU run with the oracle; returns a dict of measured errors."""
    from oracle.numerics import as_f64
    r0 = om.route(wl, as_f64(inp["x"], wl.dtype), as_f64(inp["wg"], wl.dtype), inp.get("bias"))
    ad = compare.adopt(wl, r0["logits"], r0["idx"], gpu["idx"])
    assert ad["bad"] == [], f"{wl.name}: non-admissible routing at tokens {ad['bad'][:10]}"
    if max_adopted is not None:
        assert len(ad["adopted"]) <= max_adopted, f"{wl.name}: {len(ad['adopted'])} tokens adopted"
    routed = {"idx": ad["idx"], "w": ad["w"]}
    full = om.forward(wl, inp, ffn_tokens=y_tokens, routed=routed)
    errs = {"adopted": len(ad["adopted"])}
    assert np.array_equal(gpu["idx"], full["idx"]), "idx"
    errs["w"] = compare.rel_l2(gpu["w"], full["w"])
    assert errs["w"] <= TOL_F32, errs
    assert np.array_equal(gpu["counts"], full["counts"]), "counts"
    assert np.array_equal(gpu["kept_counts"], full["kept_counts"]), "kept_counts"
    errs["p"] = compare.rel_l2(gpu["p"], full["p"])
    errs["f"] = compare.rel_l2(gpu["f"], full["f"])
    errs["l_aux"] = abs(float(gpu["l_aux"][0]) - full["l_aux"]) / max(abs(full["l_aux"]), 1e-30)
    assert errs["p"] <= TOL_F32 and errs["f"] <= TOL_F32 and errs["l_aux"] <= TOL_F32, errs
    if "logits" in gpu and gpu["logits"] is not None:
        errs["logits"] = compare.rel_l2(gpu["logits"], full["logits"])
        assert errs["logits"] <= TOL_F32, errs
    # dispatch plan: bit-exact
    R = int(full["offsets"][-1])
    assert np.array_equal(gpu["offsets"], full["offsets"]), "offsets"
    assert np.array_equal(gpu["pos"], full["pos"]), "pos"
    assert np.array_equal(gpu["src"][:R], full["src"]), "src"
    assert np.array_equal(gpu["drop"].astype(bool), full["drop"]), "drop"
    # dispatch buffer (absent in the fused layer): bit-exact
    if wl.buf == "fp8":
        if gpu["x_perm"] is not None:
            assert np.array_equal(gpu["x_perm"][:R], full["xperm"]), "fp8 codes"
        assert np.array_equal(gpu["row_scale"][:R], full["row_scale"]), "fp8 scales"
    elif gpu["x_perm"] is not None:
        assert np.array_equal(gpu["x_perm"][:R], full["xperm"]), "x_perm"
    # expert outputs and y
    tol = TOL_F32 if wl.dtype == "f32" else TOL_BF16
    toks = full["y_tokens"]
    rows = full["pos"][toks]
    rows = rows[rows >= 0]
    if rows.size:
        got, want = as_values(gpu["out"][rows], wl.dtype), full["o_rows"][rows]
        errs["out"] = compare.rel_l2(got, want)
        # every row on its own too, so that one wrong tile cannot hide in the mean
        errs["out_row_max"] = row_max_rel(got, want)
        assert errs["out"] <= tol and errs["out_row_max"] <= tol, errs
    if wl.shared:
        errs["shared"] = compare.rel_l2(as_values(gpu["out_shared"][toks], wl.dtype), full["shared"])
        assert errs["shared"] <= tol, errs
    got_y = as_values(gpu["y"][toks], wl.dtype)
    errs["y"] = compare.rel_l2(got_y, full["y"])
    # and token by token, so that one mis-weighted slot cannot hide in the norm
    errs["y_row_max"] = row_max_rel(got_y, full["y"])
    assert errs["y"] <= tol and errs["y_row_max"] <= tol, errs
    if wl.buf == "fp8" and getattr(wl, "wfmt", "bf16") != "mxfp4":
        # the same layer without the fp8 step (the shared expert never had one):
        # how far the quantised dispatch moves y, reported beside the error
        # against the fp8-defined oracle
        nofp8 = om.forward(wl.replace(buf=wl.dtype), inp, ffn_tokens=toks, routed=routed)
        errs["y_vs_no_fp8"] = compare.rel_l2(got_y, nofp8["y"])
    return errs


def row_max_rel(got, want):
    """Largest per-row relative L2 difference (absolute where a reference row
    is all zeros)."""
    if got.size == 0:
        return 0.0
    num = np.sqrt(np.sum((got - want) ** 2, axis=1))
    den = np.sqrt(np.sum(want ** 2, axis=1))
    return float(np.max(np.where(den > 0, num / np.maximum(den, 1e-300), num)))


def gemm_tail_split(counts, bm, nt):
    """The grouped GEMMs' tail split, restated on the host: m-tiles of height bm
    per expert segment times nt n-tiles, cut at total - r, r = total % slots,
    when 0 < r <= slots / 4 (slots: the device's CUs, rounded down to a
    multiple of 8).  Returns (total, tiles before the cut, slots)."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    slots = (cus // 8) * 8
    total = int(np.sum((np.asarray(counts) + bm - 1) // bm)) * nt
    r = total % slots
    cut = total - r if 0 < r <= slots // 4 else total
    return total, cut, slots


def sample_tokens(T, n, seed=0):
    rng = np.random.default_rng(seed)
    pick = rng.choice(T, size=min(n, T), replace=False)
    return np.unique(np.concatenate([pick, [0, T - 1]]))


PLAN_KEYS = ("idx", "w", "counts", "kept_counts", "p", "f", "l_aux", "offsets", "pos", "drop", "y")
ROW_KEYS = ("src", "x_perm", "out")


def assert_same_results(a, b, fp8):
    """Two runs of the layer (moe_forward and the single-phase calls) agree bit
    for bit on every output, rows up to R = offsets[N] for the row buffers."""
    R = int(a["offsets"][-1])
    for key in PLAN_KEYS:
        assert np.array_equal(a[key], b[key]), key
    for key in ROW_KEYS:
        if a[key] is None or b[key] is None:        # (the fused layer has no x_perm)
            continue
        assert np.array_equal(a[key][:R], b[key][:R]), key
    if fp8:
        assert np.array_equal(a["row_scale"][:R], b["row_scale"][:R]), "row_scale"
    if a.get("out_shared") is not None:
        assert np.array_equal(a["out_shared"], b["out_shared"]), "out_shared"
