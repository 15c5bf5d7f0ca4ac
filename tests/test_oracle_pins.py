"""Pins of the CPU oracle against things other than itself: the pages' printed
numbers (tests/golden), closed forms, invariants, textbook special cases and a
pure-Python brute force on tiny inputs.  No GPU."""
import json
import math
import os
import struct

import numpy as np
import pytest

import synthetic_inputs as si
from oracle import brute, moe
from oracle.numerics import as_f64, bf16_to_f64, e4m3_decode, e4m3_encode

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pages_numbers.json")


def golden():
    with open(GOLDEN) as f:
        return json.load(f)


def tolist(a):
    return np.asarray(a, np.float64).tolist()


# ----------------------------------------------------------- page numbers --

def test_dispatch_bytes_worked_example():
    g = golden()
    e = g["dispatch_bytes_per_token"]
    assert moe.dispatch_bytes(e["k"], e["d"], e["s"]) == e["bytes"] == e["kib"] * 1024
    L = g["dispatch_bytes_per_layer"]
    assert moe.dispatch_bytes(L["T"] * L["k"], L["d"], 2) == L["mib_bf16"] * 2 ** 20
    assert moe.dispatch_bytes(L["T"] * L["k"], L["d"], 1) == L["mib_fp8"] * 2 ** 20
    c = g["cross_node_fp8"]
    assert moe.dispatch_bytes(c["copies"], c["d"], c["s"]) == c["kib"] * 1024


def test_dispatch_buffer_bytes_from_a_real_plan():
    """The oracle's dispatch buffer at the DeepSeek-V3 shape (k=8, d=7168, T=4096,
    no drops) holds exactly the page's 448 MiB in bf16 and 224 MiB in fp8."""
    g = golden()["dispatch_bytes_per_layer"]
    rng = np.random.default_rng(1)
    T, N, k, d = g["T"], 256, g["k"], g["d"]
    idx = np.stack([rng.permutation(N)[:k] for _ in range(T)]).astype(np.int32)
    plan = moe.dispatch_plan(idx, N, 0)
    R = int(plan["offsets"][-1])
    assert R == T * k
    assert R * d * 2 == g["mib_bf16"] * 2 ** 20
    assert R * d * 1 == g["mib_fp8"] * 2 ** 20


def touched_share(n_experts, k, batch):
    """Expected share of n_experts that a batch of tokens reads when each token
    picks k of them uniformly: an expert is missed by one token with
    probability 1 - k/n_experts, so by all of them with that to the power of
    the batch size.  Arguments outside 0 < k <= n_experts, batch >= 0 are
    rejected (the page's worked example states the same domain)."""
    if batch < 0 or k <= 0 or k > n_experts:
        raise ValueError(f"touched_share: bad arguments n={n_experts} k={k} batch={batch}")
    miss_one = 1.0 - k / n_experts
    return 1.0 - math.pow(miss_one, batch)


def test_experts_touched_page_asserts():
    g = golden()["experts_touched"]
    for B, want in g["cases"]:
        assert round(touched_share(g["N"], g["k"], B), 3) == want
    with pytest.raises(ValueError):
        touched_share(8, 9, 1)
    with pytest.raises(ValueError):
        touched_share(8, 2, -1)


def test_experts_touched_empirical_deepseek_routing():
    """The oracle's group-limited routing at the DeepSeek-V3 shape touches
    about the page's share of experts per B-token window (uniform-routing
    estimate; random router rows are exchangeable)."""
    g = golden()["experts_touched"]
    wl = si.WORKLOADS["deepseek_v3"]
    inp = si.generate(wl, experts=False)
    r = moe.route(wl, as_f64(inp["x"], wl.dtype), as_f64(inp["wg"], wl.dtype), None)
    idx = r["idx"]
    for B, want in g["cases"]:
        fr = []
        for s in range(0, wl.T - B + 1, B):
            fr.append(np.unique(idx[s:s + B]).size / wl.N)
        assert abs(np.mean(fr) - want) < 0.03 * max(want, 0.1), (B, np.mean(fr), want)


def test_switch_capacity_golden():
    g = golden()["capacity_switch"]
    assert si.switch_capacity(g["T"], g["N"], g["factor"]) == g["C"]
    assert si.WORKLOADS["switch"].capacity == g["C"]


# ------------------------------------------------------------ number formats --

def test_bf16_widening_exact():
    bits = np.arange(0, 65536, dtype=np.uint32)
    keep = ((bits >> 7) & 0xFF) != 0xFF               # finite patterns
    b = bits[keep].astype(np.uint16)
    v = bf16_to_f64(b)
    ref = np.array([struct.unpack("<f", struct.pack("<I", int(x) << 16))[0] for x in b[::97]])
    assert np.array_equal(v[::97], ref)


def test_bf16_generator_rounding_nearest_even():
    # generator's fp32 -> bf16 rounding against exact decimal reasoning on ties
    cases = {1.0: 0x3F80, 1.0 + 2 ** -8: 0x3F80, 1.0 + 3 * 2 ** -8: 0x3F82,
             1.0 + 2 ** -8 + 2 ** -20: 0x3F81, -2.5: 0xC020}
    for v, want in cases.items():
        assert int(si.f32_to_bf16_bits(np.array([v], np.float32))[0]) == want, v


def _e4m3_table():
    codes = np.arange(256, dtype=np.uint8)
    vals = e4m3_decode(codes)
    return codes, vals


def test_e4m3_decode_spec_points():
    _, vals = _e4m3_table()
    assert vals[0x00] == 0.0 and vals[0x38] == 1.0 and vals[0x7E] == 448.0
    assert vals[0x01] == 2.0 ** -9 and vals[0x08] == 2.0 ** -6 and vals[0x07] == 7 * 2.0 ** -9
    assert np.isnan(vals[0x7F]) and np.isnan(vals[0xFF]) and vals[0xFE] == -448.0
    fin = vals[:0x7F]
    assert np.all(np.diff(fin) > 0)                   # positive codes strictly increasing


def _nearest_even_bruteforce(v):
    """Nearest finite e4m3fn value by exhaustive search; ties to the code with
    an even mantissa; sign from the input."""
    codes = np.arange(0, 0x7F, dtype=np.int64)
    vals = e4m3_decode(codes.astype(np.uint8))
    out = np.empty(v.shape, np.uint8)
    for i, x in enumerate(np.asarray(v, np.float64)):
        dist = np.abs(vals - abs(x))
        best = np.flatnonzero(dist == dist.min())
        c = best[0] if best.size == 1 else [b for b in best if b % 2 == 0][0]
        out[i] = c | (0x80 if math.copysign(1, x) < 0 else 0)
    return out


def test_e4m3_encode_exhaustive_bf16_patterns():
    """Every finite bf16 bit pattern, at several scales that cover the whole
    e4m3 range, encodes to the exhaustive nearest-even table value."""
    bits = np.arange(0, 65536, dtype=np.uint32).astype(np.uint16)
    v = bf16_to_f64(bits)
    v = v[np.isfinite(v)]
    rng = np.random.default_rng(0)
    for scale in (1.0, 2.0 ** -8, 2.0 ** 5, 3.0):
        s = (v * scale).astype(np.float32)
        s = s[np.abs(s.astype(np.float64)) <= 448.0]
        got = e4m3_encode(s)
        pick = rng.choice(s.size, size=min(4000, s.size), replace=False)
        want = _nearest_even_bruteforce(s[pick])
        assert np.array_equal(got[pick], want), scale
        # and the whole set satisfies "nearest": |decode - v| <= half the local gap
        dec = e4m3_decode(got)
        assert np.all(np.abs(dec - s) <= np.abs(s) * 2.0 ** -4 + 2.0 ** -10)


def test_e4m3_encode_midpoints_ties_to_even():
    codes, vals = _e4m3_table()
    fin = vals[:0x7F]
    mids = (fin[:-1] + fin[1:]) / 2.0
    mids32 = mids.astype(np.float32)
    exact = mids32.astype(np.float64) == mids
    got = e4m3_encode(mids32[exact])
    lo = np.arange(0x7E)[exact]
    want = np.where(lo % 2 == 0, lo, lo + 1)
    assert np.array_equal(got.astype(np.int64), want)
    assert e4m3_encode(np.array([-0.0], np.float32))[0] == 0x80


def test_fp8_quantiser_definition():
    x = np.array([[1.0, -0.5, 0.25, 3.0], [0.0, 0.0, -0.0, 0.0], [1e-3, 2e-3, -4e-3, 0.0]], np.float32)
    codes, scale = moe.quantize_fp8_rows(x, "f32")
    assert scale[0] == np.float32(3.0) / np.float32(448.0)
    assert scale[1] == 1.0 and np.array_equal(codes[1], np.array([0, 0, 0x80, 0], np.uint8))
    # the row maximum always maps to the largest code
    assert codes[0, 3] == 0x7E and codes[2, 2] == 0xFE
    # a row below 2^-100 is a zero row: scale 1, every code +-0
    tiny = np.array([[1e-35, -2e-36, 0.0, 1e-38]], np.float32)
    c, sc = moe.quantize_fp8_rows(tiny, "f32")
    assert sc[0] == 1.0 and c.tolist() == [[0x00, 0x80, 0x00, 0x00]]
    # dequantised error within half an e4m3 step (relative 2^-4) of the row max scale
    dq = e4m3_decode(codes) * scale[:, None]
    assert np.all(np.abs(dq - x) <= np.abs(x) * 2.0 ** -4 + scale[:, None] * 2.0 ** -9)


# ------------------------------------------------------------------ routing --

def test_top2_matches_page_kernel_formula():
    """k = 2: the router kernel's two-term stable softmax, w0 = 1/denom and
    w1 = exp(m2 - m1)/denom with denom = exp(0) + exp(m2 - m1)."""
    rng = np.random.default_rng(3)
    l = rng.standard_normal((200, 8))
    idx = moe.top_k(l, np.ones_like(l, bool), 2)
    w = moe.sparse_softmax(l, idx)
    for t in range(200):
        order = sorted(range(8), key=lambda e: (-l[t, e], e))
        m1, m2 = l[t, order[0]], l[t, order[1]]
        denom = math.exp(m1 - m1) + math.exp(m2 - m1)
        assert list(idx[t]) == order[:2]
        assert w[t, 0] == pytest.approx(1.0 / denom, rel=1e-15)
        assert w[t, 1] == pytest.approx(math.exp(m2 - m1) / denom, rel=1e-15)


def test_weights_sum_to_one_and_k1_is_one():
    rng = np.random.default_rng(4)
    l = rng.standard_normal((300, 16)) * 5
    for k in (1, 2, 4, 16):
        w = moe.sparse_softmax(l, moe.top_k(l, np.ones_like(l, bool), k))
        assert np.allclose(w.sum(1), 1.0, rtol=0, atol=1e-14)
        assert np.all(np.diff(w, axis=1) <= 0)          # descending slots
        if k == 1:
            assert np.all(w == 1.0)


def test_full_gate_closed_forms():
    """Full-softmax gate weights ([Glossary] "Router design": the selected
    experts' G(x)_i, not renormalised): with two experts and k = 1 the weight
    is the logistic function of the logit gap; with k = N each row is the whole
    softmax (a permutation of it) and sums to 1; for any k a row is the sparse
    softmax scaled by the selected experts' total probability (written out with
    math.exp, independently of the oracle's NumPy softmax)."""
    full = si.WORKLOADS["tiny"].replace(gate="full")
    rng = np.random.default_rng(11)
    l = rng.standard_normal((100, 2)) * 3
    w = moe.gate_weights(full, l, moe.top_k(l, np.ones_like(l, bool), 1))
    for t in range(100):
        gap = abs(l[t, 0] - l[t, 1])
        assert w[t, 0] == pytest.approx(1.0 / (1.0 + math.exp(-gap)), rel=1e-14)
    l = rng.standard_normal((50, 8)) * 4
    for k in (1, 3, 8):
        idx = moe.top_k(l, np.ones_like(l, bool), k)
        wf = moe.gate_weights(full, l, idx)
        ws = moe.gate_weights(si.WORKLOADS["tiny"], l, idx)
        assert np.array_equal(ws, moe.sparse_softmax(l, idx))
        for t in range(50):
            z = [math.exp(v) for v in l[t]]
            tot = sum(z)
            sel = sum(z[e] for e in idx[t])
            for j, e in enumerate(idx[t]):
                assert wf[t, j] == pytest.approx(z[e] / tot, rel=1e-13)
                assert wf[t, j] == pytest.approx(ws[t, j] * sel / tot, rel=1e-13)
        if k == 8:
            assert np.allclose(wf.sum(1), 1.0, rtol=0, atol=1e-14)
        else:
            assert np.all(wf.sum(1) < 1.0)


def test_ties_go_to_lower_index():
    l = np.zeros((1, 8))
    assert moe.top_k(l, np.ones_like(l, bool), 3).tolist() == [[0, 1, 2]]
    l = np.array([[1.0, 2.0, 2.0, 0.0, 2.0]])
    assert moe.top_k(l, np.ones_like(l, bool), 2).tolist() == [[1, 2]]
    # group ties: equal group scores keep the lower group
    # group scores (top-2 sums) 2, 0, 2, 2: the tie among groups 0, 2, 3 keeps 0 and 2
    l = np.array([[1.0, 1.0, 0.0, 0.0, 2.0, 0.0, 1.5, 0.5]])
    m = moe.group_mask(l, 4, 2, 2)
    assert m.tolist() == [[True, True, False, False, True, True, False, False]]


def test_load_stats_closed_forms():
    N, k, T, alpha = 8, 2, 8, 0.01
    # uniform p (equal logits) and balanced counts: L_aux = alpha
    l = np.zeros((T, N))
    idx = np.array([[2 * (t % 4), 2 * (t % 4) + 1] for t in range(T)], np.int32)
    s = moe.load_stats(l, idx, N, 0, alpha)
    assert np.all(s["counts"] == 2) and s["l_aux"] == pytest.approx(alpha, rel=1e-14)
    assert s["f"].sum() == pytest.approx(1.0) and s["p"].sum() == pytest.approx(1.0)
    # every token to expert 0 with p -> 1: L_aux -> alpha * N
    l = np.full((T, N), -1e4)
    l[:, 0] = 0.0
    idx = np.zeros((T, 1), np.int32)
    s = moe.load_stats(l, idx, N, 0, alpha)
    assert s["l_aux"] == pytest.approx(alpha * N, rel=1e-12)
    # capacity clips kept counts only
    s = moe.load_stats(l, idx, N, 3, alpha)
    assert s["counts"][0] == T and s["kept_counts"][0] == 3


# --------------------------------------------------------------- dispatch --

def test_dispatch_plan_invariants_and_drops():
    rng = np.random.default_rng(5)
    T, N, k, C = 500, 16, 3, 90
    idx = np.stack([rng.choice(N, k, replace=False, p=np.linspace(2, 1, N) / np.linspace(2, 1, N).sum())
                    for _ in range(T)]).astype(np.int32)
    plan = moe.dispatch_plan(idx, N, C)
    counts = np.bincount(idx.ravel(), minlength=N)
    kept = np.minimum(counts, C)
    assert counts.sum() == T * k
    assert np.array_equal(np.diff(plan["offsets"]), kept)
    R = plan["offsets"][-1]
    assert (plan["pos"] >= 0).sum() == R and plan["drop"].sum() == T * k - R
    # each token appears once per kept slot; src strictly increasing per segment
    assert sorted(plan["pos"][plan["pos"] >= 0].tolist()) == list(range(R))
    for e in range(N):
        seg = plan["src"][plan["offsets"][e]:plan["offsets"][e + 1]]
        assert np.all(np.diff(seg) > 0)
        # every row of the segment is a token that chose e
        assert all(e in idx[t] for t in seg)
        # drops: exactly max(0, counts - C), the highest-t tokens of the expert
        toks = np.flatnonzero(np.any(idx == e, axis=1))
        dropped = [t for t in toks if plan["drop"][t][list(idx[t]).index(e)]]
        assert len(dropped) == max(0, counts[e] - C)
        assert dropped == sorted(toks)[len(toks) - len(dropped):]
        assert list(seg) == sorted(toks)[:kept[e]]


def test_permutation_equals_library_stable_sort():
    rng = np.random.default_rng(6)
    T, N, k = 300, 12, 4
    idx = np.stack([rng.permutation(N)[:k] for _ in range(T)]).astype(np.int32)
    plan = moe.dispatch_plan(idx, N, 0)
    order = sorted(range(T * k), key=lambda a: (idx.ravel()[a], a))    # Python's sort
    assert plan["src"].tolist() == [a // k for a in order]


# -------------------------------------------------------- experts / combine --

def test_relu_identity_experts_give_x():
    """ReLU MLP with W1 = [I; -I], W2 = [I, -I] is the identity (relu(v) -
    relu(-v) = v), so the layer returns x exactly: sum_j w_j x = x.  With a
    capacity the dropped slots pass x through, so y = x still."""
    d, N, k, T = 16, 4, 2, 40
    wl = si.Workload("ident", T=T, d=d, N=N, k=k, F=2 * d, act="relu", dtype="f32", buf="f32")
    rng = np.random.default_rng(7)
    x = rng.standard_normal((T, d)).astype(np.float32)
    eye = np.eye(d, dtype=np.float32)
    w1 = np.stack([np.concatenate([eye, -eye])] * N)
    w2 = np.stack([np.concatenate([eye, -eye], axis=1)] * N)
    inp = {"x": x, "wg": rng.standard_normal((N, d)).astype(np.float32), "bias": None,
           "w1": w1, "w3": None, "w2": w2}
    for cap in (0, 7):
        out = moe.forward(wl.replace(capacity=cap), inp)
        assert np.allclose(out["y"], x, rtol=0, atol=1e-12)
        if cap:
            assert out["drop"].sum() > 0
    # drop mode "zero" loses exactly the dropped weight
    out = moe.forward(wl.replace(capacity=7, drop="zero"), inp)
    lost = np.where(out["drop"], out["w"], 0.0).sum(1)
    assert np.allclose(out["y"], x * (1 - lost)[:, None], atol=1e-12)


def test_silu_and_swiglu_closed_forms():
    """The SiLU and SwiGLU experts against closed forms that follow from
    silu(v) = v * sigmoid(v) and sigmoid(v) + sigmoid(-v) = 1:
      * silu(0) = 0, silu(1) = 1 / (1 + e^-1) = 0.7310585786300049...;
      * SiLU with W1 = [I; -I], W2 = [I, I]: silu(v) + silu(-v) = v tanh(v/2)
        (NumPy's tanh; a sign slip inside silu flips the result's sign);
      * SwiGLU with W1 = [I; -I], W3 = [I; I], W2 = [I, -I]: the gate is v in
        both halves, so the output is v (silu(v) - silu(-v)) = v * v (a swap of
        the gate and W1 halves gives v^2 tanh(v/2) instead);
    so the layer returns x tanh(x/2) and x * x (sum_j w_j = 1)."""
    assert moe.activation("silu", np.array([0.0]))[0] == 0.0
    assert moe.activation("silu", np.array([1.0]))[0] == pytest.approx(0.7310585786300049, rel=1e-15)
    d, N, k, T = 12, 4, 2, 30
    rng = np.random.default_rng(12)
    x = (rng.standard_normal((T, d)) * 3).astype(np.float32)
    eye = np.eye(d, dtype=np.float32)
    W1 = np.concatenate([eye, -eye])
    common = {"x": x, "wg": rng.standard_normal((N, d)).astype(np.float32), "bias": None}
    xs = x.astype(np.float64)
    wl = si.Workload("silu_cf", T=T, d=d, N=N, k=k, F=2 * d, act="silu", dtype="f32", buf="f32")
    out = moe.forward(wl, dict(common, w1=np.stack([W1] * N), w3=None,
                               w2=np.stack([np.concatenate([eye, eye], axis=1)] * N)))
    assert np.allclose(out["y"], xs * np.tanh(xs / 2.0), rtol=1e-12, atol=1e-12)
    wl = wl.replace(name="swiglu_cf", act="swiglu")
    out = moe.forward(wl, dict(common, w1=np.stack([W1] * N),
                               w3=np.stack([np.concatenate([eye, eye])] * N),
                               w2=np.stack([np.concatenate([eye, -eye], axis=1)] * N)))
    assert np.allclose(out["y"], xs * xs, rtol=1e-12, atol=1e-12)


def test_shared_identity_doubles():
    d, N, k, T = 8, 4, 2, 20
    wl = si.Workload("ident2", T=T, d=d, N=N, k=k, F=2 * d, act="relu", dtype="f32",
                     buf="f32", shared=True)
    rng = np.random.default_rng(8)
    x = rng.standard_normal((T, d)).astype(np.float32)
    eye = np.eye(d, dtype=np.float32)
    W1 = np.concatenate([eye, -eye]); W2 = np.concatenate([eye, -eye], axis=1)
    inp = {"x": x, "wg": rng.standard_normal((N, d)).astype(np.float32), "bias": None,
           "w1": np.stack([W1] * N), "w3": None, "w2": np.stack([W2] * N),
           "ws1": W1, "ws3": None, "ws2": W2}
    out = moe.forward(wl, inp)
    assert np.allclose(out["y"], 2 * x, atol=1e-12)


def test_fallback_to_shared_expert_closed_forms():
    """drop = fallback: a slot over the capacity is served by the shared expert
    S.  With identity routed experts and an identity S every slot gives x, so
    y = x + x whatever drops; with zero routed experts only the dropped slots
    and the always-on term remain: y = (1 + sum of the dropped weights) x."""
    d, N, k, T = 8, 4, 2, 30
    wl = si.Workload("fb", T=T, d=d, N=N, k=k, F=2 * d, act="relu", dtype="f32", buf="f32",
                     shared=True, capacity=6, drop="fallback")
    rng = np.random.default_rng(9)
    x = rng.standard_normal((T, d)).astype(np.float32)
    eye = np.eye(d, dtype=np.float32)
    W1 = np.concatenate([eye, -eye]); W2 = np.concatenate([eye, -eye], axis=1)
    inp = {"x": x, "wg": rng.standard_normal((N, d)).astype(np.float32), "bias": None,
           "w1": np.stack([W1] * N), "w3": None, "w2": np.stack([W2] * N),
           "ws1": W1, "ws3": None, "ws2": W2}
    out = moe.forward(wl, inp)
    assert out["drop"].sum() > 0
    assert np.allclose(out["y"], 2 * x, rtol=0, atol=1e-12)
    inp0 = dict(inp, w1=np.zeros_like(inp["w1"]), w2=np.zeros_like(inp["w2"]))
    out = moe.forward(wl, inp0)
    dropped = np.where(out["drop"], out["w"], 0.0).sum(1)
    assert np.allclose(out["y"], x * (1.0 + dropped)[:, None], rtol=0, atol=1e-12)
    # the other drop modes on the same routing: pass-through gives 2x, zero x (1 + 1 - dropped)
    out = moe.forward(wl.replace(drop="zero"), inp)
    assert np.allclose(out["y"], x * (2.0 - dropped)[:, None], rtol=0, atol=1e-12)


def _tiny_cases():
    yield si.WORKLOADS["tiny"].replace(T=24, d=12, F=10)
    yield si.Workload("sw", T=30, d=10, N=6, k=1, F=14, act="relu", dtype="f32", buf="f32", capacity=4)
    yield si.Workload("sw0", T=30, d=10, N=6, k=2, F=14, act="relu", dtype="f32", buf="f32",
                      capacity=5, drop="zero")
    yield si.Workload("ds", T=20, d=12, N=16, k=4, F=6, act="swiglu", dtype="bf16", buf="fp8",
                      n_groups=4, topk_groups=2, shared=True)
    yield si.Workload("db", T=25, d=10, N=8, k=3, F=9, act="swiglu", dtype="bf16", buf="bf16",
                      bias="zipf2")
    yield si.Workload("kN", T=9, d=6, N=5, k=5, F=7, act="silu", dtype="f32", buf="f32")
    yield si.Workload("fullgate", T=16, d=10, N=6, k=2, F=9, act="swiglu", dtype="bf16",
                      buf="bf16", n_groups=2, topk_groups=1, gate="full")
    yield si.Workload("fallback", T=30, d=10, N=6, k=2, F=8, act="relu", dtype="f32", buf="f32",
                      capacity=5, drop="fallback", shared=True)


@pytest.mark.parametrize("wl", list(_tiny_cases()), ids=lambda w: w.name)
def test_oracle_equals_bruteforce(wl):
    inp = si.generate(wl)
    out = moe.forward(wl, inp)
    x = as_f64(inp["x"], wl.dtype)
    wg = as_f64(inp["wg"], wl.dtype)
    w1 = [tolist(as_f64(inp["w1"][e], wl.dtype)) for e in range(wl.N)]
    w3 = [tolist(as_f64(inp["w3"][e], wl.dtype)) for e in range(wl.N)] if inp["w3"] is not None else None
    w2 = [tolist(as_f64(inp["w2"][e], wl.dtype)) for e in range(wl.N)]
    ws = None
    if wl.shared:
        ws = (tolist(as_f64(inp["ws1"], wl.dtype)),
              tolist(as_f64(inp["ws3"], wl.dtype)) if inp["ws3"] is not None else None,
              tolist(as_f64(inp["ws2"], wl.dtype)))
    xq = None
    if wl.buf == "fp8":
        codes, scale = moe.quantize_fp8_rows(inp["x"], wl.dtype)
        xq = tolist(e4m3_decode(codes) * scale.astype(np.float64)[:, None])
    b = brute.forward(wl, tolist(x), tolist(wg), None if inp["bias"] is None else tolist(inp["bias"]),
                      w1, w3, w2, ws, xq)
    assert out["idx"].tolist() == b["idx"]
    assert np.allclose(out["w"], b["w"], rtol=1e-13, atol=0)
    assert out["counts"].tolist() == b["counts"]
    assert out["kept_counts"].tolist() == b["kept_counts"]
    assert np.allclose(out["p"], b["p"], rtol=1e-12) and np.allclose(out["f"], b["f"], rtol=1e-15)
    assert out["l_aux"] == pytest.approx(b["l_aux"], rel=1e-12)
    assert out["offsets"].tolist() == b["offsets"]
    assert out["pos"].tolist() == b["pos"] and out["src"].tolist() == b["src"]
    assert np.allclose(out["y"], b["y"], rtol=1e-10, atol=1e-12)


def test_oracle_sampled_ffn_equals_full():
    wl = si.small("dbrx", T=120, d=64, F=128)
    inp = si.generate(wl)
    full = moe.forward(wl, inp)
    toks = np.array([0, 7, 55, 119])
    part = moe.forward(wl, inp, ffn_tokens=toks)
    assert np.allclose(part["y"], full["y"][toks], rtol=1e-12, atol=1e-14)


# ------------------------------------------------------------------- MXFP4 --

def test_fp4_e2m1_code_table():
    """The 16 FP4 E2M1 codes: magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6 for codes
    0-7 (the format's whole value set: 2 exponent bits with bias 1, 1 mantissa
    bit, exponent 0 subnormal), the same negated for codes 8-15, code 8 being
    -0."""
    from oracle.numerics import fp4_e2m1_decode
    v = fp4_e2m1_decode(np.arange(16))
    assert v[:8].tolist() == [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    assert v[8:].tolist() == [-0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0]
    assert math.copysign(1.0, v[8]) == -1.0 and math.copysign(1.0, v[0]) == 1.0


def test_e8m0_and_mxfp4_decode_exhaustive():
    """Every code at every finite E8M0 scale decodes to the code's value times
    2^(e - 127) (math.ldexp, exact); scale 255 is NaN; element 2i sits in the
    low nibble of byte i, and each 32-element block takes its own scale."""
    from oracle.numerics import e8m0_decode, mxfp4_decode
    table = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    e = np.arange(255)
    assert np.all(e8m0_decode(e) == [math.ldexp(1.0, int(x) - 127) for x in e])
    assert np.isnan(e8m0_decode(np.array([255]))[0])
    # one row per scale: 32 elements cycling through the 16 codes twice
    K = 32
    codes = np.tile(np.arange(16, dtype=np.uint8), 2)
    packed = (codes[0::2] | (codes[1::2] << 4)).astype(np.uint8)
    buf = np.concatenate([np.tile(packed, 255), e.astype(np.uint8)])
    got = mxfp4_decode(buf, 255, K)
    for r in range(255):
        for i, c in enumerate(codes):
            want = math.ldexp(table[c & 7], r - 127) * (-1.0 if c & 8 else 1.0)
            assert got[r, i] == want, (r, i)
    # nibble order and per-block scales on a hand-made 1 x 64 row: byte 0 = 0x1F
    # holds element 0 = code 0xF (-6) and element 1 = code 0x1 (0.5); the second
    # block's scale is 2^1
    row = np.zeros(32, np.uint8)
    row[0] = 0x1F
    row[16] = 0x2A                 # elements 32, 33: codes 0xA (-1), 0x2 (1)
    got = mxfp4_decode(np.concatenate([row, np.array([127, 128], np.uint8)]), 1, 64)[0]
    assert got[0] == -6.0 and got[1] == 0.5 and got[32] == -2.0 and got[33] == 2.0
    assert np.count_nonzero(got) == 4


def test_mxfp4_storage_is_the_pages_bits_per_weight():
    g = golden()["mxfp4_bits_per_weight"]
    for rows, K in ((2048, 7168), (7168, 2048), (4096, 1024)):
        assert si.mxfp4_bytes(rows, K) * 8 / (rows * K) == g["bits"]


def test_mxfp4_identity_experts_give_x():
    """I and -I are exact in MXFP4 (codes 0x2 and 0xA at scale 2^0), so the
    ReLU identity experts (W1 = [I; -I], W2 = [I, -I]) stored as MXFP4 return x
    exactly, with capacity drops passing x through."""
    d, N, k, T = 32, 4, 2, 40
    wl = si.Workload("mxid", T=T, d=d, N=N, k=k, F=2 * d, act="relu", dtype="bf16", buf="bf16",
                     capacity=15, wfmt="mxfp4")
    rng = np.random.default_rng(13)

    def mx(m):
        # an exact MXFP4 encoding of a matrix of 0, +1, -1 (scale 2^0 everywhere)
        c = np.where(m > 0, 0x2, np.where(m < 0, 0xA, 0x0)).astype(np.uint8)
        packed = (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8)
        return np.concatenate([packed.ravel(), np.full(m.size // 32, 127, np.uint8)])

    eye = np.eye(d)
    w1 = mx(np.concatenate([eye, -eye]))
    w2 = mx(np.concatenate([eye, -eye], axis=1))
    x = si.f32_to_bf16_bits(rng.standard_normal((T, d)).astype(np.float32))
    inp = {"x": x, "wg": si.f32_to_bf16_bits(rng.standard_normal((N, d)).astype(np.float32)),
           "bias": None, "w1": np.stack([w1] * N), "w3": None, "w2": np.stack([w2] * N)}
    out = moe.forward(wl, inp)
    assert out["drop"].sum() > 0
    assert np.allclose(out["y"], as_f64(x, "bf16"), rtol=1e-14, atol=1e-14)
