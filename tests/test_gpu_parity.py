"""GPU parity: the HIP path (through the C ABI) against the float64 oracle.

Small cases span several tiles of every kernel with ragged tails; full-size
cases run the workloads at their real shapes (all of routing, the plan and the
dispatch buffer compared; y on sampled tokens)."""
import functools

import numpy as np
import pytest
import torch

import synthetic_inputs as si
from mixture_experts_layer_sparse_amd import moe as M

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from moe_gpu_util import check_layer, run_gpu, sample_tokens


def _run_and_check(wl, inp=None, y_tokens=None, max_adopted=None):
    print(f"case {wl.name}: T={wl.T} d={wl.d} N={wl.N} k={wl.k} F={wl.F}", flush=True)
    inp = inp if inp is not None else si.generate(wl)
    gpu = run_gpu(wl, inp)
    errs = check_layer(wl, inp, gpu, y_tokens=y_tokens, max_adopted=max_adopted)
    print(f"  {errs}", flush=True)
    return gpu, errs


@pytest.mark.parametrize("name", ["tiny", "mixtral", "switch", "deepseek_v3", "dbrx"])
def test_small_parity(name):
    wl = si.WORKLOADS["tiny"] if name == "tiny" else si.small(name)
    _run_and_check(wl, max_adopted=2)


def test_tiny_full_config_f32_tolerance():
    gpu, errs = _run_and_check(si.WORKLOADS["tiny"], max_adopted=0)
    assert errs["y"] <= 1e-5


# ------------------------------------------------------------- edge cases --

def test_single_token():
    _run_and_check(si.small("mixtral", T=1))


def test_t_zero_is_noop():
    wl = si.small("mixtral", T=0)
    s = M.shape_of(wl)
    x = torch.empty((0, wl.d), dtype=torch.bfloat16, device="cuda")
    wg = torch.zeros((wl.N, wl.d), dtype=torch.bfloat16, device="cuda")
    r = M.route(s, x, wg, ws=torch.empty(256, dtype=torch.uint8, device="cuda"))
    assert r["idx"].shape == (0, wl.k)


def test_all_tokens_one_expert_and_empty_segments():
    """A large bias sends every token to expert 3 first: one huge segment,
    several empty ones; with a capacity the overflow is dropped."""
    wl = si.small("switch", T=700, N=16, k=2, capacity=0)
    inp = si.generate(wl)
    b = np.zeros(wl.N, np.float32)
    b[3] = 50.0
    b[5] = 40.0
    inp["bias"] = b
    _run_and_check(wl, inp)
    wlc = wl.replace(capacity=100)
    gpu, _ = _run_and_check(wlc, inp)
    assert gpu["drop"].sum() == 2 * (700 - 100)


def test_exact_ties_go_to_lower_index():
    """Duplicated router rows give bit-identical logits: the lower expert wins."""
    wl = si.small("mixtral", T=300, N=8, k=2)
    inp = si.generate(wl)
    wg = inp["wg"].copy()
    wg[5] = wg[1]
    wg[6] = wg[2]
    inp["wg"] = wg
    gpu, _ = _run_and_check(wl, inp, max_adopted=0)
    assert not np.any(gpu["idx"] == 5) or np.all(np.any(gpu["idx"] == 1, axis=1)[np.any(gpu["idx"] == 5, axis=1)])
    for t in range(wl.T):
        sel = list(gpu["idx"][t])
        if 5 in sel:
            assert 1 in sel and sel.index(1) < sel.index(5)
        if 6 in sel:
            assert 2 in sel and sel.index(2) < sel.index(6)


def test_zero_rows_and_k_equals_n():
    wl = si.Workload("kN", T=130, d=128, N=4, k=4, F=128, act="swiglu", dtype="bf16", buf="fp8")
    inp = si.generate(wl)
    x = inp["x"].copy()
    x[7] = 0
    x[64] = 0x8000      # -0.0 everywhere
    inp["x"] = x
    gpu, _ = _run_and_check(wl, inp)
    assert np.all(gpu["row_scale"][gpu["pos"][7]] == 1.0)


def test_capacity_one_and_drop_zero():
    wl = si.small("switch", T=400, N=8, k=2, capacity=1, drop="zero")
    gpu, _ = _run_and_check(wl)
    assert gpu["offsets"][-1] == 8


def test_many_tokens_with_capacity():
    """80 dispatch blocks with a capacity that drops a few percent of the
    assignments, on a cheap layer width."""
    wl = si.Workload("mb", T=20011, d=64, N=16, k=2, F=128, act="swiglu", dtype="bf16",
                     buf="bf16", capacity=2300)
    gpu, _ = _run_and_check(wl)
    assert gpu["drop"].sum() > 0


def _check_tail_paths(wl, gpu):
    """The tail as split-K (moe_experts, with a workspace: gpu, already checked
    against the oracle) and as quarter tiles (the GEMM calls alone, without a
    workspace) must agree row by row to rounding."""
    from moe_gpu_util import rows_rel_err, run_experts_no_workspace
    q = run_experts_no_workspace(wl, si.generate(wl))
    assert np.array_equal(q["offsets"], gpu["offsets"])
    R = int(gpu["offsets"][-1])
    err = rows_rel_err(q["out"][:R], gpu["out"][:R])
    print(f"  split-K vs quarter tiles: max row rel err {err:.2e}", flush=True)
    assert err <= 1e-2


@pytest.mark.parametrize("act,buf", [("swiglu", "bf16"), ("relu", "fp8")])
def test_gemm_tail_only(act, buf):
    """Fewer 256-row tiles than a quarter of the CUs: every tile is in the
    tail, as split-K partials or as 128x128 quarters (including quarters
    wholly past a segment end or past the last output column: d = 320, and
    F = 384 with ReLU)."""
    from moe_gpu_util import gemm_tail_split
    wl = si.Workload("tq", T=2000, d=320, N=8, k=2, F=384, act=act, dtype="bf16", buf=buf)
    gpu, errs = _run_and_check(wl)
    nt_up = -(-wl.F // 128) if act == "swiglu" else -(-wl.F // 256)
    for nt in (nt_up, -(-wl.d // 256)):
        total, cut, _ = gemm_tail_split(gpu["kept_counts"], 256, nt)
        assert cut == 0 and total > 0, (total, cut)
    _check_tail_paths(wl, gpu)


def test_gemm_main_and_tail():
    """Whole rounds of 256x256 tiles plus a tail in both GEMMs; every token's
    y is compared, and both forms of the tail."""
    from moe_gpu_util import gemm_tail_split
    wl = si.Workload("tm", T=34000, d=256, N=16, k=2, F=256, act="swiglu", dtype="bf16",
                     buf="bf16")
    gpu, errs = _run_and_check(wl)
    for nt in (wl.F // 128, 1):
        total, cut, slots = gemm_tail_split(gpu["kept_counts"], 256, nt)
        assert slots <= cut < total, (total, cut, slots)
    _check_tail_paths(wl, gpu)


FULL_GATE_CASES = {
    "tiny_f32": lambda: si.WORKLOADS["tiny"],
    "switch_k1_capacity": lambda: si.small("switch"),
    "mixtral": lambda: si.small("mixtral"),
    "mixtral_one_token": lambda: si.small("mixtral", T=1),
    "deepseek_groups_fp8_shared": lambda: si.small("deepseek_v3"),
}


@pytest.mark.parametrize("name", list(FULL_GATE_CASES))
def test_full_softmax_gate(name):
    """gate = full: each selected expert weighted by its probability under the
    softmax over all N logits.  Lane and wave selection paths, split logits
    (one token), groups, capacity drops and the fp8 buffer; every output
    against the oracle, y on all tokens."""
    wl = FULL_GATE_CASES[name]().replace(gate="full")
    gpu, _ = _run_and_check(wl, max_adopted=2)
    assert np.all(gpu["w"].sum(axis=1) <= 1.0 + 1e-6)


FALLBACK_CASES = {
    "switch_k1": lambda: si.small("switch", shared=True, drop="fallback"),
    "deepseek_fp8_groups": lambda: si.small("deepseek_v3", capacity=70, drop="fallback"),
    "f32": lambda: si.Workload("fb32", T=333, d=64, N=8, k=2, F=96, act="silu", dtype="f32",
                               buf="f32", capacity=70, shared=True, drop="fallback"),
}


@pytest.mark.parametrize("name", list(FALLBACK_CASES))
def test_drop_to_shared_fallback(name):
    """drop = fallback: a slot over the capacity is served by the shared expert
    (its output row weighted by the slot's weight) on top of the always-on
    term.  Every output against the oracle, y on all tokens, with drops."""
    wl = FALLBACK_CASES[name]()
    gpu, errs = _run_and_check(wl, max_adopted=2)
    assert gpu["drop"].sum() > 0
    if wl.dtype == "f32":
        assert errs["y"] <= 1e-5


# Wide routers (bf16, 64 to 256 experts, N d >= 2^19, 512 to 16384 tokens) take
# their logits from a split-K GEMM launch; the rest from the router kernel itself.
ROUTER_GEMM_CASES = {
    # ragged last 128-token tile, N not a multiple of 16, d not a multiple of 512, bias
    "ragged": dict(T=600, d=6080, N=96, k=4, F=128, act="relu", bias="zipf2"),
    # the smallest T that takes the GEMM, group limit over groups of 24 (no butterfly)
    "t512_groups": dict(T=512, d=6144, N=96, k=6, F=128, n_groups=4, topk_groups=2),
    # the largest T that takes it (128 tiles, 2 K ranges each), 256 experts, with a capacity
    "t16384": dict(T=16384, d=2048, N=256, k=8, F=64, act="relu", capacity=400),
    # just past it: the router kernel computes the logits again
    "t16400_fallback": dict(T=16400, d=2048, N=256, k=8, F=64, act="relu"),
}


@pytest.mark.parametrize("name", list(ROUTER_GEMM_CASES))
def test_router_logits_gemm(name):
    wl = si.Workload("rg_" + name, **ROUTER_GEMM_CASES[name])
    s = M.shape_of(wl)
    # the split-K partial tiles (32 MiB on 256 CUs) are in the workspace exactly when the GEMM
    # runs: compare with the same layer one expert below the threshold
    small = M.workspace_bytes(M.shape_of(wl.replace(N=63, n_groups=0, topk_groups=0)))
    uses_gemm = name != "t16400_fallback"
    assert (M.workspace_bytes(s) - small > 16 << 20) == uses_gemm
    _run_and_check(wl, y_tokens=sample_tokens(wl.T, 256) if wl.T > 4096 else None)


# At most 16 tokens (one router tile) the router kernel writes the load
# statistics itself; 17 tokens take the statistics kernel again.
ONE_TILE_CASES = {
    "t10_groups_capacity": dict(T=10, d=256, N=32, k=3, F=128, n_groups=4, topk_groups=2, capacity=1),
    "t16_wave_bias": dict(T=16, d=512, N=64, k=4, F=128, bias="zipf2"),
    "t17_two_tiles": dict(T=17, d=512, N=64, k=4, F=128, capacity=2),
    "t5_f32": dict(T=5, d=64, N=8, k=2, F=128, act="silu", dtype="f32", buf="f32"),
}


@pytest.mark.parametrize("name", list(ONE_TILE_CASES))
def test_one_router_tile(name):
    wl = si.Workload("ot_" + name, **ONE_TILE_CASES[name])
    gpu, _ = _run_and_check(wl)
    if wl.capacity:
        assert gpu["drop"].sum() > 0


def test_groups_k_le_group_span():
    wl = si.small("deepseek_v3", T=333, N=32, k=3, n_groups=4, topk_groups=1, F=128)
    _run_and_check(wl)


def test_fp8_quantiser_exhaustive_bf16_patterns():
    """Every finite bf16 pattern goes through the fp8 dispatch quantiser at
    four relative scales: rows of 255 neighbouring patterns plus one anchor
    element A times the row's largest magnitude (A = 1, 2^6, 2^12, 2^19), so
    each pattern lands near the top, the middle, the subnormal range and below
    the smallest code.  Codes and scales must equal the oracle's bit for bit
    (rows below 2^-100 are zero rows on both sides)."""
    from moe_gpu_util import dev, host
    from oracle import moe as om
    from oracle.numerics import bf16_to_f64
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    finite = ((bits.astype(np.uint32) >> 7) & 0xFF) != 0xFF
    vals = bits[finite]
    vals = np.concatenate([vals, np.zeros((-vals.size) % 255, np.uint16)]).reshape(-1, 255)
    mags = np.abs(bf16_to_f64(vals)).max(axis=1)
    rows = []
    for A in (1.0, 2.0 ** 6, 2.0 ** 12, 2.0 ** 19):
        anchor = mags * A
        ok = anchor < 3.3e38
        a_bits = si.f32_to_bf16_bits(anchor[ok].astype(np.float32))
        assert np.array_equal(bf16_to_f64(a_bits), anchor[ok])       # exact anchors
        rows.append(np.concatenate([vals[ok], a_bits[:, None]], axis=1))
    x_all = np.concatenate(rows)
    # all rows, then the first 300 (a ragged grid)
    for x in (x_all, x_all[:300]):
        T, d = x.shape
        wl = si.Workload("q", T=T, d=d, N=4, k=1, F=64, act="swiglu", dtype="bf16", buf="fp8")
        s = M.shape_of(wl)
        idx = torch.zeros((T, 1), dtype=torch.int32, device="cuda")
        dsp = M.dispatch(s, dev(x), idx)
        torch.cuda.synchronize()
        codes, scale = om.quantize_fp8_rows(x, "bf16")
        got_c, got_s = host(dsp["x_perm"]), host(dsp["row_scale"])
        bad = np.flatnonzero(np.any(got_c != codes, axis=1))
        assert bad.size == 0, (T, bad[:5], x[bad[0]][:8], got_c[bad[0]][:8], codes[bad[0]][:8])
        assert np.array_equal(got_s, scale)


def test_determinism_bitwise():
    wl = si.small("deepseek_v3")
    inp = si.generate(wl)
    a = run_gpu(wl, inp)
    b = run_gpu(wl, inp)
    for key in a:
        if a[key] is not None:
            assert np.array_equal(a[key], b[key]), key


# ------------------------------------------------------ the one-call layer --

FORWARD_CASES = {
    "mixtral_ragged": lambda: si.small("mixtral", T=1001),
    "switch_capacity": lambda: si.small("switch"),
    "switch_drop_zero": lambda: si.small("switch", T=999, capacity=20, drop="zero"),
    "deepseek_fp8_groups_shared": lambda: si.small("deepseek_v3"),
    "dbrx_skew": lambda: si.small("dbrx"),
    "single_token": lambda: si.small("mixtral", T=1),
    "one_tile_groups_capacity": lambda: si.Workload("otc", **ONE_TILE_CASES["t10_groups_capacity"]),
    "many_tiles_capacity": lambda: si.Workload("mbf", T=20011, d=64, N=16, k=2, F=128,
                                               act="swiglu", dtype="bf16", buf="bf16",
                                               capacity=2300),
}


@pytest.mark.parametrize("name", list(FORWARD_CASES))
def test_forward_matches_oracle_and_phases(name):
    """moe_forward places tokens inside the row copy (from the router's
    per-tile counts); its outputs must pass the oracle checks and equal, bit
    for bit, those of moe_route, moe_dispatch, moe_experts and moe_combine
    called one after the other."""
    from moe_gpu_util import run_gpu_forward
    wl = FORWARD_CASES[name]()
    print(f"case {name}: T={wl.T} d={wl.d} N={wl.N} k={wl.k} cap={wl.capacity}", flush=True)
    inp = si.generate(wl)
    fwd = run_gpu_forward(wl, inp)
    errs = check_layer(wl, inp, fwd, max_adopted=2)
    print(f"  {errs}", flush=True)
    ph = run_gpu(wl, inp)
    R = int(fwd["offsets"][-1])
    for key in ("idx", "w", "counts", "kept_counts", "p", "f", "l_aux", "offsets", "pos", "drop", "y"):
        assert np.array_equal(fwd[key], ph[key]), key
    for key in ("src", "x_perm", "out"):
        assert np.array_equal(fwd[key][:R], ph[key][:R]), key
    if wl.buf == "fp8":
        assert np.array_equal(fwd["row_scale"][:R], ph["row_scale"][:R])


# ------------------------------------------------------------ graph replay --

GRAPH_CASES = {
    "mixtral_ragged": lambda: si.small("mixtral", T=1001),
    "deepseek_fp8_groups_shared": lambda: si.small("deepseek_v3"),
    "one_token_split_paths": lambda: si.small("mixtral", T=1),
}


@pytest.mark.parametrize("name", list(GRAPH_CASES))
def test_graph_replay_matches_eager(name):
    """moe_forward captured in a HIP graph (it allocates, frees and syncs
    nothing) and replayed several times, with other eager work and host
    synchronisation between the replays: every replay's y, routing and plan
    equal the eager call's bit for bit."""
    from moe_gpu_util import upload
    wl = GRAPH_CASES[name]()
    print(f"case {name}: T={wl.T} d={wl.d} N={wl.N} k={wl.k}", flush=True)
    g = upload(wl, si.generate(wl))
    s = M.shape_of(wl)
    L = M.Layer(s, g["wg"], g["w1"], g.get("w3"), g["w2"], bias=g.get("bias"), ws1=g.get("ws1"),
                ws3=g.get("ws3"), ws2=g.get("ws2"))
    x = g["x"]
    L.forward(x)
    torch.cuda.synchronize()
    ref = {k: getattr(L, k).clone() for k in ("y", "idx", "w", "offsets", "pos")}
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        L.forward(x)
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        L.forward(x)
    other = torch.randn(1024, 1024, device="cuda")
    for rep in range(3):
        for key in ("y", "idx", "w", "offsets", "pos"):
            getattr(L, key).zero_()
        graph.replay()
        torch.cuda.synchronize()
        for key, want in ref.items():
            assert torch.equal(getattr(L, key), want), (rep, key)
        other = other @ other.T / 1024.0                 # unrelated eager work between replays
        torch.cuda.synchronize()


# -------------------------------------------------------------- full sizes --

@functools.lru_cache(maxsize=1)
def _deepseek_experts():
    """The DeepSeek-V3-shaped expert weights (22.5 GB), drawn once per session."""
    return si.generate_experts(si.WORKLOADS["deepseek_v3"])


@pytest.mark.parametrize("name", ["mixtral", "switch", "deepseek_v3", "dbrx"])
def test_full_size_parity(name):
    wl = si.WORKLOADS[name]
    if name == "deepseek_v3":
        inp = dict(si.generate(wl, experts=False), **_deepseek_experts())
    else:
        inp = si.generate(wl)
    toks = sample_tokens(wl.T, 40)
    _run_and_check(wl, inp, y_tokens=toks)


@pytest.mark.parametrize("B", [1, 32, 128])
def test_decode_step_deepseek_shape(B):
    """A decode step: B tokens (the prefill batch's first B) through the full
    DeepSeek-V3-shaped layer, so most segments hold one row or none.  Routing,
    plan and fp8 dispatch buffer exact; y on every token at B = 1, on 8
    sampled tokens otherwise; the experts touched are those with a nonzero
    count."""
    wl = si.decode(B)
    inp = dict(si.generate(wl, experts=False), **_deepseek_experts())
    toks = None if B == 1 else sample_tokens(B, 8)
    gpu, _ = _run_and_check(wl, inp, y_tokens=toks)
    touched = int((gpu["counts"] > 0).sum())
    print(f"  experts touched: {touched} of {wl.N}", flush=True)
    assert touched <= min(wl.N, B * wl.k)
