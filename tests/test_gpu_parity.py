"""GPU parity: the HIP path (through the C ABI) against the float64 oracle.

Small cases span several tiles of every kernel with ragged tails; full-size
cases run the workloads at their real shapes through moe_forward (all of
routing, the plan, the dispatch buffer and y on every token compared), with
the single-phase calls bit for bit equal to it."""
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


TIE_CASES = {
    # 64 experts, groups of 8 (two lanes each), k = 8
    "groups_of_8": (lambda: si.small("deepseek_v3", T=300),
                    dict(same_lane=(8, 9), cross_lane=(10, 15), group=(1, 5))),
    # 256 experts, groups of 32 (eight lanes each), k = 8
    "groups_of_32": (lambda: si.small("deepseek_v3", T=200, N=256),
                     dict(same_lane=(32, 33), cross_lane=(37, 60), group=(2, 6))),
    # 128 experts, no groups, k = 2
    "no_groups": (lambda: si.small("switch", T=500, N=128, k=2, capacity=0),
                  dict(same_lane=(4, 5), cross_lane=(3, 70), group=None)),
}


@pytest.mark.parametrize("name", list(TIE_CASES))
def test_exact_ties_go_to_lower_index_many_experts(name):
    """More than 32 experts (one wave per token, four experts per lane):
    duplicated router rows inside one lane's four, across lanes and as whole
    groups give bit-identical logits or group scores, and the lower expert
    (group) must win; all-zero tokens tie every logit and take experts
    0 .. k-1 in order.  The oracle must match without any tie-band adoption."""
    # (the duplicated pairs lie inside one group: the group limit may keep a
    # higher group and drop a lower one)
    make, dup = TIE_CASES[name]
    wl = make()
    inp = si.generate(wl)
    wg = inp["wg"].copy()
    gsz = wl.N // wl.n_groups if wl.n_groups > 1 else wl.N
    if dup["group"] is not None:
        lo, hi = dup["group"]
        wg[hi * gsz:(hi + 1) * gsz] = wg[lo * gsz:(lo + 1) * gsz]
    for lo, hi in (dup["same_lane"], dup["cross_lane"]):
        wg[hi] = wg[lo]
    inp["wg"] = wg
    x = inp["x"].copy()
    zero = [0, 17, wl.T - 1]
    x[zero] = 0
    inp["x"] = x
    print(f"case {name}: T={wl.T} N={wl.N} k={wl.k} groups={wl.n_groups}", flush=True)
    gpu, _ = _forward_and_phases(wl, inp, max_adopted=0)
    for t in zero:
        assert list(gpu["idx"][t]) == list(range(wl.k))
    for lo, hi in (dup["same_lane"], dup["cross_lane"]):
        for t in range(wl.T):
            sel = list(gpu["idx"][t])
            if hi in sel:
                assert lo in sel and sel.index(lo) < sel.index(hi)


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
    # float32 layer (the scatter form runs the down GEMM and the combine as two launches)
    "tiny_f32": lambda: si.WORKLOADS["tiny"],
    # d = 448: the last n-tile holds 192 columns and the last 128-column group of the
    # scatter form's counters 64; capacity drops to the shared fallback expert
    "d448_fallback_shared": lambda: si.Workload("f448", T=600, d=448, N=8, k=2, F=256, capacity=110,
                                                drop="fallback", shared=True),
    "one_tile_groups_capacity": lambda: si.Workload("otc", **ONE_TILE_CASES["t10_groups_capacity"]),
    # one router tile with bf16 x: logits from whole dot products (the four
    # waves split d four or two ways below four tokens, else the tokens), the
    # plan written by the router, the fp8 codes by the logits kernel
    "one_tile_fp8_groups_shared_t1": lambda: si.small("deepseek_v3", T=1),
    "one_tile_fp8_groups_shared_t3": lambda: si.small("deepseek_v3", T=3),
    "one_tile_fp8_capacity_t16": lambda: si.small("deepseek_v3", T=16, capacity=1),
    "one_tile_fp8_fewer_experts_than_tokens": lambda: si.Workload("otf", T=16, d=256, N=8, k=2, F=128,
                                                                  buf="fp8", capacity=3),
    "one_tile_wave_bias_t16": lambda: si.Workload("otw", **ONE_TILE_CASES["t16_wave_bias"]),
    # at most four tokens with bf16 weights: the decode GEMV (no tiles); segments
    # of more than two rows take two passes; U = 1, 2, 4 chunk rounds
    "gemv_t4_relu_capacity": lambda: si.Workload("gv4", T=4, d=256, N=4, k=2, F=256, act="relu", capacity=2),
    "gemv_t4_silu_fp8_shared_full_segments": lambda: si.Workload("gv4s", T=4, d=384, N=2, k=2, F=192,
                                                                 act="silu", buf="fp8", shared=True),
    "gemv_t2_mixtral_dims": lambda: si.Workload("gvm", T=2, d=4096, N=2, k=1, F=14336),
    "many_tiles_capacity": lambda: si.Workload("mbf", T=20011, d=64, N=16, k=2, F=128,
                                               act="swiglu", dtype="bf16", buf="bf16",
                                               capacity=2300),
    # 8-token router tiles: bf16 below 512 tokens (logits from split partials)
    "split_logits_t300": lambda: si.small("mixtral", T=300),
    "split_logits_t511_capacity_fp8": lambda: si.small("mixtral", T=511, N=16, k=4, buf="fp8",
                                                       capacity=100),
    # 8-token router tiles: wide routers (logits from the split-K GEMM), with
    # capacity drops, the fp8 buffer, groups and the shared expert
    "wide_router_fp8_capacity": lambda: si.Workload("wr", T=600, d=8192, N=64, k=4, F=128,
                                                    act="swiglu", dtype="bf16", buf="fp8",
                                                    capacity=40),
    "wide_router_groups_shared": lambda: si.Workload("wrg", T=1003, d=8192, N=64, k=8, F=128,
                                                     act="swiglu", dtype="bf16", buf="fp8",
                                                     n_groups=8, topk_groups=4, shared=True),
}


@pytest.mark.parametrize("name", list(FORWARD_CASES))
def test_forward_matches_oracle_and_phases(name):
    """moe_forward places tokens inside the row copy (from the router's
    per-tile counts); its outputs must pass the oracle checks and equal, bit
    for bit, those of moe_route, moe_dispatch, moe_experts and moe_combine
    called one after the other."""
    wl = FORWARD_CASES[name]()
    print(f"case {name}: T={wl.T} d={wl.d} N={wl.N} k={wl.k} cap={wl.capacity}", flush=True)
    _forward_and_phases(wl, si.generate(wl), max_adopted=2)


def _forward_and_phases(wl, inp, y_tokens=None, max_adopted=None):
    """moe_forward (the measured path: router tiles, per-tile bases and the
    planned copy) against the oracle, then the single-phase calls (standalone
    histogram and plan kernels) bit for bit against it; inputs uploaded once."""
    from moe_gpu_util import assert_same_results, run_gpu_forward, upload
    g = upload(wl, inp)
    fwd = run_gpu_forward(wl, inp, g=g)
    errs = check_layer(wl, inp, fwd, y_tokens=y_tokens, max_adopted=max_adopted)
    print(f"  {errs}", flush=True)
    ph = run_gpu(wl, inp, logits=False, g=g)
    assert_same_results(fwd, ph, wl.buf == "fp8")
    # the fused layer (no dispatch buffer; the up GEMM gathers x through src)
    # gives the same outputs bit for bit
    fu = run_gpu_forward(wl, inp, g=g, fused=True)
    assert fu["x_perm"] is None
    assert_same_results(fu, fwd, wl.buf == "fp8")
    sc = run_gpu_forward(wl, inp, g=g, scatter=True)
    _check_scatter(wl, fwd, sc)
    if wl.T * wl.d <= 1 << 22:
        # (small cases: the scatter layer against the oracle as well)
        check_layer(wl, inp, sc, y_tokens=y_tokens, max_adopted=max_adopted)
    return fwd, errs


def _check_scatter(wl, fwd, sc):
    """moe_forward_scatter (the down GEMM's tiles write y): routing and plan bit
    for bit those of moe_forward, its y bit for bit what moe_combine makes of its
    own expert outputs, and those outputs the ones moe_forward computes (up to
    float32 rounding order where moe_forward's down GEMM splits its last tiles
    along K: the combining GEMM runs them whole)."""
    from oracle import compare
    for key in ("idx", "w", "counts", "kept_counts", "p", "f", "l_aux", "offsets", "pos", "drop"):
        assert np.array_equal(sc[key], fwd[key]), key
    R = int(fwd["offsets"][-1])
    assert np.array_equal(sc["src"][:R], fwd["src"][:R]), "src"
    assert np.array_equal(sc["y"], sc["y_combine"]), "scatter y vs moe_combine on the same outputs"
    if R > 0:
        e = compare.rel_l2(sc["out"][:R], fwd["out"][:R])
        assert e <= 2e-3, f"scatter out vs moe_forward out: {e}"
    if fwd["out_shared"] is not None:
        e = compare.rel_l2(sc["out_shared"], fwd["out_shared"])
        assert e <= 2e-3, f"scatter out_shared vs moe_forward: {e}"
    e = compare.rel_l2(sc["y"], fwd["y"])
    assert e <= 2e-3, f"scatter y vs moe_forward y: {e}"
    print(f"  scatter: y == combine(out) bit for bit; y vs moe_forward rel-L2 {e:.2e}", flush=True)


# ------------------------------------------------------------ graph replay --

GRAPH_CASES = {
    "mixtral_ragged": lambda: si.small("mixtral", T=1001),
    "deepseek_fp8_groups_shared": lambda: si.small("deepseek_v3"),
    "one_token_split_paths": lambda: si.small("mixtral", T=1),
    "deepseek_v3_full": lambda: si.WORKLOADS["deepseek_v3"],
    # the fused layer (no dispatch buffer)
    "mixtral_ragged_fused": lambda: si.small("mixtral", T=1001),
    "deepseek_v3_full_fused": lambda: si.WORKLOADS["deepseek_v3"],
    # decode steps of the fused layer: the one-tile router and the decode GEMV
    "decode_1_token_fused": lambda: si.decode(1),
    "decode_4_tokens_fused": lambda: si.decode(4),
    # the scatter layer (the down GEMM's tiles write y; its counters are set by a kernel, not a memset)
    "switch_capacity_scatter": lambda: si.small("switch"),
    "deepseek_fp8_groups_shared_scatter": lambda: si.small("deepseek_v3"),
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
    g = upload(wl, _inputs(wl))
    s = M.shape_of(wl)
    L = M.Layer(s, g["wg"], g["w1"], g.get("w3"), g["w2"], bias=g.get("bias"), ws1=g.get("ws1"),
                ws3=g.get("ws3"), ws2=g.get("ws2"), fused=name.endswith(("_fused", "_scatter")),
                scatter=name.endswith("_scatter"))
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


def _inputs(wl):
    """Seeded inputs; the DeepSeek-V3-shaped expert weights come from the
    session's one draw."""
    if wl.N == 256 and wl.d == 7168 and wl.F == 2048:
        return dict(si.generate(wl, experts=False), **_deepseek_experts())
    return si.generate(wl)


@pytest.mark.parametrize("name", ["mixtral", "switch", "deepseek_v3", "dbrx"])
def test_full_size_parity(name):
    """Every workload at its full size through moe_forward, the path that is
    benchmarked: routing, statistics, plan and dispatch buffer exact, the
    expert outputs and y of every token against the float64 oracle (each row
    on its own and the whole tensor), and the single-phase calls bit for bit
    equal to it.  The DeepSeek-V3 shape also reports y against the same layer
    without the fp8 dispatch step."""
    wl = si.WORKLOADS[name]
    print(f"case {name}: T={wl.T} d={wl.d} N={wl.N} k={wl.k} F={wl.F}", flush=True)
    gpu, errs = _forward_and_phases(wl, _inputs(wl))
    if name == "switch":
        print(f"  drops: {int(gpu['drop'].sum())}, experts over capacity: "
              f"{int((gpu['counts'] > wl.capacity).sum())}", flush=True)
        assert gpu["drop"].sum() > 0
    if wl.buf == "fp8":
        print(f"  y vs fp8-defined oracle {errs['y']:.4e}, vs oracle without fp8 step "
              f"{errs['y_vs_no_fp8']:.4e}", flush=True)
        assert errs["y_vs_no_fp8"] <= 2e-2


@pytest.mark.parametrize("B", [1, 32, 128])
def test_decode_step_deepseek_shape(B):
    """A decode step: B tokens (the prefill batch's first B) through the full
    DeepSeek-V3-shaped layer, so most segments hold one row or none.  Through
    moe_forward (few-token router split, split-K GEMMs) against the oracle on
    every token, and the single-phase calls bit for bit equal to it; the
    experts touched are those with a nonzero count."""
    wl = si.decode(B)
    print(f"case decode B={B}", flush=True)
    gpu, _ = _forward_and_phases(wl, _inputs(wl))
    touched = int((gpu["counts"] > 0).sum())
    print(f"  experts touched: {touched} of {wl.N}", flush=True)
    assert touched <= min(wl.N, B * wl.k)


# ------------------------------------------------------- fused dispatch phases --

FUSED_PHASE_CASES = {
    "mixtral_small": lambda: si.small("mixtral"),
    "switch_capacity_128_row_tiles": lambda: si.small("switch"),
    "deepseek_fp8_groups": lambda: si.small("deepseek_v3"),
    "f32_tiny": lambda: si.WORKLOADS["tiny"],
    "one_token": lambda: si.small("mixtral", T=1),
}


@pytest.mark.parametrize("name", list(FUSED_PHASE_CASES))
def test_fused_phases_equal_dispatch_buffer_phases(name):
    """moe_route_plan + moe_expert_up_gather against moe_route_dispatch +
    moe_expert_up: the same plan, the token-order fp8 codes equal the
    dispatch buffer's rows, and h is bit for bit the same."""
    from moe_gpu_util import upload
    wl = FUSED_PHASE_CASES[name]()
    print(f"case {name}: T={wl.T} d={wl.d} N={wl.N} k={wl.k}", flush=True)
    s = M.shape_of(wl)
    g = upload(wl, si.generate(wl))
    ws = M.alloc_workspace(s)
    ref = M.route_dispatch(s, g["x"], g["wg"], g.get("bias"), ws=ws)
    h_ref = M.expert_up(s, ref["x_perm"], ref["row_scale"], ref["offsets"], g["w1"], g.get("w3"), ws=ws)
    torch.cuda.synchronize()
    ws2 = M.alloc_workspace(s)
    got = M.route_plan(s, g["x"], g["wg"], g.get("bias"), ws=ws2)
    a = got["x_codes"] if wl.buf == "fp8" else g["x"]
    h = M.expert_up_gather(s, a, got["row_scale"], got["offsets"], got["src"], g["w1"], g.get("w3"), ws=ws2)
    torch.cuda.synchronize()
    R = int(ref["offsets"][-1].item())
    for key in ("idx", "w", "counts", "kept_counts", "p", "f", "l_aux", "offsets", "pos", "drop"):
        assert torch.equal(got[key], ref[key]), key
    assert torch.equal(got["src"][:R], ref["src"][:R])
    if wl.buf == "fp8":
        assert torch.equal(got["row_scale"][:R], ref["row_scale"][:R])
        assert torch.equal(got["x_codes"][got["src"][:R].long()], ref["x_perm"][:R])
    assert torch.equal(h[:R], h_ref[:R])


# ---------------------------------------------------------- MXFP4 expert weights --
# The OCP microscaling format the gpt-oss experts use ("MoE: what it costs to
# train and serve" / "Memory: sparsity only helps once it fits"): the layer
# through moe_forward against the oracle, which decodes every weight exactly,
# and the single-phase calls and the fused layer bit for bit equal to it.

MX_CASES = {
    # ReLU, bf16 activations, capacity drops, 128-row tiles and their split-K tail
    "switch_small": lambda: si.small("switch", wfmt="mxfp4"),
    # SwiGLU with bf16 activations
    "mixtral_small": lambda: si.small("mixtral", wfmt="mxfp4"),
    # bf16 activations with enough tiles for whole-tile launches: the codes on the
    # LDS-DMA pipeline, widened as fragments are read (K = 512 and 768)
    "mixtral_whole_tiles": lambda: si.small("mixtral", T=3000, wfmt="mxfp4"),
    # fp8 activations (gate/up on the scaled fp8 x FP4 MFMA), groups, MXFP4 shared expert
    "deepseek_small": lambda: si.small("deepseek_v3", wfmt="mxfp4", shared=True),
    # fp8 activations with d not a multiple of 128: the gate/up widens the weights to bf16
    "deepseek_d448": lambda: si.small("deepseek_v3", d=448, wfmt="mxfp4"),
    # one token: every GEMM split along K
    "one_token": lambda: si.small("deepseek_v3", T=1, wfmt="mxfp4", shared=True),
    "switch_full": lambda: si.WORKLOADS["switch"].replace(name="switch_mxfp4", wfmt="mxfp4"),
    "deepseek_v3_full": lambda: si.WORKLOADS["deepseek_v3"].replace(name="deepseek_v3_mxfp4", wfmt="mxfp4"),
}


@pytest.mark.parametrize("name", list(MX_CASES))
def test_mxfp4_layer(name):
    wl = MX_CASES[name]()
    print(f"case {name}: T={wl.T} d={wl.d} N={wl.N} k={wl.k} F={wl.F}", flush=True)
    _forward_and_phases(wl, si.generate(wl))


# ------------------------------------------------- the combining down GEMM --

DOWN_COMBINE_CASES = {
    # 256-row down tiles with their quarter-tile tail, capacity drops contributing zero
    "mixtral_capacity_zero": lambda: si.small("mixtral", T=1500, capacity=300, drop="zero"),
    # fp8 rows, groups, the shared expert as the extra segment of the same launch
    "deepseek_fp8_shared": lambda: si.small("deepseek_v3"),
    # capacity drops passed through (ReLU, 128-row tiles)
    "switch_passthrough": lambda: si.small("switch"),
}


@pytest.mark.parametrize("name", list(DOWN_COMBINE_CASES))
def test_expert_down_combine_equals_down_then_combine(name):
    """moe_expert_down_combine called on its own: out (and out_shared) bit for
    bit those of moe_expert_down (moe_expert_down_shared) without a workspace,
    and y bit for bit moe_combine of them, on twice-called inputs (the counters
    need no initialisation between calls)."""
    from moe_gpu_util import upload
    wl = DOWN_COMBINE_CASES[name]()
    print(f"case {name}: T={wl.T} d={wl.d} N={wl.N} k={wl.k} cap={wl.capacity}", flush=True)
    s = M.shape_of(wl)
    g = upload(wl, si.generate(wl))
    x = g["x"]
    ws = M.alloc_workspace(s)
    pl = M.route_plan(s, x, g["wg"], g.get("bias"), ws=ws)
    a = pl["x_codes"] if wl.buf == "fp8" else x
    h = M.expert_up_gather(s, a, pl["row_scale"], pl["offsets"], pl["src"], g["w1"], g.get("w3"), ws=ws)
    hs = M.shared_expert_up(s, x, g["ws1"], g.get("ws3")) if wl.shared else None
    if wl.shared:
        out_ref, outs_ref = M.expert_down_shared(s, h, pl["offsets"], g["w2"], hs, g["ws2"])
    else:
        out_ref, outs_ref = M.expert_down(s, h, pl["offsets"], g["w2"]), None
    y_ref = M.combine(s, out_ref, outs_ref, x, pl["pos"], pl["w"])
    torch.cuda.synchronize()
    R = int(pl["offsets"][-1].item())
    for rep in range(2):
        out, outs, y = M.expert_down_combine(s, h, pl["offsets"], pl["src"], g["w2"], x, pl["pos"], pl["w"],
                                             h_shared=hs, ws2=g.get("ws2"), ws=ws)
        torch.cuda.synchronize()
        assert torch.equal(out[:R], out_ref[:R]), (rep, "out")
        if wl.shared:
            assert torch.equal(outs, outs_ref), (rep, "out_shared")
        assert torch.equal(y, y_ref), (rep, "y")
