"""Benchmark of the sparse MoE-layer forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload mixtral]
                    [--no-cpu-baseline] [--mode bench|copy|sweep|decode|memory|summarize]

One step = one whole layer forward (route, dispatch, grouped GEMM up, grouped
GEMM down, shared expert if any, combine) over one batch of seeded synthetic
inputs already resident in HBM.  The timed region is bracketed by
torch.cuda.synchronize() on both sides; inside it, HIP events on the launch
stream separate the phases, so each kernel's average duration is measured on
the same launches that are timed.

Prints one JSON line: tokens/s (whole job), ms per step, per-phase times, the
dominant kernel's roofline (grouped GEMM up: algorithmic FLOPs per launch /
its measured duration, against the bf16 dense MFMA peak), the dispatch and
memory-phase bandwidths, and the float64 CPU oracle timed on a bounded sample.

--mode copy runs a plain device copy of a known size (the calibration kernel
for the hardware byte counters) and exits.  --mode sweep times every workload
family at full size, phase by phase, and prints a markdown table.  --mode
decode times decode steps (B = 1, 32, 128 tokens) at the DeepSeek-V3 shape:
experts touched and the expert-weight bytes streamed against the HBM peak.
--mode memory times the memory-bound phases alone, warm and with the caches
flushed before every launch (median and p10/p90).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s at Mixtral shape; grouped-GEMM % MFMA peak; dispatch GB/s"
# the gate/up grouped-GEMM kernel instance each workload runs (key in the counter summary)
# the gate/up kernel's name in the counter summary (template arguments as the trace prints them)
UP_KERNEL = {"mixtral": "gg_kernel<256,256,2,4,3,false,false,false,false,false,false>"}
PEAK_BF16_TFLOPS = 2516.6      # 256 CU x 2.4 GHz x 4096 dense bf16 FLOP/clk/CU
PEAK_HBM_GBPS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="mixtral",
                    help="mixtral, switch, deepseek_v3, dbrx, tiny; append _mxfp4 for MXFP4 expert weights")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--unfused", action="store_true",
                    help="time the layer with the dispatch buffer (row copy, then the up GEMM on it) "
                         "instead of the fused gather")
    ap.add_argument("--scatter", action="store_true",
                    help="time the fused layer whose down GEMM also writes y (moe_forward_scatter: "
                         "no combine launch)")
    ap.add_argument("--cpu-sample-tokens", type=int, default=0,
                    help="tokens whose expert FFNs the CPU oracle runs (0: all T)")
    ap.add_argument("--mode", choices=["bench", "copy", "summarize", "sweep", "decode", "memory"],
                    default="bench")
    ap.add_argument("--prof", default=None,
                    help="summarize: directory holding trace/ fetch/ write/ cfetch/ cwrite/ "
                         "rocprofv3 csv output")
    ap.add_argument("--out", default=None, help="summarize: markdown file to write")
    return ap.parse_args()


def workload(name):
    """A named workload; the suffix ``_mxfp4`` gives the same layer with MXFP4
    expert weights."""
    import synthetic_inputs as si
    if name.endswith("_mxfp4"):
        return si.WORKLOADS[name[:-len("_mxfp4")]].replace(name=name, wfmt="mxfp4")
    return si.WORKLOADS[name]


def alg_bytes(wl, R, fused=False):
    """Algorithmic (minimum) HBM bytes of the memory phases; R kept rows.
    Fused (no dispatch buffer): the dispatch phase is the plan alone (idx read,
    pos, drop and src written), plus for an fp8 buffer the one quantising pass
    over x (codes in token order, one scale per kept row)."""
    sx = 2 if wl.dtype == "bf16" else 4
    sb = 1 if wl.buf == "fp8" else sx
    T, d, N, k = wl.T, wl.d, wl.N, wl.k
    route = T * d * sx + N * d * sx + 8 * T * k + 4 * N
    if fused:
        dispatch = 9 * T * k + 4 * R + ((T * d * sx + T * d + 4 * R) if wl.buf == "fp8" else 0)
    else:
        dispatch = T * d * sx + R * d * sb + (4 * R if wl.buf == "fp8" else 0) + 8 * T * k + 4 * R
    combine = R * d * sx + T * d * sx + (T * d * sx if wl.shared else 0) + 8 * T * k
    return route, dispatch, combine


def layer_step(wl, L, x, h, hs):
    """One layer forward phase by phase, the kernels of moe_forward (fused or
    not, as the layer was made), with HIP events recorded between the phases
    when given: ev[0] before, ev[1] after route + dispatch (or route + plan),
    ev[2] after the up GEMM (in the fused layer with a shared expert, both up
    GEMMs in one call), ev[3] after the unfused layer's shared-expert up GEMM
    (otherwise nothing runs between ev[2] and ev[3]), ev[4] after the down GEMM
    (with a shared expert, its down GEMM in the same launch), ev[5] after the
    combine."""
    from mixture_experts_layer_sparse_amd import moe as M
    s = L.s

    def step(ev=None):
        ev and ev[0].record()
        if L.fused:
            L.route_plan(x)
            ev and ev[1].record()
            if wl.shared:
                # (routed and shared up in one call; a decode-sized call makes it one launch)
                L.expert_up_gather_shared(x, h, hs)
            else:
                L.expert_up_gather(x, h)
        else:
            L.route_dispatch(x)
            ev and ev[1].record()
            M.expert_up(s, L.x_perm, L.row_scale, L.offsets, L.w1, L.w3, h, ws=L.ws)
        ev and ev[2].record()
        if wl.shared and not L.fused:
            M.shared_expert_up(s, x, L.ws1, L.ws3, hs, ws=L.ws)
        ev and ev[3].record()
        if L.scatter:
            # the down GEMM's tiles write y (no combine launch: nothing runs between ev[4] and ev[5])
            L.expert_down_combine(x, h, hs)
            ev and ev[4].record()
            ev and ev[5].record()
            return
        if wl.shared:
            M.expert_down_shared(s, h, L.offsets, L.w2, hs, L.ws2, L.out, L.out_shared, ws=L.ws)
        else:
            M.expert_down(s, h, L.offsets, L.w2, L.out, ws=L.ws)
        ev and ev[4].record()
        L.combine(x)
        ev and ev[5].record()
    return step


def gemm_flops(wl, R):
    m = 2 if wl.act == "swiglu" else 1
    up = 2 * R * wl.d * wl.F * m
    down = 2 * R * wl.F * wl.d
    shared = (2 * wl.T * wl.d * wl.F * (m + 1)) if wl.shared else 0
    return up, down, shared


def cpu_baseline(wl, inp, n_tok):
    """The float64 oracle as it stands, on a bounded sample: routing, statistics
    and the dispatch plan for all T tokens, the expert FFNs and combine for
    ``n_tok`` sampled tokens.  Returns a tokens/s figure for the whole layer:
    1 / (routing time per token + FFN time per sampled token)."""
    import numpy as np
    from threadpoolctl import threadpool_info
    from oracle import moe as om
    toks = np.linspace(0, wl.T - 1, min(n_tok, wl.T)).astype(np.int64)
    t0 = time.perf_counter()
    om.forward(wl, {**inp, "w1": None})
    t_route = time.perf_counter() - t0
    t0 = time.perf_counter()
    om.forward(wl, inp, ffn_tokens=toks)
    t_all = time.perf_counter() - t0
    t_ffn = max(t_all - t_route, 1e-9)
    per_tok = t_route / wl.T + t_ffn / n_tok
    pools = threadpool_info()
    threads = max([p.get("num_threads", 1) for p in pools] or [1])
    # what np.show_runtime() prints, in one line: the BLAS library, its
    # threading layer and thread count
    blas = "; ".join(f"{p.get('internal_api')} {p.get('version')} ({p.get('threading_layer')}, "
                     f"{p.get('num_threads')} threads)" for p in pools)
    return {"value": 1.0 / per_tok, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "host_cpus": os.cpu_count(), "numpy": np.__version__, "blas": blas,
            "sample": f"routing + plan for all {wl.T} tokens ({t_route:.2f} s); expert FFNs + "
                      f"combine for {n_tok} evenly spaced tokens ({t_ffn:.2f} s); float64 NumPy"}


COUNTER_FILE = os.path.join(ROOT, "profiles", "grouped_gemm_mixtral_counters.md")
GEMM_SRC = os.path.join(ROOT, "mixture_experts_layer_sparse_amd", "csrc", "gemm.hip")
# counter passes of the summary (each pass its own rocprofv3 run): name, counters
COUNTER_PASSES = [
    ("fetch", "FETCH_SIZE"),
    ("write", "WRITE_SIZE"),
    ("mfma", "MfmaUtil SQ_INSTS_VALU_MFMA_MOPS_BF16 GRBM_GUI_ACTIVE"),
    ("lds", "SQ_LDS_BANK_CONFLICT SQ_LDS_IDX_ACTIVE"),
    ("occ", "OccupancyPercent"),
]
PROFILE_CMDS = [
    "rocprofv3 --kernel-trace --stats --output-format csv -d <dir>/trace -o run -- "
    "python3 bench.py --no-cpu-baseline",
    *[f"rocprofv3 --pmc {c} --output-format csv -d <dir>/{n} -o run -- "
      "python3 bench.py --no-cpu-baseline --steps 3 --warmup 1" for n, c in COUNTER_PASSES],
    "rocprofv3 --pmc FETCH_SIZE --output-format csv -d <dir>/cfetch -o run -- python3 bench.py --mode copy",
    "rocprofv3 --pmc WRITE_SIZE --output-format csv -d <dir>/cwrite -o run -- python3 bench.py --mode copy",
]


def _src_hash(path):
    import hashlib
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def _short(name):
    for key in ("gg_splitk_reduce", "gg_kernel", "logits_split_kernel", "route_kernel", "route_stats_tiles_kernel",
                "route_stats_kernel",
                "disp_hist_kernel", "disp_plan_tiles_kernel", "disp_plan_kernel", "disp_copy_kernel",
                "disp_fp8_kernel", "combine_bf16_kernel", "combine_f32_kernel", "__amd_rocclr_copyBuffer"):
        if key in name:
            i = name.find(key)
            j = name.find("(", i)
            return name[i:j if j > 0 else None].replace(" ", "")
    return None


def summarize(prof, out, steps, warmup):
    """Markdown summary of a rocprofv3 session of this benchmark: per kernel,
    the average duration over the timed steps only (dispatches warmup ..
    warmup + steps - 1 of that kernel, in start order: the bench launches each
    kernel once per step, and its warm-up, check and graph-replay calls come
    before or after), its registers and LDS from the trace, the L2-miss bytes
    per dispatch from FETCH_SIZE / WRITE_SIZE scaled by what the same counters
    read for a plain copy of known size, MFMA busy share, LDS bank-conflict
    cycles and occupancy."""
    import csv
    from collections import defaultdict

    def rows_of(sub, fname):
        path = os.path.join(prof, sub, fname)
        if not os.path.exists(path):
            return []
        with open(path) as f:
            return list(csv.DictReader(f))

    def counters(sub, name):
        agg = defaultdict(list)
        for r in rows_of(sub, "run_counter_collection.csv"):
            if r["Counter_Name"] == name:
                k = _short(r["Kernel_Name"])
                if k:
                    agg[k].append(float(r["Counter_Value"]))
        return {k: sum(v) / len(v) for k, v in agg.items()}

    calls = defaultdict(list)
    for r in rows_of("trace", "run_kernel_trace.csv"):
        k = _short(r["Kernel_Name"])
        if k:
            calls[k].append(r)
    kern = {}
    for k, rs in calls.items():
        rs.sort(key=lambda r: int(r["Start_Timestamp"]))
        dur = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in rs]
        timed = dur[warmup:warmup + steps] if len(dur) >= warmup + steps else dur
        r0 = rs[0]
        regs = (f"{r0.get('Arch_VGPR_Count', r0.get('VGPR_Count', '?'))}+{r0.get('Accum_VGPR_Count', '?')} / "
                f"{r0.get('SGPR_Count', '?')} / {int(r0.get('LDS_Block_Size', 0) or 0) // 1024} / "
                f"{r0.get('Scratch_Size', '?')}")
        kern[k] = {"calls": len(dur), "timed_us": sum(timed) / len(timed), "all_us": sum(dur) / len(dur),
                   "regs": regs, "wg": r0.get("Workgroup_Size_X", "?"), "grid": r0.get("Grid_Size_X", "?")}
    fetch, write = counters("fetch", "FETCH_SIZE"), counters("write", "WRITE_SIZE")
    cf = counters("cfetch", "FETCH_SIZE")["__amd_rocclr_copyBuffer"]
    cw = counters("cwrite", "WRITE_SIZE")["__amd_rocclr_copyBuffer"]
    mfma, mops = counters("mfma", "MfmaUtil"), counters("mfma", "SQ_INSTS_VALU_MFMA_MOPS_BF16")
    gui = counters("mfma", "GRBM_GUI_ACTIVE")
    bankc, ldsact = counters("lds", "SQ_LDS_BANK_CONFLICT"), counters("lds", "SQ_LDS_IDX_ACTIVE")
    occ = counters("occ", "OccupancyPercent")
    copy_kib = (1 << 28) / 1024
    f_scale, w_scale = copy_kib / cf, copy_kib / cw
    # GRBM_GUI_ACTIVE is summed over the XCDs
    n_xcc = 8
    for r in rows_of("trace", "run_agent_info.csv"):
        if r.get("Agent_Type", "").endswith("GPU") and r.get("Num_Xcc"):
            n_xcc = int(r["Num_Xcc"])
    rows, table, table2 = {}, [], []
    for k, v in sorted(kern.items(), key=lambda kv: -kv[1]["timed_us"]):
        if k.startswith("__amd"):
            continue
        fb = fetch.get(k, 0.0) * 1024 * f_scale
        wb = write.get(k, 0.0) * 1024 * w_scale
        rows[k] = {"avg_us": v["timed_us"], "avg_us_all_calls": v["all_us"], "fetch_bytes": fb,
                   "write_bytes": wb}
        table.append(f"| `{k}` | {v['calls']} | {v['timed_us']:.1f} | {v['all_us']:.1f} | {fb / 2**20:.1f} | "
                     f"{wb / 2**20:.1f} |")
        # the shader clock under the profiler: active GPU cycles over the dispatch's duration
        # (only for dispatches long enough that the profiler's own active
        # cycles around them do not count)
        clk = gui.get(k, 0.0) / n_xcc / (v["all_us"] * 1e3) if k in gui and v["all_us"] > 200 else 0.0
        clk_s = f"{clk:.2f}" if clk else "-"
        bf16_tflop = mops.get(k, 0.0) * 512 / 1e12
        table2.append(f"| `{k}` | {v['regs']} | {v['wg']} x {int(v['grid']) // max(int(v['wg']), 1) if str(v['grid']).isdigit() else '?'} | "
                      f"{mfma.get(k, 0.0):.1f} | {bf16_tflop:.3f} | {bankc.get(k, 0.0):.3g} | "
                      f"{ldsact.get(k, 0.0):.3g} | {occ.get(k, 0.0):.1f} | {clk_s} |")
    data = {"gemm_src_sha256_16": _src_hash(GEMM_SRC), "fetch_scale": f_scale,
            "write_scale": w_scale, "timed_steps": [warmup, steps], "kernels": rows}
    text = "\n".join([
        "# Kernels of one layer forward, Mixtral-shaped layer (T=4096, d=4096, N=8, k=2, F=14336, bf16)",
        "",
        "rocprofv3 on one MI355X; commands (run from the repository root, `<dir>` a scratch directory):",
        "",
        *[f"    {c}" for c in PROFILE_CMDS],
        "",
        f"Summarised with `python3 bench.py --mode summarize --prof <dir> --out <this file>`. Durations are "
        f"averaged over the timed steps only (each kernel's dispatches {warmup} to {warmup + steps - 1} in start "
        f"order); the average over all dispatches (warm-up, the check call and the graph replays included) "
        f"is beside it.",
        "",
        f"L2-miss bytes: FETCH_SIZE x {f_scale:.3f}, WRITE_SIZE x {w_scale:.3f} (the factors that make a plain "
        f"256 MiB copy read and write 256 MiB). These count every L2 miss, whether the Infinity Cache or HBM "
        f"serves it.",
        "",
        "| kernel | dispatches | avg us (timed) | avg us (all) | L2-miss read MiB/dispatch | "
        "L2-miss write MiB/dispatch |",
        "|---|---|---|---|---|---|",
        *table,
        "",
        "Registers as the trace reports them (its VGPR field + accumulation VGPRs / SGPRs; the code object of the gate/up kernel allocates 238 VGPRs), LDS KiB and scratch bytes per lane from the kernel "
        "trace; workgroup size x workgroups; MfmaUtil = MFMA-busy cycles / (active cycles x SIMDs), %; bf16 "
        "MFMA TFLOP per dispatch from SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512; LDS bank-conflict and LDS-active "
        "cycles (summed over the SEs); OccupancyPercent; clock = GRBM_GUI_ACTIVE cycles per dispatch and XCD "
        "over the dispatch's average duration in the trace run, GHz, for dispatches over 200 us (the counter "
        "runs are short, so they run at a higher clock than the long trace run).",
        "",
        "| kernel | VGPR / SGPR / LDS / scratch | launch | MfmaUtil % | bf16 MFMA TFLOP | LDS bank-conflict "
        "cycles | LDS active cycles | occupancy % | clock GHz |",
        "|---|---|---|---|---|---|---|---|---|",
        *table2,
        "",
        "Machine-readable (bench.py reads this to fill `roofline.traffic` while `gemm.hip` is unchanged):",
        "",
        "```json",
        json.dumps(data),
        "```",
        "",
    ])
    with open(out, "w") as f:
        f.write(text)
    print(text)


def profiled_traffic(kernel_key):
    """HBM bytes per launch of a kernel from the committed counter summary, or
    None when there is none or gemm.hip has changed since it was taken."""
    try:
        with open(COUNTER_FILE) as f:
            text = f.read()
        blob = text.split("```json", 1)[1].split("```", 1)[0]
        data = json.loads(blob)
        if data.get("gemm_src_sha256_16") != _src_hash(GEMM_SRC):
            return None
        k = data["kernels"].get(kernel_key)
        return None if k is None else k["fetch_bytes"] + k["write_bytes"]
    except (OSError, IndexError, ValueError, KeyError):
        return None


def expert_weight_bytes(wl):
    """Bytes of the expert weights one layer reads (routed + shared); MXFP4
    matrices are their codes plus block scales (4.25 bits per weight)."""
    m = 3 if wl.act == "swiglu" else 2
    n = wl.N + (1 if wl.shared else 0)
    if getattr(wl, "wfmt", "bf16") == "mxfp4":
        return n * m * (wl.F * wl.d // 2 + wl.F * wl.d // 32)
    s = 2 if wl.dtype == "bf16" else 4
    return n * m * wl.F * wl.d * s


def graph_step_time(step, steps, warmup):
    """Seconds per step when one step (a function that launches the layer's
    kernels on the current stream, allocating nothing) is captured once in a
    HIP graph and replayed: the kernels without host launch gaps."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for _ in range(warmup):
        graph.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        graph.replay()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) / steps


def _to_dev(arr):
    import numpy as np
    import torch
    if arr is None:
        return None
    if arr.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(arr)).cuda()


def shared_up_runs(wl, fused):
    """Whether layer_step launches anything between ev[2] and ev[3] (the
    unfused layer's shared-expert up GEMM); otherwise that interval holds only
    the two event records and counts as no GEMM time."""
    return bool(wl.shared) and not fused


def _phases(wl, g, x, steps, warmup, fused=True, scatter=False):
    """Runs the kernels of moe_forward phase by phase; returns (layer, mean
    phase times in us [route+dispatch, up, shared up, down (+ shared down), combine], wall time
    per step in s)."""
    import numpy as np
    import torch
    from mixture_experts_layer_sparse_amd import moe as M
    s = M.shape_of(wl)
    L = M.Layer(s, g["wg"], g["w1"], g["w3"], g["w2"], bias=g["bias"], ws1=g["ws1"],
                ws3=g["ws3"], ws2=g["ws2"], fused=fused, scatter=scatter)
    h = torch.empty((wl.T * wl.k, wl.F), dtype=s.torch_dtype, device="cuda")
    hs = torch.empty((wl.T, wl.F), dtype=s.torch_dtype, device="cuda") if wl.shared else None
    step = layer_step(wl, L, x, h, hs)

    E = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(steps + warmup)]
    for i in range(warmup):
        step(E[i])
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(warmup, warmup + steps):
        step(E[i])
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / steps
    ph = np.array([[e[j].elapsed_time(e[j + 1]) for j in range(5)] for e in E[warmup:]]).mean(0) * 1e3
    return L, ph, wall


def load_report(wl, L):
    """The layer's load statistics as the library returned them (no oracle):
    per-expert counts before drops, drops, f, p and L_aux.  Returns a dict."""
    import numpy as np
    counts = L.counts.cpu().numpy()
    kept = L.kept_counts.cpu().numpy()
    f = L.f.cpu().numpy()
    p = L.p.cpu().numpy()
    mean = wl.T * wl.k / wl.N
    rep = {"workload": wl.name, "l_aux": float(L.l_aux.item()), "alpha": wl.alpha,
           "counts_min": int(counts.min()), "counts_max": int(counts.max()),
           "hot_over_mean": float(counts.max() / mean), "dropped": int(counts.sum() - kept.sum()),
           "experts_over_capacity": int((counts > wl.capacity).sum()) if wl.capacity > 0 else 0,
           "f_sum": float(f.sum()), "f_max": float(f.max()), "p_sum": float(p.sum()),
           "p_min": float(p.min()), "p_max": float(p.max())}
    if wl.N <= 16:
        rep["counts"] = counts.tolist()
        rep["f"] = [round(float(v), 5) for v in f]
        rep["p"] = [round(float(v), 5) for v in p]
    return rep


def sweep(steps, warmup):
    """Every workload family at its full size, phase by phase (the kernels of
    moe_forward); prints a markdown table, then each workload's load
    statistics (counts histogram, drops, f, p, L_aux) as the library returned
    them."""
    import torch
    import synthetic_inputs as si
    reports = []

    print("| workload | tokens/s | ms/step | route+dispatch us | GEMM up (+ shared) us | shared up (unfused) us | GEMM down (+ shared) us | "
          "combine us | GEMM TFLOP/s (% bf16 peak) | GEMM weight GB/s (% HBM) | memory phases GB/s (% HBM) |")
    print("|---|---|---|---|---|---|---|---|---|---|---|")
    for name in ("tiny", "mixtral", "switch", "deepseek_v3", "dbrx", "switch_mxfp4", "deepseek_v3_mxfp4",
                 "mixtral_scatter", "switch_scatter", "deepseek_v3_scatter", "dbrx_scatter"):
        # (_scatter: moe_forward_scatter, the down GEMM's tiles writing y; no combine launch)
        scatter = name.endswith("_scatter")
        wl = workload(name[:-len("_scatter")] if scatter else name)
        inp = si.generate(wl)
        g = {k: _to_dev(v) for k, v in inp.items()}
        del inp
        x = g["x"]
        L, ph, wall = _phases(wl, g, x, steps, warmup, scatter=scatter)
        R = int(L.offsets[-1].item())
        up, down, shared = gemm_flops(wl, R)
        rb, db, cb = alg_bytes(wl, R, fused=True)
        if scatter:
            ph[4], cb = 0.0, 0                    # (the combine runs in the down GEMM)
        sh = shared_up_runs(wl, True)
        gemm_us = ph[1] + (ph[2] if sh else 0.0) + ph[3]
        tf = (up + down + shared) / (gemm_us * 1e-6) / 1e12
        wgb = expert_weight_bytes(wl) / (gemm_us * 1e-6) / 1e9
        mem_us = ph[0] + ph[4]
        mgb = (rb + db + cb) / (mem_us * 1e-6) / 1e9
        extra = ", MXFP4 experts" if wl.wfmt == "mxfp4" else (", combine in the down GEMM" if scatter else "")
        print(f"| {name} (T={wl.T}, d={wl.d}, N={wl.N}, k={wl.k}, F={wl.F}{extra}) | {wl.T / wall:,.0f} | "
              f"{wall * 1e3:.3f} | {ph[0]:.1f} | {ph[1]:.1f} | {f'{ph[2]:.1f}' if sh else '-'} | {ph[3]:.1f} | "
              f"{'-' if scatter else f'{ph[4]:.1f}'} | "
              f"{tf:.0f} ({100 * tf / PEAK_BF16_TFLOPS:.1f}%) | {wgb:.0f} ({100 * wgb / PEAK_HBM_GBPS:.1f}%) | "
              f"{mgb:.0f} ({100 * mgb / PEAK_HBM_GBPS:.1f}%) |", flush=True)
        if not scatter:
            reports.append(load_report(wl, L))
        del L, g, x
        torch.cuda.empty_cache()
    print()
    print("| workload | L_aux (alpha) | counts min / max (hot / mean) | dropped (experts over C) | "
          "sum f, max f | sum p, min p, max p |")
    print("|---|---|---|---|---|---|")
    for r in reports:
        print(f"| {r['workload']} | {r['l_aux']:.5f} ({r['alpha']}) | {r['counts_min']} / {r['counts_max']} "
              f"({r['hot_over_mean']:.2f}) | {r['dropped']} ({r['experts_over_capacity']}) | "
              f"{r['f_sum']:.6f}, {r['f_max']:.5f} | {r['p_sum']:.6f}, {r['p_min']:.5f}, {r['p_max']:.5f} |")
    print()
    for r in reports:
        if "counts" in r:
            print(f"{r['workload']}: per-expert counts {r['counts']}; f {r['f']}; p {r['p']}")


def decode(steps, warmup):
    """Decode steps at the DeepSeek-V3 shape (B = 1, 32, 128 tokens, the
    prefill batch's first B tokens and the same weights): experts touched
    against the uniform-routing estimate N (1 - (1 - k/N)^B), and the expert
    weight bytes the GEMMs must stream (touched routed experts + the shared
    one) over the GEMM time, against the HBM peak.  Prints a markdown table."""
    import torch
    import synthetic_inputs as si

    base = si.WORKLOADS["deepseek_v3"]
    inp = si.generate(base)
    g = {k: _to_dev(v) for k, v in inp.items()}
    del inp
    m = 3 if base.swiglu else 2
    per_expert = m * base.F * base.d * 2
    print("| B | experts touched (uniform estimate) | us/step | us/step, graph replay | tokens/s (graph) | "
          "route+dispatch us | GEMM up (+ shared) us | shared up (unfused) us | GEMM down (+ shared) us | combine us | weight bytes streamed | "
          "weight GB/s (% HBM) |")
    print("|---|---|---|---|---|---|---|---|---|---|---|---|")
    for B in (1, 32, 128):
        wl = si.decode(B)
        x = g["x"][:B].contiguous()
        L, ph, wall = _phases(wl, g, x, steps, warmup)
        gwall = graph_step_time(lambda: L.forward(x), steps, warmup)
        touched = int((L.counts > 0).sum().item())
        est = base.N * (1.0 - (1.0 - base.k / base.N) ** B)
        wbytes = (touched + (1 if base.shared else 0)) * per_expert
        sh = shared_up_runs(wl, True)
        gemm_us = ph[1] + (ph[2] if sh else 0.0) + ph[3]
        wgb = wbytes / (gemm_us * 1e-6) / 1e9
        print(f"| {B} | {touched} ({est:.1f}) | {wall * 1e6:.1f} | {gwall * 1e6:.1f} | {B / gwall:,.0f} | {ph[0]:.1f} | {ph[1]:.1f} | "
              f"{f'{ph[2]:.1f}' if sh else '-'} | {ph[3]:.1f} | {ph[4]:.1f} | {wbytes / 2**30:.2f} GiB | "
              f"{wgb:.0f} ({100 * wgb / PEAK_HBM_GBPS:.1f}%) |", flush=True)
        del L, x
        torch.cuda.empty_cache()


def memory(steps, warmup):
    """The memory-bound phases alone (route + dispatch, combine; also route
    and dispatch as separate calls) at every bf16 workload's full size, each
    launch timed with its own HIP events: warm (launches back to back) and
    cold (a 1 GiB buffer, four times the Infinity Cache, written untimed
    before every launch, so the inputs come from HBM).  Reports the median
    and p10/p90 duration and the algorithmic bytes at the median against the
    HBM peak, with a plain device copy of the same order of size as the
    ceiling.  Prints a markdown table."""
    import numpy as np
    import torch
    import synthetic_inputs as si
    from mixture_experts_layer_sparse_amd import moe as M

    flush = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")

    def timed(fn, cold):
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(steps + warmup)]
        for i, (e0, e1) in enumerate(ev):
            if cold:
                flush.fill_(i & 0xFF)
            e0.record()
            fn()
            e1.record()
        torch.cuda.synchronize()
        us = np.array([e0.elapsed_time(e1) for e0, e1 in ev[warmup:]]) * 1e3
        return np.percentile(us, [50, 10, 90])

    print("| workload | phase | algorithmic MiB | warm us (p10-p90) | warm GB/s (% HBM) | "
          "cold us (p10-p90) | cold GB/s (% HBM) |")
    print("|---|---|---|---|---|---|---|")

    def row(name, phase, nbytes, fn):
        cells = []
        for cold in (False, True):
            med, p10, p90 = timed(fn, cold)
            gbs = nbytes / (med * 1e-6) / 1e9
            cells += [f"{med:.1f} ({p10:.1f}-{p90:.1f})", f"{gbs:.0f} ({100 * gbs / PEAK_HBM_GBPS:.1f}%)"]
        print(f"| {name} | {phase} | {nbytes / 2**20:.1f} | " + " | ".join(cells) + " |", flush=True)

    for n in (1 << 26, 1 << 28):        # 64 MiB (fits the Infinity Cache) and 256 MiB copies
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        row("device copy", f"{n >> 20} MiB", 2 * n, lambda: dst.copy_(src))
        del src, dst
    for name in ("mixtral", "switch", "deepseek_v3", "dbrx"):
        wl = si.WORKLOADS[name]
        inp = si.generate(wl)
        g = {k: _to_dev(v) for k, v in inp.items()}
        del inp
        x = g["x"]
        s = M.shape_of(wl)
        L = M.Layer(s, g["wg"], g["w1"], g["w3"], g["w2"], bias=g["bias"], ws1=g["ws1"],
                    ws3=g["ws3"], ws2=g["ws2"])
        L.forward(x)                     # fills the expert outputs the combine reads
        torch.cuda.synchronize()
        R = int(L.offsets[-1].item())
        rb, db, cb = alg_bytes(wl, R)
        label = f"{name} (T={wl.T}, d={wl.d}, N={wl.N}, k={wl.k})"
        row(label, "route + dispatch", rb + db, lambda: L.route_dispatch(x))
        Lf = M.Layer(s, g["wg"], g["w1"], g["w3"], g["w2"], bias=g["bias"], ws1=g["ws1"],
                     ws3=g["ws3"], ws2=g["ws2"], fused=True)
        rf, df, _ = alg_bytes(wl, R, fused=True)
        row(label, "route + plan (fused layer)", rf + df, lambda: Lf.route_plan(x))
        del Lf
        row(label, "route", rb, lambda: L.route(x))
        row(label, "dispatch", db, lambda: L.dispatch(x))
        row(label, "combine", cb, lambda: L.combine(x))
        del L, g, x
        torch.cuda.empty_cache()


def main():
    a = parse()
    if a.mode == "summarize":
        summarize(a.prof, a.out or COUNTER_FILE, a.steps, a.warmup)
        return
    if a.mode == "sweep":
        sweep(a.steps, a.warmup)
        return
    if a.mode == "decode":
        decode(a.steps, a.warmup)
        return
    if a.mode == "memory":
        memory(a.steps, a.warmup)
        return
    if a.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU; --gpus must be 1"}))
        sys.exit(2)
    import numpy as np
    import torch
    import synthetic_inputs as si
    from mixture_experts_layer_sparse_amd import moe as M

    torch.cuda.set_device(0)
    if a.mode == "copy":
        n = 1 << 28                         # 256 MiB
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(10):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"mode": "copy", "bytes_read": n, "bytes_written": n, "launches": 10}))
        return

    wl = workload(a.workload)
    inp = si.generate(wl)

    def dev(arr):
        if arr is None:
            return None
        if arr.dtype == np.uint16:
            return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(np.ascontiguousarray(arr)).cuda()

    g = {k: dev(v) for k, v in inp.items()}
    s = M.shape_of(wl)
    fused = not a.unfused
    if a.scatter and a.unfused:
        raise SystemExit("--scatter is a form of the fused layer")
    L = M.Layer(s, g["wg"], g["w1"], g["w3"], g["w2"], bias=g["bias"], ws1=g["ws1"],
                ws3=g["ws3"], ws2=g["ws2"], fused=fused, scatter=a.scatter)
    x = g["x"]
    dt = s.torch_dtype
    h = torch.empty((wl.T * wl.k, wl.F), dtype=dt, device="cuda")
    hs = torch.empty((wl.T, wl.F), dtype=dt, device="cuda") if wl.shared else None
    # the same kernels as moe_forward, phase by phase
    step = layer_step(wl, L, x, h, hs)

    for _ in range(a.warmup):
        step()
    torch.cuda.synchronize()
    E = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(a.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(a.steps):
        step(E[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # (layer_step's phase order; with a shared expert its down GEMM runs in the routed down launch)
    ph = {"route_dispatch": [], "gemm_up": [], "shared_up": [], "gemm_down": [], "combine": []}
    for e in E:
        for j, key in enumerate(ph):
            ph[key].append(e[j].elapsed_time(e[j + 1]))
    ph_ms = {k: float(np.mean(v)) for k, v in ph.items()}
    ms = wall * 1e3 / a.steps
    R = int(L.offsets[-1].item())

    # the same result as the fused entry point
    y_split = L.y.clone()
    L.forward(x)
    torch.cuda.synchronize()
    assert torch.equal(y_split, L.y), "phase-by-phase and moe_forward results differ"
    # the same layer captured once in a HIP graph and replayed (the kernels
    # without host launch gaps); reported beside the eager steps
    gwall = graph_step_time(lambda: L.forward(x), a.steps, a.warmup)

    up, down, shared = gemm_flops(wl, R)
    rb, db, cb = alg_bytes(wl, R, fused)
    t_up = ph_ms["gemm_up"] * 1e-3
    achieved = up / t_up / 1e12
    if not shared_up_runs(wl, fused):
        ph_ms["shared_up"] = 0.0                  # (nothing launched between those two events)
    gemm_t = (ph_ms["gemm_up"] + ph_ms["shared_up"] + ph_ms["gemm_down"]) * 1e-3
    if a.scatter:
        # the combine runs in the down GEMM's epilogue: the memory phases are route + plan alone
        ph_ms["combine"] = 0.0
        cb = 0
    mem_t = (ph_ms["route_dispatch"] + ph_ms["combine"]) * 1e-3
    out = {
        "metric": METRIC,
        "value": wl.T * a.steps / wall,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if wl.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": wl.name, "T": wl.T, "d": wl.d, "N": wl.N, "k": wl.k, "F": wl.F,
                   "act": wl.act, "dispatch_buffer": "none (fused gather)" if fused else wl.buf,
                   "activations": wl.buf, "capacity": wl.capacity,
                   "groups": [wl.n_groups, wl.topk_groups], "shared_expert": wl.shared,
                   "kept_rows": R,
                   "combine": "in the down GEMM's epilogue" if a.scatter else "combine kernel"},
        "roofline": {"bound": "mfma", "kernel": "grouped GEMM up (gate/up + activation)",
                     "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / PEAK_BF16_TFLOPS,
                     "traffic": profiled_traffic(UP_KERNEL.get(wl.name)),
                     "traffic_unit": "bytes per launch: L2-miss bytes (FETCH_SIZE + WRITE_SIZE, each "
                                     "scaled by a plain copy of known size); Infinity Cache hits "
                                     "count as misses"},
        "grouped_gemm_pct_mfma_peak": 100.0 * (up + down + shared) / gemm_t / 1e12 / PEAK_BF16_TFLOPS,
        # route and dispatch run as one call, so their bytes are timed together
        "dispatch_GBps": (rb + db) / (ph_ms["route_dispatch"] * 1e-3) / 1e9,
        "dispatch_GBps_covers": ("route + plan (moe_route_plan; no dispatch copy: the up GEMM gathers x "
                                 "through src)") if fused else "route + dispatch (moe_route_dispatch)",
        "combine_GBps": cb / (ph_ms["combine"] * 1e-3) / 1e9 if cb else None,
        "memory_phases": {"bytes": rb + db + cb, "us": mem_t * 1e6,
                          "GBps": (rb + db + cb) / mem_t / 1e9,
                          "frac_hbm": (rb + db + cb) / mem_t / 1e9 / PEAK_HBM_GBPS},
        "phases_us": {k: v * 1e3 for k, v in ph_ms.items()},
        "graph_replay": {"ms_per_step": gwall * 1e3, "tokens_per_s": wl.T / gwall},
    }
    if not a.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wl, inp, a.cpu_sample_tokens or wl.T)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
