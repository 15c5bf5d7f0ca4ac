"""The sparse MoE-layer forward, step by step, in float64 (test infrastructure).

Sources (web pages; cited by title and section):
  [Part5]    "Advanced GPU Optimization: How to tech an LLM with CUDA and ROCm? -
             Part 5 (Final Part)": "The Math"; "1.1 The Router Kernel (Top-k
             Gating)"; "1.2 Expert Parallelism with All-to-All Communication".
  [Costs]    "MoE: what it costs to train and serve": "Expert parallelism and two
             all-to-alls"; "Worked example: how many bytes does one token send?";
             "Limit how many machines a token touches".
  [Glossary] "moe communication costs": "Router design" (G(x) and y equations);
             "Load balancing - the critical auxiliary loss" (L_aux, f_i, p_i);
             "Capacity factor and token dropping"; the architecture table.

Readings taken where the pages are silent or disagree (each is also listed with
the design notes):
  * mixture weights are the softmax over only the k selected logits ([Part5]
    "The Math" and the router kernel's sparse softmax), not the full-softmax
    G(x)_i of [Glossary];
  * the exploration noise epsilon of [Glossary] "Router design" is a training
    device and is zero here;
  * top-k order is logit descending, ties to the lower expert index (the router
    kernel scans experts in index order and replaces only on a strictly larger
    score);
  * the group limit ([Costs] "Limit how many machines a token touches") scores
    each contiguous group of N/G experts by the sum of its ``group_score_k``
    largest logits and keeps the ``topk_groups`` best groups (ties to the lower
    group);
  * f_i = counts_i / (T k), counted before capacity drops; p_i = the mean over
    tokens of the full softmax over all N (biased) logits, no group mask;
  * capacity keeps the first C assignments of each expert in token order; a
    dropped slot passes the token through (weight times x) or contributes zero;
  * a router bias, when present, is added to the logits before every use;
  * the shared expert runs on the unquantised input with weight 1;
  * MXFP4 expert weights (an option): each weight is its FP4 E2M1 code's
    value times its 32-element block's E8M0 scale, decoded exactly;
  * fp8 dispatch: per token, amax = max|x|, inv = fl32(448 / amax),
    code = e4m3(fl32(x * inv)), scale = fl32(amax / 448); amax < 2^-100
    (zero included) gives inv = scale = 1, so every code is +-0.
"""
from __future__ import annotations

import numpy as np

from .numerics import E4M3_MAX, as_f64, as_weights, e4m3_decode, e4m3_encode, f32


# ----------------------------------------------------------------- routing --

def router_logits(x: np.ndarray, wg: np.ndarray, bias: np.ndarray | None = None) -> np.ndarray:
    """l[t][e] = sum_j x[t][j] W_g[e][j] (+ b[e]).  [Glossary] "Router design":
    W_g has one row of length d per expert; [Part5] 1.1: gate_logits[t][e] is
    the dot product of token t with router row e."""
    l = np.asarray(x, np.float64) @ np.asarray(wg, np.float64).T
    if bias is not None:
        l = l + np.asarray(bias, np.float64)[None, :]
    return l


def group_scores(l: np.ndarray, n_groups: int, score_k: int) -> np.ndarray:
    """gs[t][g] = sum of the score_k largest logits among experts
    g*N/G .. (g+1)*N/G - 1.  [Costs] "Limit how many machines a token touches"."""
    T, N = l.shape
    gsz = N // n_groups
    lg = l.reshape(T, n_groups, gsz)
    top = -np.sort(-lg, axis=2)[:, :, :score_k]
    return top.sum(axis=2)


def group_mask(l: np.ndarray, n_groups: int, topk_groups: int, score_k: int) -> np.ndarray:
    """Boolean [T][N]: True for experts inside the topk_groups best groups of
    each token, ranked by group score descending, ties to the lower group."""
    T, N = l.shape
    if n_groups <= 1:
        return np.ones((T, N), dtype=bool)
    gs = group_scores(l, n_groups, score_k)
    order = np.argsort(-gs, axis=1, kind="stable")
    keep = np.zeros((T, n_groups), dtype=bool)
    np.put_along_axis(keep, order[:, :topk_groups], True, axis=1)
    return np.repeat(keep, N // n_groups, axis=1)


def top_k(l: np.ndarray, mask: np.ndarray, k: int) -> np.ndarray:
    """idx[t][j]: the k largest unmasked logits, descending, ties to the lower
    index (stable sort of the negated logits).  [Part5] 1.1, [Glossary] TopK."""
    key = np.where(mask, l, -np.inf)
    return np.argsort(-key, axis=1, kind="stable")[:, :k].astype(np.int32)


def sparse_softmax(l: np.ndarray, idx: np.ndarray) -> np.ndarray:
    """w[t][j] = exp(l_j - l_max) / sum_i exp(l_i - l_max) over the k selected
    logits only ([Part5] "1.1 The Router Kernel": the softmax runs over the two
    kept scores alone; generalised here to k; max-subtracted for stability as
    the kernel does)."""
    sel = np.take_along_axis(l, idx.astype(np.int64), axis=1)
    z = np.exp(sel - sel.max(axis=1, keepdims=True))
    return z / z.sum(axis=1, keepdims=True)


def full_softmax(l: np.ndarray) -> np.ndarray:
    """G(x) = softmax over all N logits.  [Glossary] "Router design"."""
    z = np.exp(l - l.max(axis=1, keepdims=True))
    return z / z.sum(axis=1, keepdims=True)


def gate_weights(wl, l: np.ndarray, idx: np.ndarray) -> np.ndarray:
    """Weights of the selected experts.  "sparse": the softmax over the k
    selected logits ([Part5] The Math, 1.1).  "full": each selected expert's
    probability under the softmax over all N logits, not renormalised
    ([Glossary] "Router design": y = sum over the top-k of G(x)_i E_i(x),
    G(x) = softmax(W_g x))."""
    if getattr(wl, "gate", "sparse") == "full":
        return np.take_along_axis(full_softmax(l), idx.astype(np.int64), axis=1)
    return sparse_softmax(l, idx)


def load_stats(l: np.ndarray, idx: np.ndarray, N: int, capacity: int, alpha: float) -> dict:
    """counts, kept_counts, f, p and L_aux = alpha * N * sum_i f_i p_i.
    [Glossary] "Load balancing": f_i the fraction of routed assignments that go
    to expert i, p_i the mean router probability of expert i over the batch;
    "Capacity factor": at most C tokens per expert."""
    T = l.shape[0]
    k = idx.shape[1] if idx.ndim == 2 else 0
    counts = np.bincount(idx.ravel().astype(np.int64), minlength=N)[:N].astype(np.int64)
    kept = np.minimum(counts, capacity) if capacity > 0 else counts.copy()
    if T == 0:
        f = np.zeros(N)
        p = np.zeros(N)
    else:
        f = counts / float(T * k)
        p = full_softmax(l).mean(axis=0)
    return {"counts": counts, "kept_counts": kept, "f": f, "p": p,
            "l_aux": float(alpha * N * np.sum(f * p))}


def route(wl, x: np.ndarray, wg: np.ndarray, bias: np.ndarray | None) -> dict:
    """Router: logits, group limit, top-k, gate weights, load statistics.
    ``x`` and ``wg`` are float64 (already widened)."""
    l = router_logits(x, wg, bias)
    mask = group_mask(l, wl.n_groups, wl.topk_groups, wl.group_score_k)
    idx = top_k(l, mask, wl.k)
    w = gate_weights(wl, l, idx)
    out = {"logits": l, "idx": idx, "w": w}
    out.update(load_stats(l, idx, wl.N, wl.capacity, wl.alpha))
    return out


# ---------------------------------------------------------------- dispatch --

def dispatch_plan(idx: np.ndarray, N: int, capacity: int) -> dict:
    """Expert-major stable order of the assignments a = t*k + j.

    rank[a] = number of earlier assignments (smaller a) to the same expert; an
    assignment is kept when capacity <= 0 or rank < capacity; offsets is the
    exclusive scan of the kept counts; pos[a] = offsets[e] + rank for kept
    assignments and -1 otherwise; src[pos] = t.  This is the single-GPU form
    of the dispatch all-to-all's send buffer ([Part5] 1.2 step 1, [Costs]
    "Expert parallelism": per-destination contiguous slices)."""
    T, k = idx.shape
    flat = idx.ravel().astype(np.int64)
    order = np.argsort(flat, kind="stable")
    counts = np.bincount(flat, minlength=N)[:N]
    starts = np.concatenate([[0], np.cumsum(counts)])
    rank = np.empty(flat.size, dtype=np.int64)
    rank[order] = np.arange(flat.size) - starts[flat[order]]
    keep = (rank < capacity) if capacity > 0 else np.ones(flat.size, dtype=bool)
    kept_counts = np.minimum(counts, capacity) if capacity > 0 else counts
    offsets = np.concatenate([[0], np.cumsum(kept_counts)]).astype(np.int64)
    pos = np.where(keep, offsets[flat] + rank, -1)
    R = int(offsets[N])
    src = np.full(R, -1, dtype=np.int64)
    src[pos[keep]] = (np.arange(flat.size) // k)[keep]
    return {"offsets": offsets, "pos": pos.reshape(T, k), "src": src,
            "drop": (~keep).reshape(T, k), "rank": rank.reshape(T, k)}


def quantize_fp8_rows(x_bits_or_vals: np.ndarray, dtype: str) -> tuple:
    """Per-token fp8 e4m3fn quantisation of the dispatch payload ([Costs] worked
    example on bytes per token: FP8 before dispatch, s = 1).  The scale is one
    float32 per token; every step is float32 arithmetic on the stored values:
    amax = max|x| (exact), inv = fl32(448/amax), code = e4m3(fl32(x*inv)),
    scale = fl32(amax/448); a row with amax < 2^-100 gets inv = scale = 1.
    Returns (codes uint8 [T][d], scale float32 [T])."""
    xv = f32(as_f64(x_bits_or_vals, dtype))
    T = xv.shape[0]
    amax = np.abs(xv).max(axis=1) if xv.shape[1] else np.zeros(T, np.float32)
    amax = f32(amax)
    # a row whose largest magnitude is below 2^-100 (zero included) is treated
    # as a zero row: 448/amax would overflow float32 below about 1.3e-36
    zero = amax < np.float32(2.0 ** -100)
    safe = np.where(zero, np.float32(1), amax)
    inv = np.where(zero, np.float32(1), f32(np.float32(E4M3_MAX) / safe))
    scale = np.where(zero, np.float32(1), f32(safe / np.float32(E4M3_MAX)))
    v = f32(xv * inv[:, None])
    return e4m3_encode(v), f32(scale)


def dispatch_values(wl, x_store: np.ndarray, plan: dict) -> dict:
    """The expert-ordered buffer X_perm[pos[t][j]] = Q(x[t]) for kept slots.
    Q is the identity for f32/bf16 buffers (values are the stored values), or
    the fp8 quantiser.  Returns the stored buffer (values, bf16 bits or fp8
    codes), per-row scales (fp8 only), and the dequantised float64 rows."""
    src = plan["src"]
    if wl.buf == "fp8":
        codes, scale = quantize_fp8_rows(x_store, wl.dtype)
        buf = codes[src]
        row_scale = scale[src]
        rows = e4m3_decode(buf) * row_scale.astype(np.float64)[:, None]
        return {"buf": buf, "row_scale": row_scale, "rows": rows,
                "tok_codes": codes, "tok_scale": scale}
    buf = np.asarray(x_store)[src]
    return {"buf": buf, "row_scale": None, "rows": as_f64(buf, wl.dtype)}


# ----------------------------------------------------------------- experts --

def activation(act: str, u: np.ndarray, g: np.ndarray | None = None) -> np.ndarray:
    """silu(u) = u / (1 + e^-u); relu(u) = max(u, 0); swiglu = silu(u) * g
    (textbook definitions; the pages name the expert FFN without fixing it)."""
    with np.errstate(over="ignore"):
        if act == "relu":
            return np.maximum(u, 0.0)
        s = u / (1.0 + np.exp(-u))
    if act == "silu":
        return s
    if act == "swiglu":
        return s * g
    raise ValueError(act)


def expert_ffn(act: str, a: np.ndarray, w1: np.ndarray, w3: np.ndarray | None,
               w2: np.ndarray) -> np.ndarray:
    """One expert on rows a [m][d]: o = W2 act(W1 a, W3 a), W1/W3 [F][d], W2 [d][F].
    [Glossary] "The core idea": each expert is a feed-forward network."""
    u = a @ w1.T
    g = a @ w3.T if w3 is not None else None
    return activation(act, u, g) @ w2.T


def combine(wl, x: np.ndarray, w: np.ndarray, pos: np.ndarray, o_rows: np.ndarray,
            shared: np.ndarray | None) -> np.ndarray:
    """y[t] = sum_j w[t][j] * (O[pos[t][j]] if kept, else x[t] (pass-through),
    0, or S[t] (fallback to the shared expert)) + S[t].  [Glossary] y = sum over
    TopK of weight times E_i(x); "Capacity factor and token dropping" for
    dropped slots (skip through the residual, or a shared fallback expert)."""
    T, d = x.shape
    y = np.zeros((T, d))
    for j in range(w.shape[1] if w.ndim == 2 else 0):
        pj = pos[:, j]
        kept = pj >= 0
        term = np.zeros((T, d))
        term[kept] = o_rows[pj[kept]]
        if wl.drop == "passthrough":
            term[~kept] = x[~kept]
        elif wl.drop == "fallback":
            term[~kept] = shared[~kept]
        y += w[:, j:j + 1] * term
    if shared is not None:
        y += shared
    return y


# ----------------------------------------------------------------- forward --

def forward(wl, inp: dict, ffn_tokens: np.ndarray | None = None,
            routed: dict | None = None) -> dict:
    """The whole layer.  ``inp`` holds the stored inputs from the generator.
    ``ffn_tokens`` (optional) restricts the expert FFNs and combine to a subset
    of tokens (routing, statistics and the plan are always computed on all T);
    y then has one row per listed token.  ``routed`` (optional) supplies an
    already-adopted routing (idx, w) to use instead of the oracle's own."""
    x = as_f64(inp["x"], wl.dtype)
    r = route(wl, x, as_f64(inp["wg"], wl.dtype), inp.get("bias"))
    if routed is not None:
        r["idx"], r["w"] = routed["idx"], routed["w"]
        r.update(load_stats(r["logits"], r["idx"], wl.N, wl.capacity, wl.alpha))
    plan = dispatch_plan(r["idx"], wl.N, wl.capacity)
    vals = dispatch_values(wl, inp["x"], plan)
    out = dict(r)
    out.update(plan)
    out.update({"xperm": vals["buf"], "row_scale": vals["row_scale"]})
    if "w1" not in inp or inp["w1"] is None:
        return out

    T = wl.T
    toks = np.arange(T) if ffn_tokens is None else np.asarray(ffn_tokens, np.int64)
    pos = plan["pos"][toks]
    # rows of the dispatch buffer that the chosen tokens need
    need = np.unique(pos[pos >= 0])
    o_rows = np.zeros((plan["src"].size, wl.d))
    offs = plan["offsets"]
    # expert weights: the layer's storage type, or MXFP4 blocks decoded exactly
    wf = getattr(wl, "wfmt", "bf16")
    F, d = wl.F, wl.d

    def w_up(a):
        return as_weights(a, wf, wl.dtype, F, d)

    def w_down(a):
        return as_weights(a, wf, wl.dtype, d, F)

    for e in range(wl.N):
        sel = need[(need >= offs[e]) & (need < offs[e + 1])]
        if sel.size == 0:
            continue
        w1 = w_up(inp["w1"][e])
        w3 = w_up(inp["w3"][e]) if inp.get("w3") is not None else None
        w2 = w_down(inp["w2"][e])
        o_rows[sel] = expert_ffn(wl.act, vals["rows"][sel], w1, w3, w2)
    shared = None
    if wl.shared:
        ws3 = w_up(inp["ws3"]) if inp.get("ws3") is not None else None
        shared = expert_ffn(wl.act, x[toks], w_up(inp["ws1"]), ws3, w_down(inp["ws2"]))
    y = combine(wl, x[toks], r["w"][toks], pos, o_rows, shared)
    out.update({"o_rows": o_rows, "shared": shared, "y": y, "y_tokens": toks})
    return out


def dispatch_bytes(R: int, d: int, s: int) -> int:
    """Payload of the dispatch buffer: R rows of d numbers of s bytes; with no
    drops R = T k, i.e. k*d*s bytes per token ([Costs] "bytes = k x d x s")."""
    return R * d * s
