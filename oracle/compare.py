"""Comparison procedure for routing decisions (test infrastructure).

The GPU computes logits in float32, the oracle in float64, so a token whose
k-th and (k+1)-th logits are nearly equal may legitimately be routed
differently.  The acceptance rule: routing must be bit-exact except where the
oracle's k-th and (k+1)-th logits differ by less than 1e-5 relative.

Reading of "relative" (a pure relative test breaks near zero): token t is in
the tie band when the gap is at most delta_t = tol * max_e |l[t][e]|.  The same
band applies to the group ranking (the topk_groups-th versus the next group
score) and to the order of adjacent selected slots.

``adopt`` checks each differing token: when the GPU's selection is admissible
(it contains every candidate clearly above the band and fills the rest from
inside the band, in an order that is descending up to the band), the oracle
takes the GPU's selection for that token and recomputes that token's weights
from its own float64 logits.  Anything else is a mismatch.
"""
from __future__ import annotations

import itertools
import math

import numpy as np

from . import moe


def _band(scores: np.ndarray, allowed: np.ndarray, m: int, delta: float):
    """The tie band of an m-selection among the ``allowed`` indices: ``must``
    (scores clearly above the m-th largest, thr + delta) and ``band`` (scores
    within delta of it).  An m-subset S is admissible exactly when
    must <= S <= must | band."""
    cand = np.flatnonzero(allowed)
    vals = scores[cand]
    order = cand[np.argsort(-vals, kind="stable")]
    thr = scores[order[m - 1]]
    must = {int(i) for i in cand if scores[i] > thr + delta}
    band = {int(i) for i in cand if abs(scores[i] - thr) <= delta}
    return must, band


def _set_admissible(sel: set, must: set, band: set, m: int) -> bool:
    return len(sel) == m and must <= sel and sel <= (must | band)


# group sets enumerated at most (a tie among more groups is checked by the
# necessary conditions only)
_MAX_GROUP_SETS = 1 << 16


def admissible(wl, l_t: np.ndarray, sel: np.ndarray, tol: float = 1e-5) -> bool:
    """Is the GPU selection ``sel`` (k expert ids in slot order) admissible for
    a token with float64 logits ``l_t``?"""
    N, k = wl.N, wl.k
    sel = [int(e) for e in sel]
    if len(set(sel)) != k or min(sel) < 0 or max(sel) >= N:
        return False
    delta = tol * float(np.max(np.abs(l_t))) if l_t.size else 0.0
    # slot order: descending up to the band
    for a, b in zip(sel[:-1], sel[1:]):
        if l_t[a] < l_t[b] - delta:
            return False
    S = set(sel)
    if wl.n_groups <= 1:
        must, band = _band(l_t, np.ones(N, bool), k, delta)
        return _set_admissible(S, must, band, k)
    G, gsz, kg = wl.n_groups, N // wl.n_groups, wl.topk_groups
    gs = moe.group_scores(l_t[None, :], G, wl.group_score_k)[0]
    gmust, gband = _band(gs, np.ones(G, bool), kg, delta)
    used = {e // gsz for e in sel}
    # the groups a selection may use: an admissible group set holds gmust, lies
    # inside gmust | gband and has kg groups, so the used groups must fit too
    if not used <= (gmust | gband):
        return False
    free = sorted(gband - gmust - used)
    need = kg - len(gmust | used)
    if need < 0 or need > len(free):
        return False
    if math.comb(len(free), need) > _MAX_GROUP_SETS:
        # a tie among very many groups: every expert of the used and the
        # clearly better groups is a candidate; the selection must hold every
        # expert clearly above the band of that candidate set
        mk = np.zeros(N, bool)
        for g in gmust | used:
            mk[g * gsz:(g + 1) * gsz] = True
        must, band = _band(l_t, mk, k, delta)
        return must <= S
    for fill in itertools.combinations(free, need):
        mk = np.zeros(N, bool)
        for g in gmust | used | set(fill):
            mk[g * gsz:(g + 1) * gsz] = True
        must, band = _band(l_t, mk, k, delta)
        if _set_admissible(S, must, band, k):
            return True
    return False


def adopt(wl, logits: np.ndarray, oracle_idx: np.ndarray, gpu_idx: np.ndarray,
          tol: float = 1e-5) -> dict:
    """Merge the GPU's routing into the oracle's where it is admissible.

    Returns {"idx", "w", "adopted": [tokens], "bad": [tokens]}.  ``w`` is the
    oracle's float64 gate weights for the (possibly adopted) selection."""
    gpu_idx = np.asarray(gpu_idx).astype(np.int64).reshape(oracle_idx.shape)
    idx = oracle_idx.astype(np.int64).copy()
    diff = np.flatnonzero(np.any(idx != gpu_idx, axis=1))
    adopted, bad = [], []
    for t in diff:
        if admissible(wl, logits[t], gpu_idx[t], tol):
            idx[t] = gpu_idx[t]
            adopted.append(int(t))
        else:
            bad.append(int(t))
    w = moe.gate_weights(wl, logits, idx) if idx.size else np.zeros(idx.shape)
    return {"idx": idx.astype(np.int32), "w": w, "adopted": adopted, "bad": bad}


def rel_l2(a: np.ndarray, ref: np.ndarray) -> float:
    """||a - ref||_2 / ||ref||_2 over the whole tensor, in float64."""
    a = np.asarray(a, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.linalg.norm(ref.ravel())
    num = np.linalg.norm((a - ref).ravel())
    if den == 0.0:
        return 0.0 if num == 0.0 else float("inf")
    return float(num / den)
