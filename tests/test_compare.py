"""The tie-band adoption procedure used by the GPU parity tests (CPU only)."""
import numpy as np

import synthetic_inputs as si
from oracle import compare, moe


def wl(**kw):
    base = dict(T=4, d=4, N=8, k=2, F=8, act="silu", dtype="f32", buf="f32")
    base.update(kw)
    return si.Workload("cmp", **base)


def test_identical_selection_needs_no_adoption():
    w = wl()
    l = np.array([[3.0, 1.0, 2.0, 0.0, -1.0, 0.5, 0.2, 0.1]])
    idx = moe.top_k(l, np.ones_like(l, bool), 2)
    r = compare.adopt(w, l, idx, idx)
    assert r["adopted"] == [] and r["bad"] == []


def test_near_tie_at_kth_is_adopted():
    w = wl()
    l = np.array([[3.0, 1.0, 2.0, 2.0 + 1e-9, -1.0, 0.5, 0.2, 0.1]])
    o = moe.top_k(l, np.ones_like(l, bool), 2)
    assert o.tolist() == [[0, 3]]
    r = compare.adopt(w, l, o, np.array([[0, 2]]))
    assert r["adopted"] == [0] and r["bad"] == []
    assert np.allclose(r["w"][0], moe.sparse_softmax(l, np.array([[0, 2]]))[0])


def test_clear_gap_is_rejected():
    w = wl()
    l = np.array([[3.0, 1.0, 2.0, 2.1, -1.0, 0.5, 0.2, 0.1]])
    o = moe.top_k(l, np.ones_like(l, bool), 2)
    r = compare.adopt(w, l, o, np.array([[0, 2]]))
    assert r["bad"] == [0]
    # wrong slot order outside the band is also rejected
    r = compare.adopt(w, l, o, np.array([[3, 0]]))
    assert r["bad"] == [0]
    # duplicates are never admissible
    r = compare.adopt(w, l, o, np.array([[0, 0]]))
    assert r["bad"] == [0]


def test_group_level_near_tie():
    w = wl(N=8, k=2, n_groups=4, topk_groups=1, group_score_k=2)
    # group scores: g0 = 3, g1 = 3 + 1e-9 -> oracle keeps g1; the GPU may keep g0
    l = np.array([[2.0, 1.0, 1.5, 1.5 + 1e-9, 0.0, 0.0, -1.0, -1.0]])
    mask = moe.group_mask(l, 4, 1, 2)
    o = moe.top_k(l, mask, 2)
    assert o.tolist() == [[3, 2]]
    r = compare.adopt(w, l, o, np.array([[0, 1]]))
    assert r["adopted"] == [0]
    r = compare.adopt(w, l, o, np.array([[0, 4]]))         # mixes groups: never admissible
    assert r["bad"] == [0]


def test_rel_l2():
    a = np.array([1.0, 2.0, 2.0])
    assert compare.rel_l2(a, a) == 0.0
    assert abs(compare.rel_l2(a * 1.01, a) - 0.01) < 1e-12


def test_twenty_way_tie_keeps_the_clear_winners():
    """A token whose logits tie 20 ways below two clear leaders: any selection
    of the leaders plus band members is admissible, one that leaves a leader
    out is not (checked without enumerating the band's subsets)."""
    w = wl(N=24, k=4)
    l = np.zeros((1, 24))
    l[0, 5], l[0, 17] = 3.0, 2.0
    l[0, 20:] = -1.0                              # below the band
    o = moe.top_k(l, np.ones_like(l, bool), 4)
    assert o.tolist() == [[5, 17, 0, 1]]
    r = compare.adopt(w, l, o, np.array([[5, 17, 19, 3]]))
    assert r["adopted"] == [0] and r["bad"] == []
    r = compare.adopt(w, l, o, np.array([[5, 19, 3, 2]]))       # leader 17 left out
    assert r["bad"] == [0]
    r = compare.adopt(w, l, o, np.array([[5, 17, 3, 21]]))      # 21 is below the band
    assert r["bad"] == [0]


def test_many_group_tie_keeps_the_clear_group():
    """64 groups of one expert with 40 of them tied: a selection must keep the
    clearly best group's expert, whichever tied groups fill the rest."""
    w = wl(N=64, k=2, n_groups=64, topk_groups=20, group_score_k=1)
    l = np.full((1, 64), -2.0)
    l[0, :40] = 0.0
    l[0, 50] = 5.0
    mask = moe.group_mask(l, 64, 20, 1)
    o = moe.top_k(l, mask, 2)
    assert o.tolist() == [[50, 0]]
    r = compare.adopt(w, l, o, np.array([[50, 33]]))
    assert r["adopted"] == [0]
    r = compare.adopt(w, l, o, np.array([[33, 12]]))             # the clear winner left out
    assert r["bad"] == [0]
    r = compare.adopt(w, l, o, np.array([[50, 45]]))             # expert 45 is below the band
    assert r["bad"] == [0]
