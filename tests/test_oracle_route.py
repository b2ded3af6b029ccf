"""Pins for the oracle's sigmoid score and group-limited top-k gating.

The gating pins do not re-type the oracle's loops: the brute force below
characterises the selection as the subset with the largest exact sum (with
the lexicographically smallest index set among equals), which is what
"take the k best, lower index first" means, and enumerates all subsets."""
import itertools
import math
from fractions import Fraction

import numpy as np
import pytest


def test_sigmoid_landmarks(orc):
    s = orc.sigmoid(np.array([0.0, 1.0, -1.0, 87.0, -87.0, 1000.0, -1000.0], np.float32))
    assert s[0] == 0.5
    assert s[1] == np.float32(1.0 / (1.0 + math.exp(-1.0)))
    assert s[1] + s[2] == 1.0
    assert s[5] == s[3] and s[6] == s[4] > 0  # clamp to [-87, 87] keeps results normal


def test_sigmoid_strided_sweep(orc):
    # every 13th positive fp32 up to 87 and its negation, against fp64 libm
    worst, n, nonmono = orc.sigmoid_sweep(0, 0x42AE0000, 13)
    assert n > 1.5e8
    assert worst <= 0.5 + 1e-6, worst
    assert nonmono == 0


@pytest.mark.slow
def test_sigmoid_exhaustive_sweep(orc):
    # every fp32 in [-87, 87]
    worst, n, nonmono = orc.sigmoid_sweep(0, 0x42AE0000, 1)
    assert n == 2 * (0x42AE0000 + 1)
    assert worst <= 0.5 + 1e-6, worst
    assert nonmono == 0


def brute_select(s, n_group, topk_group, K):
    """s: float32 scores of one token.  Exhaustive over subsets."""
    N = len(s)
    gs = N // n_group
    # group score: the largest fp32 pair sum inside the group (fp32 rounding is
    # monotone, so this is the fp32 sum of the two largest)
    gsc = []
    for j in range(n_group):
        mem = s[j * gs:(j + 1) * gs]
        if gs == 1:
            gsc.append(mem[0])
        else:
            gsc.append(max(np.float32(mem[a] + mem[b]) for a, b in itertools.combinations(range(gs), 2)))

    def best_subset(vals, cand, k):
        best, best_key = None, None
        for sub in itertools.combinations(cand, k):  # combinations are in lexicographic order
            tot = sum(Fraction(float(vals[i])) for i in sub)
            if best is None or tot > best_key:
                best, best_key = sub, tot
        return best

    groups = best_subset(gsc, range(n_group), topk_group)
    cand = [e for g in groups for e in range(g * gs, (g + 1) * gs)]
    chosen = best_subset(s, sorted(cand), K)
    return sorted(chosen, key=lambda e: (-s[e], e)), groups


def check_invariants(s, ids, w, n_group, topk_group, K, scale):
    N = len(s)
    gs = N // n_group
    assert len(set(ids)) == K
    groups = {e // gs for e in ids}
    assert len(groups) <= topk_group
    # ordering: score desc, index asc
    keys = [(-s[e], e) for e in ids]
    assert keys == sorted(keys)
    # weights: positive, follow the score order, sum to scale
    assert np.all(w > 0)
    assert np.all(np.diff(w.astype(np.float64)) <= 0)
    assert abs(float(np.sum(w.astype(np.float64))) - scale) <= 4 * np.finfo(np.float32).eps * scale
    for k in range(K):
        assert abs(float(w[k]) - float(s[ids[k]]) / sum(float(s[e]) for e in ids) * scale) <= \
            np.finfo(np.float32).eps * scale


def _cases():
    rng = np.random.default_rng(7)
    out = [(4, 2, 4, 4)]  # the tiny workload's routing shape: 16 experts
    while len(out) < 40:
        n_group = int(rng.integers(2, 7))
        gs = int(rng.integers(1, 6))
        tg = int(rng.integers(1, n_group + 1))
        if tg * gs > 12:
            continue
        K = int(rng.integers(1, min(6, tg * gs) + 1))
        out.append((n_group, gs, tg, K))
    return out


@pytest.mark.parametrize("n_group,gs,topk_group,K", _cases())
@pytest.mark.parametrize("ties", [False, True])
def test_route_brute_force(orc, n_group, gs, topk_group, K, ties):
    rng = np.random.default_rng([n_group, gs, topk_group, K, ties])
    B = 24
    N = n_group * gs
    if ties:  # exact ties are common with logits from {-1, 0, 1}
        logits = rng.integers(-1, 2, (B, N)).astype(np.float32)
    else:
        logits = rng.standard_normal((B, N)).astype(np.float32)
    scale = 1.0 if not ties else 2.5
    ids, w = orc.route(logits, n_group, topk_group, K, scale)
    s = orc.sigmoid(logits)
    for t in range(B):
        want, _ = brute_select(s[t], n_group, topk_group, K)
        assert list(ids[t]) == want, (t, logits[t])
        check_invariants(s[t], list(ids[t]), w[t], n_group, topk_group, K, scale)


def test_route_no_groups_is_plain_topk(orc):
    # one group (or all groups kept) reduces to an ordinary top-K, which
    # numpy's lexsort on (index, -score) gives directly
    rng = np.random.default_rng(11)
    logits = rng.standard_normal((300, 64)).astype(np.float32)
    logits[:50] = np.round(logits[:50])  # plenty of ties
    s = orc.sigmoid(logits)
    for n_group, tg in [(1, 1), (8, 8), (64, 64)]:
        ids, _ = orc.route(logits, n_group, tg, 6)
        for t in range(len(logits)):
            order = np.lexsort((np.arange(64), -s[t].astype(np.float64)))[:6]
            assert list(ids[t]) == list(order)


def test_route_deepseek_shape_invariants(orc):
    # 256 experts in 8 groups of 32, 4 groups kept, top-8: no unselected expert
    # inside a kept group beats a selected one, and every kept group's score is
    # at least every dropped group's score
    rng = np.random.default_rng(5)
    logits = (rng.standard_normal((256, 256)) + rng.normal(0, 0.5, 256)).astype(np.float32)
    ids, w = orc.route(logits, 8, 4, 8)
    s = orc.sigmoid(logits)
    for t in range(256):
        st = s[t]
        gsc = np.array([np.float32(np.sort(st[j * 32:(j + 1) * 32])[-1] + np.sort(st[j * 32:(j + 1) * 32])[-2])
                        for j in range(8)])
        used = sorted({e // 32 for e in ids[t]})
        # the selection may use fewer than 4 groups, but all used groups rank in the top 4
        rank = sorted(range(8), key=lambda j: (-gsc[j], j))[:4]
        assert set(used) <= set(rank)
        assert min(gsc[j] for j in rank) >= max(gsc[j] for j in range(8) if j not in rank)
        cand = [e for g in rank for e in range(g * 32, (g + 1) * 32) if e not in ids[t]]
        worst_sel = min((st[e], -e) for e in ids[t])
        assert all((st[e], -e) < worst_sel for e in cand)
        check_invariants(st, list(ids[t]), w[t], 8, 4, 8, 1.0)


def test_route_rejects_bad_shapes(orc):
    with pytest.raises(ValueError):
        orc.route(np.zeros((2, 10), np.float32), 4, 2, 2)   # 10 not divisible by 4
    with pytest.raises(ValueError):
        orc.route(np.zeros((2, 8), np.float32), 4, 1, 3)    # K > candidates


# ---------------------------------------------------------------- selection-only bias
# (a variant not on the pages: a per-expert correction added to the scores for
# the choice only; the weights renormalise the plain scores)

@pytest.mark.parametrize("n_group,gs,topk_group,K", _cases()[:20])
@pytest.mark.parametrize("ties", [False, True])
def test_biased_route_brute_force(orc, n_group, gs, topk_group, K, ties):
    rng = np.random.default_rng([n_group, gs, topk_group, K, ties, 99])
    B, N = 24, n_group * gs
    if ties:
        logits = rng.integers(-1, 2, (B, N)).astype(np.float32)
        bias = (rng.integers(-2, 3, N) * 0.125).astype(np.float32)     # exact sums: ties survive
    else:
        logits = rng.standard_normal((B, N)).astype(np.float32)
        bias = rng.normal(0.0, 0.7, N).astype(np.float32)             # negative choosing scores too
    ids, w = orc.route(logits, n_group, topk_group, K, 1.0, bias=bias)
    s = orc.sigmoid(logits)
    for t in range(B):
        sel = (s[t] + bias).astype(np.float32)                         # one fp32 rounding per expert
        want, _ = brute_select(sel, n_group, topk_group, K)
        assert list(ids[t]) == want, (t, logits[t])
        # weights from the plain scores of the chosen experts
        plain = np.array([float(s[t][e]) for e in ids[t]])
        assert np.allclose(w[t], plain / plain.sum(), rtol=2e-7, atol=0)


def test_zero_bias_is_the_plain_route(orc):
    rng = np.random.default_rng(21)
    logits = (rng.standard_normal((200, 256)) + rng.normal(0, 0.5, 256)).astype(np.float32)
    a = orc.route(logits, 8, 4, 8)
    b = orc.route(logits, 8, 4, 8, bias=np.zeros(256, np.float32))
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_large_bias_forces_the_choice(orc):
    # a +10 bias on experts 40..47 (all in group 1 of 8 groups of 32) outranks
    # any sigmoid score: those 8 are chosen for every token, in the order of
    # their plain scores, whatever the logits
    rng = np.random.default_rng(22)
    logits = rng.standard_normal((64, 256)).astype(np.float32) * 3
    bias = np.zeros(256, np.float32)
    bias[40:48] = 10.0
    ids, w = orc.route(logits, 8, 4, 8, bias=bias)
    s = orc.sigmoid(logits)
    for t in range(64):
        assert sorted(ids[t]) == list(range(40, 48))
        sel = (s[t] + bias).astype(np.float32)
        assert list(ids[t]) == sorted(range(40, 48), key=lambda e: (-sel[e], e))
