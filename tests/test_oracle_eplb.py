"""Pins of the EPLB placement oracle (oracle/eplb.py) against what holds
independently of it: hand-worked examples of the stated rules, brute force
for the replica step, structural invariants, and the pages' claim that the
balancer raises the balance statistic ("Large-scale EP ..." page, section
"EPLB: redundant experts and rebalancing"; H100 deployment article, section
"Expert-parallel load balancer")."""
import itertools

import numpy as np
import pytest

from oracle import eplb


def test_worked_example_hierarchical():
    # 8 experts in 4 groups of 2, 2 nodes x 2 GPUs x 3 slots.
    # loads 10 2 | 6 6 | 1 1 | 9 5  -> group loads 12 12 2 14
    # groups by load: g3 (14), g0 (12, tie with g1: lower id first), g1, g2
    #   g3 -> node0 (both empty, lower id); g0 -> node1; g1 -> node1 (12 < 14,
    #   node1 then full); g2 -> node0
    # node0 = experts 4 5 6 7, two extra slots: e6 (9) then e7 (5 > 4.5)
    #   copies 4.5 4.5 2.5 2.5 1 1 alternate GPU0/GPU1 on ties:
    #   GPU0 = e6 e7 e4 (8), GPU1 = e6 e7 e5 (8)
    # node1 = experts 0 1 2 3, extra slots: e0 (10), then e2 (6, tie e3)
    #   copies (6,e3) (5,e0) (5,e0) (3,e2) (3,e2) (2,e1):
    #   GPU2 <- e3 (6); GPU3 <- e0 (5); GPU3 <- e0 (10); GPU2 <- e2 (9);
    #   GPU2 <- e2 (12, full); GPU3 <- e1 (12)
    r = eplb.place([10, 2, 6, 6, 1, 1, 9, 5], n_groups=4, n_nodes=2, n_gpus=4, n_physical=12)
    assert r["hierarchical"]
    assert r["phy2log"] == [6, 7, 4, 6, 7, 5, 3, 2, 2, 0, 0, 1]
    assert r["log2phy"] == [[9, 10], [11], [7, 8], [6], [2], [5], [0, 3], [1, 4]]
    assert r["n_replica"] == [2, 1, 2, 1, 1, 1, 2, 2]
    assert r["gpu_load"] == [8.0, 8.0, 12.0, 12.0]
    assert eplb.balance(r["gpu_load"]) == pytest.approx(10.0 / 12.0)


def test_worked_example_flat():
    # 3 groups cannot be spread evenly over 2 nodes: one node of 2 GPUs x 2
    # slots.  loads 3 1 2; the extra slot goes to e0 (copies of 1.5).
    # copies (2,e2) (1.5,e0) (1.5,e0) (1,e1): GPU0 <- e2; GPU1 <- e0;
    # GPU1 <- e0 (1.5 < 2; GPU1 full); GPU0 <- e1
    r = eplb.place([3, 1, 2], n_groups=3, n_nodes=2, n_gpus=2, n_physical=4)
    assert not r["hierarchical"]
    assert r["phy2log"] == [2, 1, 0, 0]
    assert r["log2phy"] == [[2, 3], [1], [0]]
    assert r["gpu_load"] == [3.0, 3.0]


def _compositions(total, parts):
    """All tuples of `parts` integers >= 1 summing to `total`."""
    for cut in itertools.combinations(range(1, total), parts - 1):
        b = (0,) + cut + (total,)
        yield tuple(b[i + 1] - b[i] for i in range(parts))


@pytest.mark.parametrize("seed", range(12))
def test_replicas_minimise_the_largest_load_per_copy(seed):
    # one node, one GPU: only the replica step acts; brute force over every
    # split of the slots gives the smallest achievable max(load / copies)
    rng = np.random.default_rng(seed)
    N = int(rng.integers(1, 5))
    S = N + int(rng.integers(0, 4))
    load = [float(v) for v in rng.integers(0, 20, size=N)]
    r = eplb.place(load, n_groups=1, n_nodes=1, n_gpus=1, n_physical=S)
    got = max(load[e] / r["n_replica"][e] for e in range(N))
    best = min(max(load[e] / c[e] for e in range(N)) for c in _compositions(S, N))
    assert got == best
    assert sum(r["n_replica"]) == S


def _check_structure(r, N, n_groups, n_gpus, n_physical, load):
    spg = n_physical // n_gpus
    phy2log = r["phy2log"]
    assert len(phy2log) == n_physical and min(phy2log) >= 0
    for e in range(N):
        assert r["n_replica"][e] >= 1
        assert len(r["log2phy"][e]) == r["n_replica"][e]
        assert sorted(r["log2phy"][e]) == [p for p in range(n_physical) if phy2log[p] == e]
    # each GPU's load is the sum of its copies' loads
    for g in range(n_gpus):
        s = sum(load[phy2log[p]] / r["n_replica"][phy2log[p]] for p in range(g * spg, (g + 1) * spg))
        assert r["gpu_load"][g] == pytest.approx(s, rel=1e-12, abs=1e-9)
    assert sum(r["gpu_load"]) == pytest.approx(sum(load), rel=1e-12)


@pytest.mark.parametrize("shape", [(256, 8, 4, 32, 288), (256, 8, 9, 72, 288), (256, 8, 1, 8, 256),
                                   (64, 8, 2, 6, 72), (16, 4, 2, 4, 24)])
def test_structure_and_locality(shape):
    N, G, nodes, gpus, phys = shape
    rng = np.random.default_rng(sum(shape))
    load = list(rng.zipf(1.6, size=N).astype(float))
    r = eplb.place(load, G, nodes, gpus, phys)
    _check_structure(r, N, G, gpus, phys, load)
    if r["hierarchical"]:
        # every copy of a group's experts sits on one node
        gpn, spg, per_group = gpus // nodes, phys // gpus, N // G
        for g in range(G):
            node_set = {p // spg // gpn for e in range(g * per_group, (g + 1) * per_group) for p in r["log2phy"][e]}
            assert len(node_set) == 1
        # and each node holds the same number of groups
        counts = np.bincount([r["log2phy"][g * per_group][0] // spg // gpn for g in range(G)], minlength=nodes)
        assert (counts == G // nodes).all()


def test_equal_loads_fill_gpus_evenly():
    # equal loads, no redundancy: copies alternate over the GPUs in id order
    r = eplb.place([1.0] * 8, n_groups=1, n_nodes=1, n_gpus=4, n_physical=8)
    assert r["phy2log"] == [0, 4, 1, 5, 2, 6, 3, 7]
    assert r["gpu_load"] == [2.0] * 4


@pytest.mark.parametrize("nodes,gpus", [(4, 32), (9, 72)])
def test_balancer_raises_balance_under_zipf(nodes, gpus):
    # Zipf(1.1) popularity over a permutation (the prefill workloads' skew):
    # the balancer's placement beats the static one (expert e on GPU e // per)
    # -- the effect the pages measure
    N, phys = 256, 288
    rng = np.random.default_rng(7)
    pop = 1.0 / np.arange(1, N + 1) ** 1.1
    load = list((pop[rng.permutation(N)] * 1e6).round())
    static = np.zeros(gpus)
    per = -(-N // gpus)
    for e in range(N):
        static[e // per] += load[e]
    r = eplb.place(load, 8, nodes, gpus, phys)
    assert eplb.balance(r["gpu_load"]) > eplb.balance(list(static)) + 0.2


def test_invalid_shapes():
    with pytest.raises(ValueError):
        eplb.place([1.0] * 10, n_groups=4, n_nodes=1, n_gpus=2, n_physical=12)   # groups do not divide N
    with pytest.raises(ValueError):
        eplb.place([1.0] * 8, n_groups=2, n_nodes=1, n_gpus=2, n_physical=6)     # fewer slots than experts
    with pytest.raises(ValueError):
        eplb.place([1.0] * 8, n_groups=2, n_nodes=2, n_gpus=3, n_physical=12)    # nodes do not divide GPUs
    with pytest.raises(ValueError):
        eplb.place([1.0] * 8, n_groups=2, n_nodes=1, n_gpus=4, n_physical=10)    # GPUs do not divide slots
