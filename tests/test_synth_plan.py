"""The EPLB plans of the rank-share workloads (workload preparation, not a
hot-path step): the greedy replica rule is pinned by brute force on small
cases and the whole plan against the placement oracle run flat (one node)
on the same expected loads; the one-extra-copy variant by its definition.
("Large-scale EP: DeepEP, EPLB and two-batch overlap", section "EPLB":
256 logical experts in 288 physical slots, popular experts replicated, each
copy taking a share of the load.)"""
import itertools

import numpy as np
import pytest

import synth
from oracle import eplb


@pytest.mark.parametrize("seed", range(6))
def test_greedy_replicas_minimise_the_largest_load_per_copy(seed):
    rng = np.random.default_rng(700 + seed)
    N, extra = 5, 4
    pop = rng.random(N) ** 3
    got = synth.replica_counts(pop, extra, "greedy")
    assert got.sum() == N + extra and got.min() >= 1
    best = min(max(pop[e] / (1 + c[e]) for e in range(N))
               for c in itertools.product(range(extra + 1), repeat=N) if sum(c) == extra)
    assert max(pop / got) == best


def test_greedy_ties_go_to_the_lower_id():
    pop = np.array([1.0, 2.0, 2.0, 1.0])
    # 2 -> e1 (2 vs 2, lower id); then e2 (2 > 1); then e0 (1 vs 1 vs 1, lowest)
    assert synth.replica_counts(pop, 3, "greedy").tolist() == [2, 2, 2, 1]


def test_one_extra_copy_variant():
    pop = np.array([0.1, 0.4, 0.3, 0.4, 0.05])
    assert synth.replica_counts(pop, 2, "one_each").tolist() == [1, 2, 1, 2, 1]


@pytest.mark.parametrize("name", ["decode_rank_fp8", "prefill_rank_fp8"])
@pytest.mark.parametrize("rule", ["greedy", "one_each"])
def test_plan_matches_the_flat_placement_oracle(name, rule):
    cfg = synth.WORKLOADS[name]
    plan = synth.eplb_plan(cfg, rule)
    pop = synth.expected_popularity(cfg)
    n_gpus = cfg["n_ranks"]
    n_phys = n_gpus * cfg["n_local"]
    assert plan["n_replica"].sum() == n_phys
    if rule == "greedy":
        # the oracle's flat placement applies the same replica rule to the same loads
        ref = eplb.place(pop.tolist(), n_groups=1, n_nodes=1, n_gpus=n_gpus, n_physical=n_phys)
        assert plan["n_replica"].tolist() == ref["n_replica"]
        for e in range(cfg["N"]):
            assert plan["log2phy"][e, :plan["n_replica"][e]].tolist() == ref["log2phy"][e]
        assert np.array_equal(plan["load"], np.array(ref["gpu_load"]))
    # every physical slot holds exactly one copy, and each rank n_local of them
    slots = np.concatenate([plan["log2phy"][e, :plan["n_replica"][e]] for e in range(cfg["N"])])
    assert sorted(slots.tolist()) == list(range(n_phys))
    # the measured rank is the one with the highest expected load (ties: lower rank)
    assert plan["bottleneck"] == int(np.argmax(plan["load"]))
    assert plan["phys_begin"] == plan["bottleneck"] * cfg["n_local"]


def test_greedy_plan_is_better_balanced():
    for name in ("decode_rank_fp8", "prefill_rank_fp8"):
        cfg = synth.WORKLOADS[name]
        g = synth.eplb_plan(cfg, "greedy")["load"]
        o = synth.eplb_plan(cfg, "one_each")["load"]
        assert g.max() < o.max()
