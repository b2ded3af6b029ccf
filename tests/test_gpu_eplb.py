"""The balancer's loop on the GPU, at the prefill rank shape (256 logical
experts in 288 slots, 4 nodes x 8 GPUs, Zipf(1.1) popularity): the router
runs on the device, the dispatch recorder (rdg_layout.expert_load) measures
each expert's load, rdg_eplb_place turns it into a placement (checked against
the placement oracle), and rdg_eplb_remap applies it to the same batch for
every rank (checked against the remap oracle).  The pages' claim that
rebalancing raises the balance (mean over maximum of the GPUs' loads;
"Large-scale EP ..." page, section "EPLB: redundant experts and
rebalancing") is checked on the rows each rank then receives."""
import numpy as np
import pytest
import torch

import oracle
import synth
from oracle import eplb
from harness import DEV, np_of, rdg

pytestmark = pytest.mark.gpu


def test_rebalance_loop():
    m = rdg()
    cfg = dict(synth.WORKLOADS["prefill_rank_fp8"])
    B, K, N = 8192, cfg["K"], cfg["N"]
    n_ranks, n_local, n_nodes = cfg["n_ranks"], cfg["n_local"], 4
    n_phys = n_ranks * n_local
    logits = synth.logits(cfg, B)
    ids = torch.empty((B, K), dtype=torch.int32, device=DEV)
    w = torch.empty((B, K), dtype=torch.float32, device=DEV)
    m.rdg_route(torch.from_numpy(logits).to(DEV), cfg["n_group"], cfg["topk_group"], K, cfg["scale"], ids, w)
    ri, _ = oracle.route(logits, cfg["n_group"], cfg["topk_group"], K, cfg["scale"])
    assert np.array_equal(np_of(ids), ri)

    # the load estimator: dispatch over all logical experts, recorder on
    load = torch.zeros(N, dtype=torch.int64, device=DEV)
    L = m.Layout(m.RDG_CONTIGUOUS, N, B, K, DEV, block_m=16, expert_load=load)
    x = torch.zeros((B, 128), dtype=torch.bfloat16, device=DEV)
    xp = torch.empty((L.m_cap, 128), dtype=torch.bfloat16, device=DEV)
    m.rdg_dispatch(x, None, m.RDG_BF16, ids, L, xp)
    assert m.rdg_check_status(L) == (0, 0)
    counts = np_of(load)
    assert np.array_equal(counts, np.bincount(ri.ravel(), minlength=N))

    # placement, native and oracle
    ref = eplb.place(list(counts.astype(np.float64)), cfg["n_group"], n_nodes, n_ranks, n_phys)
    r_max = max(ref["n_replica"])
    phy2log, log2phy, n_rep, gpu_load = m.rdg_eplb_place(counts, cfg["n_group"], n_nodes, n_ranks, n_phys, r_max)
    assert phy2log.tolist() == ref["phy2log"] and n_rep.tolist() == ref["n_replica"]
    assert gpu_load.tolist() == ref["gpu_load"]

    # apply it: every rank's received rows
    gidx = np.arange(B, dtype=np.int64)
    gidx_d, l2p_d, nrep_d = (torch.from_numpy(a).to(DEV) for a in (gidx, log2phy, n_rep))
    loc = torch.empty_like(ids)
    rows = np.zeros(n_ranks)
    for r in range(n_ranks):
        m.rdg_eplb_remap(ids, gidx_d, l2p_d, nrep_d, r * n_local, n_local, loc)
        got = np_of(loc)
        if r in (0, n_ranks - 1) or r == int(np.argmax(ref["gpu_load"])):
            assert np.array_equal(got, oracle.eplb_remap(ri, gidx, log2phy, n_rep, r * n_local, n_local))
        rows[r] = (got >= 0).sum()
    assert rows.sum() == B * K
    # the rows follow the placement's predicted loads, and the balance rises
    # over the static placement (experts e in [8r, 8r + 8) on rank r)
    assert np.allclose(rows, gpu_load, rtol=0.05, atol=8)
    static = counts.reshape(n_ranks, N // n_ranks).sum(1)
    bal = rows.mean() / rows.max()
    bal_static = static.mean() / static.max()
    print("balance: static %.3f  rebalanced %.3f" % (bal_static, bal), flush=True)
    assert bal > bal_static + 0.2
