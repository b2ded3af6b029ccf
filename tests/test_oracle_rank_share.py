"""Pin for the rank-share reading: with EPLB replicas spread over ranks, the
partial combines of all ranks add up to the full layer's routed output."""
import numpy as np


def test_rank_shares_sum_to_full_layer(orc):
    rng = np.random.default_rng(50)
    N, K, H, I, Tg = 16, 4, 256, 128, 160
    n_ranks, n_local = 5, 4  # 20 physical slots = 16 logical + 4 replicas
    logits = rng.standard_normal((Tg, N)).astype(np.float32)
    ids, w = orc.route(logits, 4, 2, K)
    # hand-made placement: logical e on physical e; replicas of 0..3 on 16..19
    l2p = np.stack([np.arange(N), np.arange(N)], 1).astype(np.int32)
    nrep = np.ones(N, np.int32)
    nrep[:4] = 2
    l2p[:4, 1] = 16 + np.arange(4)
    phys2log = np.empty(n_ranks * n_local, np.int64)
    for e in range(N):
        for r in range(nrep[e]):
            phys2log[l2p[e, r]] = e
    weights = [dict(W1=(rng.standard_normal((I, H)) * 0.05).astype(np.float32),
                    W3=(rng.standard_normal((I, H)) * 0.05).astype(np.float32),
                    W2=(rng.standard_normal((H, I)) * 0.05).astype(np.float32)) for _ in range(N)]
    x = rng.standard_normal((Tg, H)).astype(np.float32)
    gidx = np.arange(Tg, dtype=np.int64)
    full = orc.moe_layer(orc.F32, x, ids, w, weights)
    total = np.zeros((Tg, H))
    rows = 0
    for r in range(n_ranks):
        loc = orc.eplb_remap(ids, gidx, l2p, nrep, r * n_local, n_local)
        rows += int((loc >= 0).sum())
        ex = [weights[phys2log[r * n_local + s]] for s in range(n_local)]
        total += orc.moe_layer(orc.F32, x, loc, w, ex).astype(np.float64)
    assert rows == Tg * K  # every row lands on exactly one rank
    assert orc.rel_err(total, full) <= 1e-6
