"""Pins for the oracle's dispatch layouts and EPLB remap: library
reductions (bincount, stable argsort, cumsum), bijection invariants, the
capacity conventions, and the replica-share statistics."""
import numpy as np
import pytest


def _ids(rng, T, K, E, skew=False, holes=0.0):
    out = np.empty((T, K), np.int32)
    p = None
    if skew:
        p = 1.0 / np.arange(1, E + 1) ** 1.1
        p /= p.sum()
    for t in range(T):
        out[t] = rng.choice(E, size=K, replace=False, p=p)
    if holes:
        out[rng.random((T, K)) < holes] = -1
    return out


@pytest.mark.parametrize("T,K,E,block_m,skew,holes", [
    (64, 4, 16, 16, False, 0.0), (300, 8, 37, 32, True, 0.0), (257, 8, 64, 64, True, 0.3),
    (1, 1, 1, 16, False, 0.0), (5, 2, 9, 128, False, 0.5), (0, 8, 4, 16, False, 0.0)])
def test_contiguous_layout(orc, T, K, E, block_m, skew, holes):
    rng = np.random.default_rng([T, K, E])
    ids = _ids(rng, T, K, E, skew, holes)
    L = orc.layout(ids, E, orc.CONTIGUOUS, block_m=block_m)
    assert L["status"] == orc.OK
    flat = ids.ravel()
    local = flat[flat >= 0]
    counts = np.bincount(local, minlength=E)
    assert np.array_equal(L["counts"], counts)
    padded = (counts + block_m - 1) // block_m * block_m
    assert np.array_equal(L["offsets"], np.concatenate([[0], np.cumsum(padded)]))
    assert np.array_equal(L["masked_m"], counts)
    # stable order by expert: numpy's stable argsort of the flat ids
    order = np.argsort(np.where(flat >= 0, flat, E), kind="stable")[:len(local)]
    want = np.full(flat.shape, -1, np.int64)
    for e in range(E):
        rows = order[int(counts[:e].sum()):int(counts[:e + 1].sum())]
        want[rows] = L["offsets"][e] + np.arange(len(rows))
    assert np.array_equal(L["pos"].ravel(), want)
    # bijection between local rows and non-padding slots
    rs = L["row_src"]
    assert len(rs) == T * K + E * (block_m - 1)
    filled = np.flatnonzero(rs >= 0)
    assert len(filled) == len(local)
    assert np.array_equal(L["pos"].ravel()[rs[filled]], filled)


@pytest.mark.parametrize("m_max", [256, 7, 1])
def test_masked_layout_and_capacity(orc, m_max):
    rng = np.random.default_rng(m_max)
    T, K, E = 128, 8, 32
    ids = _ids(rng, T, K, E, skew=True)
    L = orc.layout(ids, E, orc.MASKED, m_max=m_max)
    counts = np.bincount(ids.ravel(), minlength=E)
    assert np.array_equal(L["counts"], counts)
    assert np.array_equal(L["masked_m"], np.minimum(counts, m_max))
    assert np.array_equal(L["offsets"], np.arange(E + 1) * m_max)
    over = counts.max() > m_max
    # exceeding the preallocated rows is an error carrying the largest count
    assert L["status"] == (orc.ECAPACITY if over else orc.OK)
    if over:
        assert L["detail"] == counts.max()
    flat = ids.ravel()
    for e in range(E):
        rows = np.flatnonzero(flat == e)
        kept, dropped = rows[:m_max], rows[m_max:]
        assert np.array_equal(L["pos"].ravel()[kept], e * m_max + np.arange(len(kept)))
        assert np.all(L["pos"].ravel()[dropped] == -1)
        seg = L["row_src"][e * m_max:(e + 1) * m_max]
        assert np.array_equal(seg[:len(kept)], kept) and np.all(seg[len(kept):] == -1)


def test_contiguous_capacity_overflow(orc):
    rng = np.random.default_rng(9)
    ids = _ids(rng, 100, 4, 8)
    full = orc.layout(ids, 8, orc.CONTIGUOUS, block_m=16)
    need = int(full["offsets"][-1])
    small = orc.layout(ids, 8, orc.CONTIGUOUS, block_m=16, m_cap=need - 40)
    assert small["status"] == orc.ECAPACITY and small["detail"] == need
    pos = small["pos"].ravel()
    assert pos.max() < need - 40
    kept = pos >= 0
    assert np.array_equal(pos[kept], full["pos"].ravel()[kept])


def test_remap_identity_and_shares(orc):
    rng = np.random.default_rng(4)
    T, K, N = 4000, 8, 32
    ids = _ids(rng, T, K, N)
    gidx = np.arange(T, dtype=np.int64) + 12345
    # one replica each, identity placement over a single "rank" -> identity
    l2p = np.stack([np.arange(N), np.arange(N)], 1).astype(np.int32)
    out = orc.eplb_remap(ids, gidx, l2p, np.ones(N, np.int32), 0, N)
    assert np.array_equal(out, ids)
    # two replicas for experts 0..7 on physical ids N..N+7; rank range splits
    nrep = np.ones(N, np.int32)
    nrep[:8] = 2
    l2p[:8, 1] = N + np.arange(8)
    both = [orc.eplb_remap(ids, gidx, l2p, nrep, b, n) for b, n in [(0, N), (N, 8)]]
    for e in range(8):
        rows = ids == e
        a = (both[0][rows] == e).sum()
        b = (both[1][rows] == e).sum()
        assert a + b == rows.sum()          # every row goes to exactly one replica
        assert abs(a - b) <= 1 + 4 * np.sqrt(rows.sum())  # an even split
    # the choice is token-keyed: all rows of one token use the same parity
    par = (gidx % 2).astype(bool)
    sel = ids[par] < 8
    assert np.all(both[1][par][sel] >= 0)
    # -1 input stays -1; ids outside the local range become -1
    ids2 = ids.copy()
    ids2[:, 0] = -1
    out2 = orc.eplb_remap(ids2, gidx, l2p, nrep, 0, 16)
    assert np.all(out2[:, 0] == -1)
    assert np.all((out2 == -1) | ((out2 >= 0) & (out2 < 16)))
