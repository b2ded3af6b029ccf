"""The library's EPLB placement (rdg_eplb_place, host code in librdg.so)
against the placement oracle: identical integer outputs and loads on the
pages' shapes (256 logical experts in 288 slots over 32 or 72 GPUs) and on
small shapes with many ties; argument errors as documented."""
import numpy as np
import pytest

from oracle import eplb


def _lib_place(load, G, nodes, gpus, phys, r_max):
    import routing_dispatch_grouped_amd as m
    return m.rdg_eplb_place(np.asarray(load, np.float64), G, nodes, gpus, phys, r_max)


def _loads(kind, N, rng):
    if kind == "zipf":
        pop = 1.0 / np.arange(1, N + 1) ** 1.1
        return (pop[rng.permutation(N)] * 1e5).round()
    if kind == "ties":
        return rng.integers(0, 3, size=N).astype(np.float64)
    if kind == "zeros":
        return np.zeros(N)
    return rng.random(N) * 100.0


@pytest.mark.parametrize("shape", [(256, 8, 4, 32, 288), (256, 8, 9, 72, 288), (256, 8, 1, 8, 256),
                                   (256, 8, 8, 64, 320), (64, 8, 2, 6, 72), (16, 4, 2, 4, 24), (3, 3, 2, 2, 4)])
@pytest.mark.parametrize("kind", ["zipf", "ties", "zeros", "uniform"])
def test_matches_oracle(shape, kind):
    N, G, nodes, gpus, phys = shape
    rng = np.random.default_rng(hash((shape, kind)) % 2**32)
    load = _loads(kind, N, rng)
    ref = eplb.place(list(load), G, nodes, gpus, phys)
    r_max = max(ref["n_replica"])
    phy2log, log2phy, n_rep, gpu_load = _lib_place(load, G, nodes, gpus, phys, r_max)
    assert phy2log.tolist() == ref["phy2log"]
    assert n_rep.tolist() == ref["n_replica"]
    want = np.full((N, r_max), -1, np.int32)
    for e, ps in enumerate(ref["log2phy"]):
        want[e, :len(ps)] = ps
    assert np.array_equal(log2phy, want)
    assert gpu_load.tolist() == ref["gpu_load"]      # same sums in the same order: exact


def test_errors():
    import routing_dispatch_grouped_amd as m
    with pytest.raises(m.RdgError) as ei:
        _lib_place(np.ones(10), 4, 1, 2, 12, 2)       # groups do not divide the experts
    assert ei.value.code == m.RDG_EINVAL
    with pytest.raises(m.RdgError) as ei:
        _lib_place(np.ones(8), 2, 1, 2, 6, 2)         # fewer slots than experts
    assert ei.value.code == m.RDG_EINVAL
    with pytest.raises(m.RdgError) as ei:
        _lib_place(np.array([1.0, -1.0]), 1, 1, 1, 2, 2)   # negative load
    assert ei.value.code == m.RDG_EINVAL
    with pytest.raises(m.RdgError) as ei:
        _lib_place(np.array([1.0, np.nan]), 1, 1, 1, 2, 2)
    assert ei.value.code == m.RDG_EINVAL
    with pytest.raises(m.RdgError) as ei:
        _lib_place(np.array([100.0, 1.0]), 1, 1, 1, 6, 2)  # the hot expert needs 5 copies
    assert ei.value.code == m.RDG_ECAPACITY
