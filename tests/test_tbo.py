"""Two-batch-overlap split: the oracle against worked cases of the pages'
rule ("Large-scale EP ..." page, TBO section and its split-point exercise),
and the library's rdg_tbo_split against the oracle."""
import numpy as np
import pytest

from oracle import tbo


def test_worked_cases():
    assert tbo.split([2048, 2048]) == 1            # the prefill layer's two sequences: an even cut
    assert tbo.split([100, 300, 200]) == 2         # 400 | 200 beats 100 | 500
    assert tbo.split([5, 5, 5, 5, 4]) == 2         # 10 | 14 (gap 4) beats 15 | 9 (gap 6)
    assert tbo.split([1, 2, 1]) == 1               # 1 | 3 and 3 | 1 tie: the earlier cut
    assert tbo.split([10000, 1, 1]) == 1           # never inside a sequence: unequal halves
    assert tbo.split([7]) == 0 and tbo.split([]) == 0
    assert tbo.split([1] * 9, decode=True) == 4    # decode: half the requests


@pytest.mark.parametrize("seed", range(20))
def test_cut_is_a_best_sequence_boundary(seed):
    # exhaustive over the boundaries: no other cut is closer to half
    rng = np.random.default_rng(seed)
    lens = [int(v) for v in rng.integers(0, 5000, size=int(rng.integers(2, 12)))]
    i = tbo.split(lens)
    total = sum(lens)
    assert 1 <= i < len(lens)
    for j in range(1, len(lens)):
        assert abs(2 * sum(lens[:i]) - total) <= abs(2 * sum(lens[:j]) - total)


@pytest.mark.parametrize("seed", range(30))
def test_library_matches_oracle(seed):
    import routing_dispatch_grouped_amd as m
    rng = np.random.default_rng(100 + seed)
    n = int(rng.integers(0, 40))
    lens = [int(v) for v in rng.integers(0, 4 if seed % 3 == 0 else 9000, size=n)]
    for decode in (False, True):
        assert m.rdg_tbo_split(lens, decode) == tbo.split(lens, decode)


def test_library_rejects_negative_lengths():
    import routing_dispatch_grouped_amd as m
    with pytest.raises(m.RdgError):
        m.rdg_tbo_split([3, -1, 2])
