"""The work partition between the polling combine and its finishing form,
explored over every interleaving (DeepGEMM single-batch-overlap pull
request, section 2: the consumer takes each block of rows once its counter
is complete; here a few polling waves take the blocks that complete early
and the finishing form the rest).

The polling waves each repeat: claimed = fetch_add(counter, CH); stop if
claimed < 0 or claimed >= n_units, else combine the units [claimed,
min(claimed + CH, n_units)).  The kernel claims one unit at a time (CH = 1);
claims of several units are explored as well, since the partition rule does
not depend on CH.  The
finishing form does old = fetch_add(counter, CLOSED) once, sets
start = old if 0 <= old < n_units else n_units, and combines every unit
u >= start.  Counters are 32-bit and wrap.  Atomic adds are linearisable, so
an execution is an interleaving of these adds; every interleaving of a few
waves, one or more closes and small unit counts is explored, and each must
combine every unit exactly once.  Seeded mistakes (an off-by-one start, a
missing per-unit range test, a close that does not stop the waves, a start
rule without its sign test, a start rounded to a chunk boundary) are caught,
so the model can fail."""
import pytest

CLOSED = 1 << 30


def wrap32(v):
    v &= 0xFFFFFFFF
    return v - (1 << 32) if v >= (1 << 31) else v


def kernel_start(old, n_units):
    return old if 0 <= old < n_units else n_units


def explore(n_units, n_waves, closes=1, start_rule=kernel_start, stop_rule=None, close_add=CLOSED, chunk=1,
            clip=True):
    """Yields, for every schedule, the (unit, who) pairs combined."""
    stop_rule = stop_rule or (lambda c: c < 0 or c >= n_units)

    def run(counter, live, closes_left, done):
        moves = [i for i in range(n_waves) if live[i]] + (["close"] if closes_left else [])
        if not moves:
            yield done
            return
        for m in moves:
            if m != "close":
                claimed = counter
                nl = list(live)
                nd = done
                if stop_rule(claimed):
                    nl[m] = False
                else:
                    end = min(claimed + chunk, n_units) if clip else claimed + chunk
                    nd = done + tuple((u, "wave%d" % m) for u in range(claimed, end))
                yield from run(wrap32(counter + chunk), tuple(nl), closes_left, nd)
            else:
                s = start_rule(counter, n_units)
                nd = done + tuple((u, "finish%d" % closes_left) for u in range(n_units) if u >= s)
                yield from run(wrap32(counter + close_add), live, closes_left - 1, nd)

    yield from run(0, tuple([True] * n_waves), closes, ())


def all_exactly_once(n_units, n_waves, **kw):
    count = 0
    for done in explore(n_units, n_waves, **kw):
        count += 1
        if sorted(u for u, _ in done) != list(range(n_units)):
            return False, done, count
    return True, None, count


@pytest.mark.parametrize("n_units,n_waves", [(0, 1), (1, 1), (1, 2), (2, 2), (3, 2), (4, 2), (3, 3), (5, 2)])
def test_every_unit_exactly_once(n_units, n_waves):
    ok, bad, count = all_exactly_once(n_units, n_waves)
    assert ok, bad
    assert count > 1


@pytest.mark.parametrize("n_units,n_waves,chunk", [(5, 2, 2), (7, 2, 3), (4, 3, 2), (6, 2, 4), (3, 2, 8)])
def test_chunked_claims_every_unit_exactly_once(n_units, n_waves, chunk):
    ok, bad, count = all_exactly_once(n_units, n_waves, chunk=chunk)
    assert ok, bad
    ok, bad, _ = all_exactly_once(n_units, n_waves, chunk=chunk, closes=0)
    assert ok, bad
    ok, bad, _ = all_exactly_once(n_units, n_waves, chunk=chunk, closes=3)
    assert ok, bad


def test_chunked_claims_with_a_start_inside_a_chunk_are_caught():
    # a close that took the counter's value rounded down to a chunk boundary
    # would hand the finishing form units a wave already holds
    ok, _, _ = all_exactly_once(5, 2, chunk=2, start_rule=lambda old, n: min(old - old % 4, n) if old >= 0 else n)
    assert not ok


@pytest.mark.parametrize("n_units,n_waves", [(2, 2), (3, 2)])
def test_polling_alone_covers_everything(n_units, n_waves):
    ok, bad, _ = all_exactly_once(n_units, n_waves, closes=0)
    assert ok, bad


@pytest.mark.parametrize("closes", [2, 3])
def test_repeated_closes_still_partition(closes):
    # the second close takes the counter to 2^31 and past (wrapped negative):
    # waves then stop (claimed < 0), and every later close finds its old
    # value at least CLOSED or negative, and takes nothing
    ok, bad, _ = all_exactly_once(3, 2, closes=closes)
    assert ok, bad


@pytest.mark.parametrize("mistake", ["start_one_late", "start_one_early", "no_exhaustion_test", "close_adds_one",
                                     "start_without_sign_test"])
def test_seeded_mistakes_are_caught(mistake):
    n_units, n_waves, closes = 3, 2, 1
    kw = {}
    if mistake == "start_one_late":
        kw["start_rule"] = lambda old, n: min(old + 1, n)
    elif mistake == "start_one_early":
        kw["start_rule"] = lambda old, n: max(min(old, n) - 1, 0)
    elif mistake == "no_exhaustion_test":
        # no per-unit test against n_units (the kernel's lanes each check
        # theirs): a wave whose claim ends past the units combines phantoms
        kw["stop_rule"] = lambda c: c < 0 or c > n_units
        kw["clip"] = False
        kw["chunk"] = 2
    elif mistake == "close_adds_one":
        kw["close_add"] = 1
    elif mistake == "start_without_sign_test":
        kw["start_rule"] = lambda old, n: min(old, n)
        closes = 3  # the third close sees the wrapped, negative counter
    ok, _, _ = all_exactly_once(n_units, n_waves, closes=closes, **kw)
    assert not ok


def test_the_exploration_branches():
    # schedules differ in who combines what: the close first (the finishing
    # form takes everything), last (the waves take everything), or between
    parts = {tuple(sorted(d)) for d in explore(2, 1)}
    assert ((0, "finish1"), (1, "finish1")) in parts
    assert ((0, "wave0"), (1, "wave0")) in parts
    assert ((0, "wave0"), (1, "finish1")) in parts
    assert sum(1 for _ in explore(3, 2)) > 20
