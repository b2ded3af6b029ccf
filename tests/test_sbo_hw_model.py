"""Operational model of the single-batch-overlap hand-off (signalled down
GEMM -> polling combine; DeepGEMM single-batch-overlap pull request, section
2: a counter per block of rows, incremented once part of the work is done
and polled by the consumer up to a threshold; section 3: the increment is
release-ordered), under the cache rules of this GPU, explored exhaustively.

C11 has no memory scopes and ThreadSanitizer does not follow standalone
fences, so the TSan model (test_sbo_model.py) checks the C11 counterpart of
the protocol (an acquire load of the counter).  The kernels do something C11
cannot state: the producer stores its rows with relaxed device-scope stores,
waits for them to complete and adds to the counter (relaxed, device scope)
with no fence; the consumer polls with relaxed device-scope loads, issues
only a workgroup-scope fence, and reads the rows with relaxed device-scope
loads.  Their correctness rests on these rules of the GPU, which this model
states as its semantics:

* each XCD has its own write-back L2; plain stores land there (dirty) and
  plain loads are served from it when the line is present, possibly stale;
* device-scope stores are written through to memory, and a wave's wait for
  its stores to complete returns once memory holds them; an add issued
  after that wait is performed at memory after them;
* a device-scope release fence writes the XCD's dirty lines back to memory
  (the alternative for plain stores; it costs a write-back of the L2);
* device-scope loads (the polls, and the combine's row loads) read memory,
  never a possibly stale L2 line, and a load issued after an earlier load
  has returned sees memory at least as new as that load did (the consumer
  issues its row loads only once the poll's value has arrived).

Two producer workgroups on two XCDs each store half of a row tile and
publish; the consumer, on a third XCD whose L2 holds stale copies of the
rows, waits until the counter reaches 2 and reads both halves.  Caches may
evict at any moment.  Every interleaving is explored.  The protocol as
shipped never reads a stale value, and neither does the plain-store
protocol with a release write-back; plain stores without it, or reading the
rows with plain loads, do -- so the model can fail -- and plain loads after a
device-scope acquire (an L2 invalidation) are again correct."""

import pytest

Y = ("y0", "y1")      # the two halves of the row tile
P_XCD = (0, 2)        # producer workgroups' XCDs
C_XCD = 1             # consumer's XCD


def _explore(stores="device", row_loads="device", acquire=False):
    """All final consumer readings (tuple of the two halves' values).
    stores: "device" (write-through, completed before the add), "release"
    (plain stores, then an L2 write-back before the add) or "plain" (plain
    stores, nothing else)."""
    # state: (mem, l2 per xcd as frozenset of (loc, value, dirty)), producer pcs, consumer pc, regs
    mem0 = (("s", 0), ("y0", 0), ("y1", 0))
    l2_0 = {0: frozenset(), 1: frozenset({("y0", 0, False), ("y1", 0, False)}), 2: frozenset()}
    start = (mem0, tuple(sorted(l2_0.items())), (0, 0), 0, ())
    finals = set()
    seen = set()
    stack = [start]

    def get(mem, loc):
        return dict(mem)[loc]

    def put(mem, loc, v):
        d = dict(mem)
        d[loc] = v
        return tuple(sorted(d.items()))

    def l2get(l2, x, loc):
        for (l, v, dirty) in dict(l2)[x]:
            if l == loc:
                return v
        return None

    def l2set(l2, x, line):
        d = dict(l2)
        d[x] = frozenset({e for e in d[x] if e[0] != line[0]} | {line})
        return tuple(sorted(d.items()))

    def l2drop(l2, x, loc):
        d = dict(l2)
        d[x] = frozenset(e for e in d[x] if e[0] != loc)
        return tuple(sorted(d.items()))

    while stack:
        st = stack.pop()
        if st in seen:
            continue
        seen.add(st)
        mem, l2, ppc, cpc, regs = st
        nxt = []
        # producers: store own half -> (release: write back own L2) -> add to counter at memory
        for i, x in enumerate(P_XCD):
            pc = ppc[i]
            steps = {"device": ["store_dev", "add"], "release": ["store", "release", "add"],
                     "plain": ["store", "add"]}[stores]
            if pc >= len(steps):
                continue
            op = steps[pc]
            npc = tuple(pc + 1 if j == i else p for j, p in enumerate(ppc))
            if op == "store":
                nxt.append((mem, l2set(l2, x, (Y[i], 1, True)), npc, cpc, regs))
            elif op == "store_dev":   # written through; completion (the wait before the add) = in memory
                nxt.append((put(mem, Y[i], 1), l2drop(l2, x, Y[i]), npc, cpc, regs))
            elif op == "release":
                m, c = mem, l2
                for (loc, v, dirty) in dict(l2)[x]:
                    if dirty:
                        m = put(m, loc, v)
                        c = l2set(c, x, (loc, v, False))
                nxt.append((m, c, npc, cpc, regs))
            else:
                nxt.append((put(mem, "s", get(mem, "s") + 1), l2, npc, cpc, regs))
        # consumer: poll until 2, (acquire: invalidate own L2), then read both halves
        if cpc == 0:
            if get(mem, "s") >= 2:
                nxt.append((mem, l2, ppc, 1, regs))
            else:
                nxt.append((mem, l2, ppc, 0, regs))   # poll again (a self-loop, pruned by `seen`)
        elif cpc == 1:
            c = l2
            if acquire:
                for (loc, v, dirty) in dict(l2)[C_XCD]:
                    c = l2drop(c, C_XCD, loc)
            nxt.append((mem, c, ppc, 2, regs))
        elif cpc in (2, 3):
            loc = Y[cpc - 2]
            if row_loads == "device":
                v, c = get(mem, loc), l2
            else:
                v = l2get(l2, C_XCD, loc)
                c = l2
                if v is None:
                    v = get(mem, loc)
                    c = l2set(l2, C_XCD, (loc, v, False))
            nxt.append((mem, c, ppc, cpc + 1, regs + (v,)))
        else:
            finals.add(regs)
        # the environment: any XCD writes back or evicts any line at any time
        for x in (0, 1, 2):
            for (loc, v, dirty) in dict(l2)[x]:
                m = put(mem, loc, v) if dirty else mem
                nxt.append((m, l2drop(l2, x, loc), ppc, cpc, regs))
        stack.extend(nxt)
    return finals


@pytest.mark.parametrize("stores", ["device", "release"])
def test_protocols_never_read_stale_rows(stores):
    # "device": the shipped protocol; "release": plain stores and a release
    assert _explore(stores=stores, row_loads="device") == {(1, 1)}


@pytest.mark.parametrize("stores,row_loads", [("plain", "device"), ("device", "plain"), ("release", "plain")])
def test_model_catches_a_broken_protocol(stores, row_loads):
    finals = _explore(stores=stores, row_loads=row_loads)
    assert any(v != (1, 1) for v in finals), finals


def test_plain_loads_after_a_device_scope_acquire_are_correct():
    assert _explore(stores="device", row_loads="plain", acquire=True) == {(1, 1)}
