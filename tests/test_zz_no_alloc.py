"""The allocation-free dispatch (rdg_dispatch_noalloc): its scratch lives in
the library's static device array instead of a caller workspace.  Through
the C ABI, two calls in a row -- the second smaller, so that it reuses the
array over stale contents of the first -- must give exactly the outputs of
rdg_dispatch on the same inputs: counts, offsets, masked_m, positions, row
sources, status, the row-tile tables, and the permuted rows and scales.
Entry counts beyond the array's stated maximum are refused."""
import numpy as np
import pytest
import torch

from harness import DEV, np_of, rdg

pytestmark = pytest.mark.gpu


def _layout(m, kind, n_local, T, K, block_m, m_max, tables_only):
    L = m.Layout(kind, n_local, T, K, DEV, block_m=block_m, m_max=m_max)
    if tables_only:
        # the no-allocation call needs only the row-tile tables in layout.work
        nb = m.rdg_layout_tables_bytes(n_local)
        L.work = torch.zeros(nb, dtype=torch.uint8, device=DEV)
        L.c.work = L.work.data_ptr()
    return L


def _case(m, T, K, n_local, H, kind, fp8, seed, block_m=128, m_max=0):
    rng = np.random.default_rng(seed)
    ids_np = rng.integers(-1, n_local, (T, K)).astype(np.int32)
    ids_np[: T // 3, 0] = 0  # a busy expert spanning several row tiles
    ids = torch.from_numpy(ids_np).to(DEV)
    if fp8:
        x = torch.from_numpy(rng.integers(0, 255, (T, H)).astype(np.uint8)).to(DEV)
        xs = torch.from_numpy(rng.random((T, H // 128)).astype(np.float32)).to(DEV)
        dt = m.RDG_FP8_E4M3
    else:
        x = torch.from_numpy(rng.standard_normal((T, H)).astype(np.float32)).to(DEV).to(torch.bfloat16)
        xs = None
        dt = m.RDG_BF16
    out = {}
    for name, fn, tables_only in (("plain", m.rdg_dispatch, False), ("noalloc", m.rdg_dispatch_noalloc, True)):
        L = _layout(m, kind, n_local, T, K, block_m, m_max, tables_only)
        xp = torch.zeros((L.m_cap, H), dtype=x.dtype, device=DEV)
        xps = torch.zeros((L.m_cap, H // 128), dtype=torch.float32, device=DEV) if fp8 else None
        fn(x, xs, dt, ids, L, xp, xps)
        st = m.rdg_check_status(L)
        out[name] = (L, xp, xps, st)
    return out


def _compare(m, out, n_local):
    La, xa, sa, sta = out["plain"]
    Lb, xb, sb, stb = out["noalloc"]
    assert sta == stb
    for f in ("counts", "offsets", "masked_m", "pos", "row_src"):
        assert torch.equal(getattr(La, f), getattr(Lb, f)), f
    nb = m.rdg_layout_tables_bytes(n_local)
    assert torch.equal(La.work[:nb], Lb.work[:nb]), "row-tile tables"
    rows = torch.from_numpy(np.flatnonzero(np_of(La.row_src) >= 0)).to(DEV)
    assert torch.equal(xa[rows].view(torch.uint8), xb[rows].view(torch.uint8)), "permuted rows"
    if sa is not None:
        assert torch.equal(sa[rows], sb[rows]), "permuted scales"


@pytest.mark.parametrize("fp8", [False, True])
@pytest.mark.parametrize("kind", [0, 1])
def test_noalloc_dispatch_matches_dispatch(fp8, kind):
    m = rdg()
    n_local, K, H = 37, 8, 512
    # first call large, second smaller: the second runs over the first's scratch
    for T, seed in ((4100, 1), (300, 2)):
        m_max = T if kind == m.RDG_MASKED else 0
        out = _case(m, T, K, n_local, H, kind, fp8, seed, m_max=m_max)
        _compare(m, out, n_local)
        print("no-alloc dispatch T=%d kind=%d fp8=%s equals rdg_dispatch" % (T, kind, fp8), flush=True)


def test_noalloc_refuses_beyond_its_maximum():
    m = rdg()
    T, K, n_local = (1 << 20) // 8 + 1, 8, 4       # one token past 2^20 entries
    L = _layout(m, m.RDG_CONTIGUOUS, n_local, T, K, 128, 0, True)
    x = torch.empty((T, 16), dtype=torch.bfloat16, device=DEV)
    ids = torch.full((T, K), -1, dtype=torch.int32, device=DEV)
    xp = torch.empty((L.m_cap, 16), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(m.RdgError) as ei:
        m.rdg_dispatch_noalloc(x, None, m.RDG_BF16, ids, L, xp)
    assert ei.value.code == m.RDG_EUNSUPPORTED
