"""GPU parity: EPLB remap, dispatch layouts (bit-exact against the
oracle's stable counting sort), payload rows, capacity status, and the
fp8 block quantiser (codes and scales bit-exact)."""
import numpy as np
import pytest
import torch

import oracle
from harness import DEV, check_layout, np_of, rdg

pytestmark = pytest.mark.gpu


def _ids(rng, T, K, E, skew=False, holes=0.0):
    p = None
    if skew:
        p = 1.0 / np.arange(1, E + 1) ** 1.1
        p = p / p.sum()
    out = np.stack([rng.choice(E, size=K, replace=False, p=p) for _ in range(T)]).astype(np.int32) \
        if T else np.zeros((0, K), np.int32)
    if holes:
        out[rng.random(out.shape) < holes] = -1
    return out


def _dispatch(ids_np, E, kind, block_m=128, m_max=0, m_cap=None, H=256, dtype="bf16", seed=0):
    m = rdg()
    T, K = ids_np.shape
    L = m.Layout(kind, E, T, K, DEV, block_m=block_m, m_max=m_max, m_cap=m_cap)
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    if dtype == "f32":
        x = torch.randn((T, H), generator=g, device=DEV)
        code, xs = m.RDG_F32, None
    elif dtype == "bf16":
        x = torch.randn((T, H), generator=g, device=DEV).to(torch.bfloat16)
        code, xs = m.RDG_BF16, None
    else:
        x = torch.randint(0, 0x7f, (T, H), generator=g, device=DEV, dtype=torch.int32).to(torch.uint8)
        xs = torch.rand((T, H // 128), generator=g, device=DEV)
        code = m.RDG_FP8_E4M3
    x_perm = torch.zeros((L.m_cap, H), dtype=x.dtype, device=DEV)
    xps = torch.zeros((L.m_cap, H // 128), dtype=torch.float32, device=DEV) if xs is not None else None
    ids = torch.from_numpy(ids_np).to(DEV)
    m.rdg_dispatch(x, xs, code, ids, L, x_perm, xps)
    st = m.rdg_check_status(L)
    return L, st, x, xs, x_perm, xps


@pytest.mark.parametrize("T,K,E,block_m,skew,holes,dtype", [
    (64, 4, 16, 128, False, 0.0, "f32"), (4096, 8, 256, 128, True, 0.0, "bf16"),
    (1000, 8, 37, 64, True, 0.2, "bf16"), (257, 8, 9, 128, True, 0.0, "fp8"),
    (1, 1, 1, 16, False, 0.0, "bf16"), (3, 2, 300, 32, False, 0.0, "f32"), (0, 8, 4, 128, False, 0.0, "bf16"),
    (16384, 8, 1024, 128, False, 0.9, "fp8")])
def test_contiguous(T, K, E, block_m, skew, holes, dtype):
    print("contiguous", T, K, E, block_m, dtype, flush=True)
    ids = _ids(np.random.default_rng([T, K, E]), T, K, E, skew, holes)
    L, st, x, xs, xp, xps = _dispatch(ids, E, rdg().RDG_CONTIGUOUS, block_m=block_m, dtype=dtype)
    ref = oracle.layout(ids, E, oracle.CONTIGUOUS, block_m=block_m)
    assert st == (0, 0)
    check_layout(L, ref, ids.shape)
    # payload: every filled row is its token's row, bit for bit
    rs = ref["row_src"]
    filled = np.flatnonzero(rs >= 0)
    xn, xpn = np_of(x), np_of(xp)
    assert np.array_equal(xpn[filled], xn[rs[filled] // K])
    if xs is not None:
        assert np.array_equal(np_of(xps)[filled], np_of(xs)[rs[filled] // K])


@pytest.mark.parametrize("T,K,E,m_max", [(128, 8, 256, 256), (128, 8, 32, 7), (500, 6, 16, 1000), (40, 3, 5, 1)])
def test_masked_and_capacity(T, K, E, m_max):
    print("masked", T, K, E, m_max, flush=True)
    m = rdg()
    ids = _ids(np.random.default_rng([T, E, m_max]), T, K, E, skew=True)
    L, st, x, _, xp, _ = _dispatch(ids, E, m.RDG_MASKED, m_max=m_max)
    ref = oracle.layout(ids, E, oracle.MASKED, m_max=m_max)
    assert st == (ref["status"], ref["detail"])
    check_layout(L, ref, ids.shape)
    rs = ref["row_src"]
    filled = np.flatnonzero(rs >= 0)
    assert np.array_equal(np_of(xp)[filled], np_of(x)[rs[filled] // K])


@pytest.mark.parametrize("T,K,E,kind,m_max", [(4096, 8, 256, 0, 0), (1000, 8, 37, 0, 0), (16384, 8, 1024, 0, 0),
                                                (128, 8, 32, 1, 7), (0, 8, 4, 0, 0)])
def test_layout_only(T, K, E, kind, m_max):
    # x_perm = NULL: the same layout (for a grouped GEMM that gathers the
    # rows through row_src), nothing copied, x not read
    m = rdg()
    ids = _ids(np.random.default_rng([T, K, E, 5]), T, K, E, skew=True, holes=0.1)
    L = m.Layout(kind, E, T, K, DEV, block_m=128, m_max=m_max)
    x = torch.empty((T, 256), dtype=torch.bfloat16, device=DEV)
    m.rdg_dispatch(x, None, m.RDG_BF16, torch.from_numpy(ids).to(DEV), L, None, None)
    ref = oracle.layout(ids, E, oracle.MASKED if kind else oracle.CONTIGUOUS, block_m=128, m_max=m_max)
    assert m.rdg_check_status(L) == (ref["status"], ref["detail"])
    check_layout(L, ref, ids.shape)


def test_contiguous_overflow():
    m = rdg()
    ids = _ids(np.random.default_rng(3), 300, 8, 20)
    full = oracle.layout(ids, 20, oracle.CONTIGUOUS, block_m=32)
    cap = int(full["offsets"][-1]) - 100
    L, st, *_ = _dispatch(ids, 20, m.RDG_CONTIGUOUS, block_m=32, m_cap=cap)
    ref = oracle.layout(ids, 20, oracle.CONTIGUOUS, block_m=32, m_cap=cap)
    assert st == (m.RDG_ECAPACITY, int(full["offsets"][-1])) == (ref["status"], ref["detail"])
    check_layout(L, ref, ids.shape)


def test_remap_parity():
    m = rdg()
    rng = np.random.default_rng(8)
    T, K, N, r_max = 5000, 8, 256, 2
    ids = _ids(rng, T, K, N, skew=True, holes=0.05)
    gidx = rng.integers(0, 1 << 40, T).astype(np.int64)
    nrep = np.ones(N, np.int32)
    nrep[rng.choice(N, 32, replace=False)] = 2
    l2p = rng.integers(0, 288, (N, r_max)).astype(np.int32)
    for pb, nl in [(0, 288), (36, 4), (279, 9)]:
        out = torch.empty((T, K), dtype=torch.int32, device=DEV)
        m.rdg_eplb_remap(torch.from_numpy(ids).to(DEV), torch.from_numpy(gidx).to(DEV),
                         torch.from_numpy(l2p).to(DEV), torch.from_numpy(nrep).to(DEV), pb, nl, out)
        ref = oracle.eplb_remap(ids, gidx, l2p, nrep, pb, nl)
        assert np.array_equal(np_of(out), ref)


@pytest.mark.parametrize("rows,cols,block_rows,src", [(300, 7168, 1, "bf16"), (129, 256, 1, "f32"),
                                                      (256, 384, 128, "f32"), (200, 256, 128, "bf16")])
def test_quantiser_bit_exact(rows, cols, block_rows, src):
    m = rdg()
    print("quant", rows, cols, block_rows, src, flush=True)
    rng = np.random.default_rng([rows, cols])
    v = (rng.standard_normal((rows, cols)) * np.exp(rng.uniform(-12, 8, (rows, 1)))).astype(np.float32)
    v[0, :128] = 0.0                        # an all-zero block
    v[1, :128] = 0.0
    v[1, 5] = 3.0                           # one element: lands exactly on 448
    v[2, :] = np.float32(1e-30)             # tiny magnitudes
    table = oracle.fp8_decode(np.arange(127))
    mid = ((table[:-1] + table[1:]) / 2).astype(np.float32)
    v[3, :126] = mid[:126]                  # ties, scaled by 448/amax (amax=448 -> scale 1)
    v[3, 126] = 448.0
    t = torch.from_numpy(v).to(DEV)
    if src == "bf16":
        t = t.to(torch.bfloat16)
        host = np_of(t)
    else:
        host = v
    q = torch.empty((rows, cols), dtype=torch.uint8, device=DEV)
    s = torch.empty(((rows + block_rows - 1) // block_rows, cols // 128), dtype=torch.float32, device=DEV)
    m.rdg_quantize_fp8(t, m.RDG_BF16 if src == "bf16" else m.RDG_F32, block_rows, q, s)
    rq, rs = oracle.quantize_fp8(host, block_rows)
    assert np.array_equal(np_of(s), rs)
    assert np.array_equal(np_of(q), rq)


@pytest.mark.parametrize("block_rows", [1, 128])
def test_quantiser_ue8m0_clamp_edge(block_rows):
    # power-of-two scales at their lower clamp (2^-126), fp32-subnormal
    # blocks and an all-zero block: device codes and scales equal the oracle's
    from harness import ue8m0_clamp_edge_rows
    m = rdg()
    rows = ue8m0_clamp_edge_rows()
    if block_rows == 128:
        # 128 x 128 weight blocks: each block's rows scaled to one edge row's amax
        v = np.concatenate([np.tile(rows[i:i + 1], (128, 1)) * np.float32(0.5) for i in range(0, len(rows), 3)])
        for b in range(len(v) // 128):
            v[b * 128 + 17] = rows[3 * b]     # the edge amax itself, inside the block
        v = np.concatenate([v, v[:, ::-1]], 1)   # two column blocks
    else:
        v = rows
    R, C = v.shape
    t = torch.from_numpy(np.ascontiguousarray(v)).to(DEV)
    q = torch.empty((R, C), dtype=torch.uint8, device=DEV)
    s = torch.empty(((R + block_rows - 1) // block_rows, C // 128), dtype=torch.float32, device=DEV)
    m.rdg_quantize_fp8_ue8m0(t, m.RDG_F32, block_rows, q, s)
    rq, rs = oracle.quantize_fp8(np.ascontiguousarray(v), block_rows, ue8m0=True)
    assert (rs[rs != 1.0] <= 2.0 ** -125).all()
    assert np.array_equal(np_of(s), rs)
    assert np.array_equal(np_of(q), rq)


def test_expert_load_recorder():
    """rdg_dispatch accumulates each expert's routed rows (before capacity
    drops) into the layout's expert_load buffer across calls."""
    m = rdg()
    E, K = 24, 6
    load = torch.zeros(E, dtype=torch.int64, device=DEV)
    want = np.zeros(E, np.int64)
    rng = np.random.default_rng(11)
    for T, kind, m_max, holes in ((300, m.RDG_CONTIGUOUS, 0, 0.0), (200, m.RDG_MASKED, 20, 0.0),
                                  (157, m.RDG_CONTIGUOUS, 0, 0.3), (0, m.RDG_MASKED, 8, 0.0)):
        ids_np = _ids(rng, T, K, E, skew=True, holes=holes)
        L = m.Layout(kind, E, T, K, DEV, block_m=64, m_max=m_max, expert_load=load)
        x = torch.zeros((T, 128), dtype=torch.bfloat16, device=DEV)
        xp = torch.zeros((L.m_cap, 128), dtype=torch.bfloat16, device=DEV)
        m.rdg_dispatch(x, None, m.RDG_BF16, torch.from_numpy(ids_np).to(DEV), L, xp)
        st = m.rdg_check_status(L)
        ref = oracle.layout(ids_np, E, oracle.MASKED if kind == m.RDG_MASKED else oracle.CONTIGUOUS, block_m=64,
                            m_max=m_max)
        assert st == (ref["status"], ref["detail"])
        want += ref["counts"]
        assert np.array_equal(np_of(load), want)
    assert want.sum() > 0


# batches of at most 8192 entries over at most 512 experts take the
# one-workgroup dispatch, larger ones the three-pass form: both sides of
# each limit, in both layouts (capacity drops included), with the payload
# copied and the expert loads recorded
@pytest.mark.parametrize("T,K,E,kind,m_max,holes", [
    (1024, 8, 512, 0, 0, 0.0), (1025, 8, 512, 0, 0, 0.0), (1024, 8, 513, 0, 0, 0.0),
    (1024, 8, 512, 1, 9, 0.0), (1025, 8, 512, 1, 9, 0.0), (1024, 8, 513, 1, 9, 0.0),
    (1023, 8, 500, 0, 0, 0.3), (8192, 1, 3, 1, 4000, 0.0), (8193, 1, 3, 1, 4000, 0.0)])
def test_small_and_large_dispatch_limits(T, K, E, kind, m_max, holes):
    print("dispatch limits", T, K, E, kind, m_max, flush=True)
    m = rdg()
    ids = _ids(np.random.default_rng([T, K, E, kind]), T, K, E, skew=True, holes=holes)
    load = torch.zeros(E, dtype=torch.int64, device=DEV)
    L = m.Layout(kind, E, T, K, DEV, block_m=128, m_max=m_max, expert_load=load)
    x = torch.randn((T, 256), device=DEV).to(torch.bfloat16)
    xp = torch.zeros((L.m_cap, 256), dtype=torch.bfloat16, device=DEV)
    m.rdg_dispatch(x, None, m.RDG_BF16, torch.from_numpy(ids).to(DEV), L, xp)
    ref = oracle.layout(ids, E, oracle.MASKED if kind else oracle.CONTIGUOUS, block_m=128, m_max=m_max)
    assert m.rdg_check_status(L) == (ref["status"], ref["detail"])
    check_layout(L, ref, ids.shape)
    assert np.array_equal(np_of(load), ref["counts"])
    rs = ref["row_src"]
    filled = np.flatnonzero(rs >= 0)
    assert np.array_equal(np_of(xp)[filled], np_of(x)[rs[filled] // K])
