"""GPU parity of rdg_combine alone on synthetic expert outputs (seeded, not
produced by the HIP path): fp32 accumulation in slot order vs the oracle's
fp64 sum, identity-expert and unpermute special cases."""
import numpy as np
import pytest
import torch

import oracle
from harness import DEV, np_of, rdg

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("T,K,E,H,ydt,shared", [(200, 8, 16, 7168, "bf16", True), (33, 4, 8, 256, "f32", False),
                                                (1, 1, 1, 8, "bf16", False), (1000, 6, 64, 512, "bf16", False)])
def test_combine_parity(T, K, E, H, ydt, shared):
    m = rdg()
    rng = np.random.default_rng([T, K, E, H])
    ids = np.stack([rng.choice(E, K, replace=False) for _ in range(T)]).astype(np.int32)
    ids[rng.random(ids.shape) < 0.1] = -1
    w = rng.random((T, K)).astype(np.float32)
    ref_l = oracle.layout(ids, E, oracle.CONTIGUOUS, block_m=16)
    m_cap = ref_l["m_cap"]
    if ydt == "bf16":
        y_h = torch.randn((m_cap, H), dtype=torch.float32).to(torch.bfloat16)
        sh_h = torch.randn((T, H), dtype=torch.float32).to(torch.bfloat16) if shared else None
        code = m.RDG_BF16
    else:
        y_h = torch.randn((m_cap, H), dtype=torch.float32)
        sh_h = torch.randn((T, H), dtype=torch.float32) if shared else None
        code = m.RDG_F32
    L = m.Layout(m.RDG_CONTIGUOUS, E, T, K, DEV, block_m=16)
    # the layout comes from the device dispatch (checked bit-exact elsewhere); the
    # payload rows are the synthetic y below
    dummy = torch.zeros((T, 16), dtype=torch.float32, device=DEV)
    xp = torch.zeros((L.m_cap, 16), dtype=torch.float32, device=DEV)
    m.rdg_dispatch(dummy, None, m.RDG_F32, torch.from_numpy(ids).to(DEV), L, xp)
    assert np.array_equal(np_of(L.pos), ref_l["pos"].ravel())
    out = torch.empty((T, H), dtype=y_h.dtype, device=DEV)
    y_d = y_h.to(DEV)
    m.rdg_combine(y_d, code, L, torch.from_numpy(w).to(DEV), T, K, H, None if sh_h is None else sh_h.to(DEV),
                  out, code)
    ref = oracle.combine(np_of(y_h), ref_l["pos"], w, shared_out=None if sh_h is None else np_of(sh_h),
                         out_dt=oracle.F32 if ydt == "f32" else oracle.BF16)
    g = np_of(out)
    if ydt == "f32":
        assert oracle.rel_err(g, ref) <= 1e-6
    else:
        # fp32 (slot order) vs fp64 accumulation: the fp32 sum is within
        # (K+2) * 2^-24 of the sum of |terms|; rounding both to bf16 can then
        # land on neighbouring values, one bf16 step (2^-7 relative) apart
        gd, rd = oracle.bf16_decode(g), oracle.bf16_decode(ref)
        yd = oracle.bf16_decode(np_of(y_h))
        pos = ref_l["pos"]
        mag = np.zeros((T, H))
        for k in range(K):
            ok = pos[:, k] >= 0
            mag[ok] += np.abs(w[ok, k, None].astype(np.float64) * yd[pos[ok, k]])
        if sh_h is not None:
            mag += np.abs(oracle.bf16_decode(np_of(sh_h)))
        bound = np.maximum(np.abs(rd), np.abs(gd)) * 2.0 ** -7 + mag * (K + 2) * 2.0 ** -24 + 1e-30
        assert np.all(np.abs(gd - rd) <= bound)
        assert np.mean(g != ref) < 1e-3


@pytest.mark.parametrize("max_blocks", [1, 7, 64, 1000])
def test_combine_workgroup_cap_is_bit_equal(max_blocks):
    # a cap on the plain form's workgroups makes each wave walk several
    # (token, 512-feature slice) units in turn; every unit is still combined
    # once, in the same slot order
    m = rdg()
    T, K, E, H = 700, 8, 32, 2048
    rng = np.random.default_rng([T, K, E, H, 9])
    ids = np.stack([rng.choice(E, K, replace=False) for _ in range(T)]).astype(np.int32)
    ids[rng.random(ids.shape) < 0.1] = -1
    w = torch.from_numpy(rng.random((T, K)).astype(np.float32)).to(DEV)
    L = m.Layout(m.RDG_CONTIGUOUS, E, T, K, DEV, block_m=16)
    dummy = torch.zeros((T, 16), dtype=torch.float32, device=DEV)
    xp = torch.zeros((L.m_cap, 16), dtype=torch.float32, device=DEV)
    m.rdg_dispatch(dummy, None, m.RDG_F32, torch.from_numpy(ids).to(DEV), L, xp)
    y = torch.randn((L.m_cap, H), dtype=torch.float32).to(torch.bfloat16).to(DEV)
    sh = torch.randn((T, H), dtype=torch.float32).to(torch.bfloat16).to(DEV)
    ref = torch.empty((T, H), dtype=torch.bfloat16, device=DEV)
    got = torch.full((T, H), float("nan"), dtype=torch.bfloat16, device=DEV)
    m.rdg_combine(y, m.RDG_BF16, L, w, T, K, H, sh, ref, m.RDG_BF16)
    m.rdg_combine(y, m.RDG_BF16, L, w, T, K, H, sh, got, m.RDG_BF16, max_blocks=max_blocks)
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int16), ref.view(torch.int16))


def test_finishing_form_alone_repeated_and_after_polling_stops():
    """rdg_combine_finish with no polling combine beside it takes every token
    (equal to the plain form bit for bit); a second call finds the counter
    closed and combines nothing; a polling combine started after the close
    claims nothing and waits for no tile (its counters are never signalled
    here); zeroing the two words hands everything to the next call again."""
    m = rdg()
    T, K, E, H = 300, 6, 20, 1024
    rng = np.random.default_rng(91)
    ids = np.stack([rng.choice(E, K, replace=False) for _ in range(T)]).astype(np.int32)
    ids[rng.random(ids.shape) < 0.2] = -1
    ids[:7] = -1  # tokens without a row
    w = torch.from_numpy(rng.random((T, K)).astype(np.float32)).to(DEV)
    L = m.Layout(m.RDG_CONTIGUOUS, E, T, K, DEV, block_m=16)
    dummy = torch.zeros((T, 16), dtype=torch.float32, device=DEV)
    xp = torch.zeros((L.m_cap, 16), dtype=torch.float32, device=DEV)
    m.rdg_dispatch(dummy, None, m.RDG_F32, torch.from_numpy(ids).to(DEV), L, xp)
    y = torch.randn((L.m_cap, H), device=DEV).to(torch.bfloat16)
    sh = torch.randn((T, H), device=DEV).to(torch.bfloat16)
    ref = torch.empty((T, H), dtype=torch.bfloat16, device=DEV)
    m.rdg_combine(y, m.RDG_BF16, L, w, T, K, H, sh, ref, m.RDG_BF16)
    rows = 16
    n_sig = (L.m_cap + rows - 1) // rows
    sig = torch.zeros((n_sig + 2,), dtype=torch.int32, device=DEV)
    out = torch.full((T, H), float("nan"), dtype=torch.bfloat16, device=DEV)
    m.rdg_combine_finish(y, m.RDG_BF16, L, w, T, K, H, sh, out, m.RDG_BF16, sig, rows)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
    assert int(sig[n_sig + 1]) == 0  # the first unit no polling wave held
    poison = torch.full_like(out, float("nan"))
    out.copy_(poison)
    m.rdg_combine_finish(y, m.RDG_BF16, L, w, T, K, H, sh, out, m.RDG_BF16, sig, rows)
    m.rdg_combine(y, m.RDG_BF16, L, w, T, K, H, sh, out, m.RDG_BF16, sig, rows, 1, 2_000_000, 4)
    torch.cuda.synchronize()
    assert m.rdg_check_status(L) == (0, 0)
    assert torch.equal(out.view(torch.int16), poison.view(torch.int16)), "nothing is left after the close"
    n_units = L.m_cap + (T + 63) // 64
    assert int(sig[n_sig + 1]) == n_units
    m.rdg_fill_i32(sig[n_sig:], 0)
    m.rdg_combine_finish(y, m.RDG_BF16, L, w, T, K, H, sh, out, m.RDG_BF16, sig, rows)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
    assert not bool(sig[:n_sig].any()), "the tile counters are the down GEMM's; the combine only reads them"


def test_finishing_form_argument_checks():
    m = rdg()
    T, K, E, H = 8, 2, 4, 256
    ids = np.tile(np.arange(K, dtype=np.int32), (T, 1))
    L = m.Layout(m.RDG_CONTIGUOUS, E, T, K, DEV, block_m=16)
    dummy = torch.zeros((T, 16), dtype=torch.float32, device=DEV)
    xp = torch.zeros((L.m_cap, 16), dtype=torch.float32, device=DEV)
    m.rdg_dispatch(dummy, None, m.RDG_F32, torch.from_numpy(ids).to(DEV), L, xp)
    y = torch.zeros((L.m_cap, H), dtype=torch.bfloat16, device=DEV)
    w = torch.ones((T, K), dtype=torch.float32, device=DEV)
    out = torch.empty((T, H), dtype=torch.bfloat16, device=DEV)
    sig = torch.zeros((L.m_cap + 2,), dtype=torch.int32, device=DEV)
    for bad in (dict(signals=None), dict(rows=7), dict(y_dt=m.RDG_F32), dict(K=3)):
        with pytest.raises(RuntimeError):
            m.rdg_combine_finish(y, bad.get("y_dt", m.RDG_BF16), L, w, T, bad.get("K", K), H, None, out, m.RDG_BF16,
                                 bad.get("signals", sig), bad.get("rows", 16))
    torch.cuda.synchronize()
