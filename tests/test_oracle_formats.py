"""Pins for the oracle's number formats (bf16, OCP fp8 e4m3fn) and its
block quantiser, against torch's CPU casts and the formats' definitions."""
import numpy as np
import pytest
import torch


def test_bf16_encode_matches_torch_rne(orc):
    rng = np.random.default_rng(1)
    v = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(-30, 30, 20000),
                        # exact halfway cases: 8 significant bits + a trailing half
                        (np.arange(256, 512, dtype=np.float64) + 0.5) * 2.0 ** -8,
                        [0.0, -0.0, 1.0, -1.0, 2.0 ** -126, 3e38]])
    v32 = v.astype(np.float32)
    ours = orc.bf16_encode(v32.astype(np.float64))
    ref = torch.from_numpy(v32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    assert np.array_equal(orc.bf16_decode(ours), torch.from_numpy(ref.view(np.int16)).view(torch.bfloat16)
                          .float().numpy().astype(np.float64))


def test_fp8_table_from_definition(orc):
    table = orc.fp8_decode(np.arange(256))
    # the format's landmarks
    assert table[0x7E] == 448.0 and table[0xFE] == -448.0
    assert np.isnan(table[0x7F]) and np.isnan(table[0xFF])
    assert table[0x01] == 2.0 ** -9 and table[0x08] == 2.0 ** -6 and table[0x38] == 1.0
    # torch's e4m3fn decoding of every code (library routine)
    ref = torch.arange(256, dtype=torch.int16).to(torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    same = (table == ref) | (np.isnan(table) & np.isnan(ref))
    assert same.all()
    # monotone over the positive finite codes
    assert np.all(np.diff(table[:127]) > 0)


def test_fp8_encode_brute_force_and_torch(orc):
    table = orc.fp8_decode(np.arange(127))
    rng = np.random.default_rng(2)
    v = np.concatenate([rng.uniform(-448, 448, 4000), rng.standard_normal(4000) * 0.01,
                        (table[:-1] + table[1:]) / 2,            # every exact midpoint
                        -(table[:-1] + table[1:]) / 2, table, -table, [0.0]]).astype(np.float32)
    ours = orc.fp8_encode(v.astype(np.float64))
    # brute force: nearest magnitude, ties to even code
    a = np.abs(v.astype(np.float64))[:, None]
    d = np.abs(table[None, :] - a)
    best = np.empty(len(v), np.int64)
    for i in range(len(v)):
        c = np.flatnonzero(d[i] == d[i].min())
        best[i] = c[0] if len(c) == 1 else [x for x in c if x % 2 == 0][0]
    best = best | np.where(np.signbit(v), 0x80, 0)
    assert np.array_equal(ours, best.astype(np.uint8))
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


def test_torch_e4m3_cast_needs_clamp():
    # why the quantiser clamps: torch turns values past the top rounding
    # boundary into NaN, so an unclamped cast is not a usable reference
    out = torch.tensor([470.0, 449.0]).to(torch.float8_e4m3fn).float()
    assert torch.isnan(out[0]) and out[1] == 448.0


@pytest.mark.parametrize("block_rows", [1, 128])
def test_quantiser_blocks(orc, block_rows):
    rng = np.random.default_rng(3)
    rows, cols = 256, 384
    x = (rng.standard_normal((rows, cols)) * rng.uniform(0.01, 5, (rows, 1))).astype(np.float32)
    x[:block_rows, 128:256] = 0.0  # an all-zero block -> scale 1
    q, s = orc.quantize_fp8(x, block_rows)
    assert s.shape == (rows // block_rows, cols // 128)
    deq = orc.fp8_decode(q) * np.repeat(np.repeat(s, block_rows, 0), 128, 1)
    for br in range(s.shape[0]):
        for bc in range(s.shape[1]):
            blk = x[br * block_rows:(br + 1) * block_rows, bc * 128:(bc + 1) * 128]
            amax = np.float32(np.abs(blk).max())
            want = np.float32(amax / np.float32(448.0)) if amax > 0 else np.float32(1.0)
            assert s[br, bc] == want
            if amax > 0:  # the block's largest element lands on +-448
                qb = q[br * block_rows:(br + 1) * block_rows, bc * 128:(bc + 1) * 128]
                assert (qb & 0x7F).max() == 0x7E
    # each element is the nearest representable after scaling: relative error
    # at most half a step of 3 mantissa bits (2^-4) above the subnormal range
    big = np.abs(x) > np.repeat(np.repeat(s, block_rows, 0), 128, 1) * 2.0 ** -6
    rel = np.abs(deq - x)[big] / np.abs(x)[big]
    assert rel.max() <= 2.0 ** -4 + 1e-12
    # a bf16 source gives the same codes as its fp32 image
    xb = torch.from_numpy(x).to(torch.bfloat16)
    qb, sb = orc.quantize_fp8(xb.view(torch.int16).numpy().view(np.uint16), block_rows)
    qf, sf = orc.quantize_fp8(xb.float().numpy(), block_rows)
    assert np.array_equal(qb, qf) and np.array_equal(sb, sf)


def test_ue8m0_scale_rule(orc):
    # power-of-two block scales: the smallest 2^k with amax / 2^k <= 448,
    # checked against the closed form 2^ceil(log2(amax / 448)) and by its
    # defining inequalities; an all-zero block gets 1
    rng = np.random.default_rng(8)
    rows, cols = 64, 512
    mag = 2.0 ** rng.uniform(-30, 30, (rows, 1))
    x = (rng.standard_normal((rows, cols)) * mag).astype(np.float32)
    x[3, 128:256] = 0.0
    q, s = orc.quantize_fp8(x, 1, ue8m0=True)
    amax = np.abs(x.reshape(rows, -1, 128)).max(-1).astype(np.float64)
    s64 = s.astype(np.float64)
    nz = amax > 0
    assert (np.frexp(s64)[0] == 0.5).all()                        # powers of two
    assert (amax[nz] / s64[nz] <= 448.0).all() and (amax[nz] / (s64[nz] / 2) > 448.0).all()
    assert (s64[nz] == 2.0 ** np.ceil(np.log2(amax[nz] / 448.0))).all()
    assert s[3, 1] == 1.0
    # each element is the nearest representable after scaling
    deq = orc.fp8_decode(q) * np.repeat(s64, 128, 1)
    big = np.abs(x) > np.repeat(s64, 128, 1) * 2.0 ** -6
    assert (np.abs(deq - x)[big] / np.abs(x)[big]).max() <= 2.0 ** -4 + 1e-12


def test_ue8m0_matches_fp32_rule_at_exact_powers(orc):
    # a block whose amax is 448 * 2^j has the same scale 2^j under both rules,
    # hence the same codes; one ulp more moves the power-of-two scale up
    rng = np.random.default_rng(9)
    x = rng.uniform(-1, 1, (8, 256)).astype(np.float32)
    for r in range(8):
        j = r - 4
        x[r, 7] = np.float32(448.0 * 2.0 ** j)
        x[r, 128:] = np.clip(x[r, 128:], -0.5, 0.5) * np.float32(448.0 * 2.0 ** j)
        x[r, 200] = np.nextafter(np.float32(448.0 * 2.0 ** j), np.float32(np.inf))
    qa, sa = orc.quantize_fp8(x, 1)
    qb, sb = orc.quantize_fp8(x, 1, ue8m0=True)
    for r in range(8):
        j = r - 4
        assert sb[r, 0] == 2.0 ** j and sa[r, 0] == sb[r, 0]
        assert np.array_equal(qa[r, :128], qb[r, :128])
        assert sb[r, 1] == 2.0 ** (j + 1)


def test_ue8m0_clamp_edge(orc):
    # amax at and below 448 * 2^-126: the power-of-two scale stops at 2^-126
    # (the smallest normal fp32 and the lowest 8-bit exponent kept), so the
    # codes are the nearest e4m3 values of v * 2^126; checked against the
    # closed form of the scale with its clamp and a brute-force nearest-even
    # encoder over the 127 non-negative finite codes
    from harness import ue8m0_clamp_edge_rows
    x = ue8m0_clamp_edge_rows()
    q, s = orc.quantize_fp8(x, 1, ue8m0=True)
    amax = np.abs(x).max(1).astype(np.float64)
    want_s = np.where(amax > 0, np.maximum(2.0 ** np.ceil(np.log2(np.maximum(amax, 1e-300) / 448.0)), 2.0 ** -126), 1.0)
    assert np.array_equal(s[:, 0].astype(np.float64), want_s)
    assert (s[:-3, 0] <= 2.0 ** -125).all()
    table = orc.fp8_decode(np.arange(127))
    t = np.abs(x.astype(np.float64)) / want_s[:, None]          # exact: a power-of-two scale
    d = np.abs(t[..., None] - table)
    best = d.min(-1, keepdims=True)
    cand = d == best
    # ties to the even code (the one with a zero last mantissa bit)
    code = np.where(cand.sum(-1) > 1, np.argmax(cand & (np.arange(127) % 2 == 0), -1), np.argmax(cand, -1))
    code = code | np.where(np.signbit(x) & (code > 0), 0x80, 0)
    mag_q = q & 0x7f
    assert np.array_equal(np.where(mag_q == 0, 0, q), code.astype(np.uint8))
