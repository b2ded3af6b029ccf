"""Pins for the oracle's expert FFN, combine and the layer definition.

Independent references: dense fp64 matmuls in numpy (a library routine)
for the FFN, torch's e4m3fn cast for the fp8 re-quantisation of h, exact
identities (identity experts, K=1 unpermute, power-of-two linearity), and
the equality of the definition path with the layout path."""
import numpy as np
import pytest
import torch


def _bf16(a):
    return torch.from_numpy(np.asarray(a, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _silu(g):
    return g / (1.0 + np.exp(-g))


def _make(rng, dt, H, I, E, orc):
    ex = []
    dense = []
    for e in range(E):
        W1 = (rng.standard_normal((I, H)) * 0.05).astype(np.float32)
        W3 = (rng.standard_normal((I, H)) * 0.05).astype(np.float32)
        W2 = (rng.standard_normal((H, I)) * 0.05).astype(np.float32)
        if dt == orc.F32:
            ex.append(dict(W1=W1, W3=W3, W2=W2))
            dense.append((W1.astype(np.float64), W3.astype(np.float64), W2.astype(np.float64)))
        elif dt == orc.BF16:
            b = [_bf16(w) for w in (W1, W3, W2)]
            ex.append(dict(W1=b[0], W3=b[1], W2=b[2]))
            dense.append(tuple(orc.bf16_decode(w) for w in b))
        else:
            d = {}
            dd = []
            for name, w in (("1", W1), ("3", W3), ("2", W2)):
                q, s = orc.quantize_fp8(w, 128, ue8m0=dt == orc.FP8_UE8M0)
                d["W" + name] = q
                d["s" + name] = s
                dd.append(orc.fp8_decode(q) * np.repeat(np.repeat(s.astype(np.float64), 128, 0), 128, 1))
            ex.append(d)
            dense.append(tuple(dd))
    return ex, dense


def _x(rng, dt, T, H, orc):
    x = rng.standard_normal((T, H)).astype(np.float32)
    if dt == orc.F32:
        return x, None, x.astype(np.float64)
    xb = _bf16(x)
    if dt == orc.BF16:
        return xb, None, orc.bf16_decode(xb)
    q, s = orc.quantize_fp8(xb, 1, ue8m0=dt == orc.FP8_UE8M0)
    return q, s, orc.fp8_decode(q) * np.repeat(s.astype(np.float64), 128, 1)


def _ref_ffn(dt, a, W1, W3, W2, orc):
    """Dense numpy reference of one expert on rows a [m, H] (fp64)."""
    g = a @ W1.T
    u = a @ W3.T
    h = _silu(g) * u
    if dt == orc.F32:
        h = h.astype(np.float32).astype(np.float64)
    elif dt == orc.BF16:
        h = torch.from_numpy(h).to(torch.bfloat16).double().numpy()
    else:  # 1x128 blocks along I, scale amax/448 in fp32 (or the power of two
        # 2^ceil(log2(amax/448))), torch's e4m3fn cast
        hf = torch.from_numpy(h.astype(np.float32)).view(h.shape[0], -1, 128)
        amax = hf.abs().amax(-1, keepdim=True)
        if dt == orc.FP8_UE8M0:
            s = torch.exp2(torch.ceil(torch.log2(amax.double() / 448.0))).float()
        else:
            s = amax / 448.0
        s = torch.where(amax > 0, s, torch.ones_like(s))
        q = (hf / s).clamp(-448, 448).to(torch.float8_e4m3fn).double()
        h = (q * s.double()).view(h.shape[0], -1).numpy()
    y = h @ W2.T
    if dt == orc.F32:
        return y.astype(np.float32).astype(np.float64)
    return torch.from_numpy(y).to(torch.bfloat16).double().numpy()


@pytest.mark.parametrize("dt,tol", [(0, 1e-6), (1, 8e-3), (2, 8e-3), (3, 8e-3)])
def test_expert_ffn_against_dense_matmul(orc, dt, tol):
    rng = np.random.default_rng(dt)
    T, H, I, E, K = 12, 256, 384, 3, 2
    ex, dense = _make(rng, dt, H, I, E, orc)
    x, xs, a = _x(rng, dt, T, H, orc)
    ids = np.stack([np.arange(T) % E, (np.arange(T) + 1) % E], 1).astype(np.int32)
    w = np.full((T, K), 0.5, np.float32)
    _, y = orc.moe_layer(dt, x, ids, w, ex, x_scales=xs, want_y=True, out_dt=orc.F32)
    for t in range(T):
        for k in range(K):
            e = ids[t, k]
            ref = _ref_ffn(dt, a[t:t + 1], *dense[e], orc)[0]
            assert orc.rel_err(y[t, k], ref) <= tol, (dt, t, k, orc.rel_err(y[t, k], ref))


def test_swapped_gate_and_up_is_detected(orc):
    # the dense check above fails for a plausible mistake: gate and up swapped
    rng = np.random.default_rng(3)
    ex, dense = _make(rng, orc.F32, 256, 128, 1, orc)
    x, _, a = _x(rng, orc.F32, 4, 256, orc)
    _, y = orc.moe_layer(orc.F32, x, np.zeros((4, 1), np.int32), np.ones((4, 1), np.float32), ex,
                         want_y=True, out_dt=orc.F32)
    W1, W3, W2 = dense[0]
    wrong = _ref_ffn(orc.F32, a, W3, W1, W2, orc)
    assert orc.rel_err(y[:, 0], wrong) > 1e-2


@pytest.mark.parametrize("dt", [0, 1, 2, 3])
def test_linearity_power_of_two(orc, dt):
    # doubling W2 doubles every stored output exactly (all roundings commute
    # with a power-of-two scale; fp8 scales double exactly)
    rng = np.random.default_rng(10 + dt)
    T, H, I = 6, 256, 256
    W1 = (rng.standard_normal((I, H)) * 0.05).astype(np.float32)
    W3 = (rng.standard_normal((I, H)) * 0.05).astype(np.float32)
    W2 = (rng.standard_normal((H, I)) * 0.05).astype(np.float32)

    def pack(w2):
        if dt == orc.F32:
            return dict(W1=W1, W3=W3, W2=w2)
        if dt == orc.BF16:
            return dict(W1=_bf16(W1), W3=_bf16(W3), W2=_bf16(w2))
        d = {}
        for n, w in (("1", W1), ("3", W3), ("2", w2)):
            d["W" + n], d["s" + n] = orc.quantize_fp8(w, 128, ue8m0=dt == orc.FP8_UE8M0)
        return d

    x, xs, _ = _x(rng, dt, T, H, orc)
    ids = np.zeros((T, 1), np.int32)
    one = np.ones((T, 1), np.float32)
    _, y1 = orc.moe_layer(dt, x, ids, one, [pack(W2)], x_scales=xs, want_y=True)
    _, y2 = orc.moe_layer(dt, x, ids, one, [pack(2 * W2)], x_scales=xs, want_y=True)
    assert np.array_equal(y2, 2 * y1)


def test_identity_experts_and_unpermute(orc):
    # with "identity experts" (expert output = its input row) the combine of a
    # layout returns x * sum(w) = x * scale; with K = 1 and w = 1 it is an exact
    # unpermute
    rng = np.random.default_rng(21)
    T, K, E, H = 200, 8, 16, 64
    logits = rng.standard_normal((T, E)).astype(np.float32)
    ids, w = orc.route(logits, 4, 2, K)
    x = _bf16(rng.standard_normal((T, H)))
    for kind in (orc.CONTIGUOUS, orc.MASKED):
        L = orc.layout(ids, E, kind, block_m=16, m_max=T)
        y_perm = np.zeros((L["m_cap"], H), np.uint16)
        src = L["row_src"]
        y_perm[src >= 0] = x[src[src >= 0] // K]
        out = orc.combine(y_perm, L["pos"], w)
        assert np.array_equal(out, x)  # sum(w) = 1 within 4 ulp: bf16(x * (1 +- 5e-7)) == x
        ids1 = ids[:, :1].copy()
        L1 = orc.layout(ids1, E, kind, block_m=16, m_max=T)
        yp = rng.integers(0, 0x7F80, (L1["m_cap"], H)).astype(np.uint16)  # finite bf16 patterns
        out1 = orc.combine(yp, L1["pos"], np.ones((T, 1), np.float32))
        assert np.array_equal(out1, yp[L1["pos"][:, 0]])


@pytest.mark.parametrize("dt", [0, 1, 2, 3])
def test_definition_path_equals_layout_path(orc, dt):
    rng = np.random.default_rng(30 + dt)
    T, H, I, E, K = 40, 256, 128 if dt < 2 else 256, 8, 3
    ex, _ = _make(rng, dt, H, I, E, orc)
    sh, _ = _make(rng, dt, H, I, 1, orc)
    x, xs, _ = _x(rng, dt, T, H, orc)
    ids, w = orc.route(rng.standard_normal((T, E)).astype(np.float32), 4, 2, K)
    out_dt = orc.F32 if dt == orc.F32 else orc.BF16
    out, y = orc.moe_layer(dt, x, ids, w, ex, shared=sh[0], x_scales=xs, want_y=True)
    sh_out = orc.moe_layer(dt, x, np.full((T, 1), -1, np.int32), np.zeros((T, 1), np.float32), [None] * E,
                           shared=sh[0], x_scales=xs)
    L = orc.layout(ids, E, orc.CONTIGUOUS, block_m=16)
    y_perm = np.zeros((L["m_cap"], H), np.float32 if dt == orc.F32 else np.uint16)
    src = L["row_src"]
    for p in np.flatnonzero(src >= 0):
        t, k = divmod(int(src[p]), K)
        y_perm[p] = y[t, k] if dt == orc.F32 else orc.bf16_encode(y[t, k])
    out2 = orc.combine(y_perm, L["pos"], w, shared_out=sh_out, out_dt=out_dt)
    if dt == orc.F32:
        # the definition sums the unrounded shared output; allow its fp32 rounding
        assert orc.rel_err(out2, out) <= 1e-6
    else:
        assert np.array_equal(out2, out)


def test_identical_experts_reduce_to_dense_ffn(orc):
    # all experts identical: out = shared(x) + scale * FFN(x) for every token
    rng = np.random.default_rng(40)
    T, H, I, E, K = 16, 256, 128, 8, 4
    ex, dense = _make(rng, orc.F32, H, I, 1, orc)
    sh, shd = _make(rng, orc.F32, H, I, 1, orc)
    x, _, a = _x(rng, orc.F32, T, H, orc)
    ids, w = orc.route(rng.standard_normal((T, E)).astype(np.float32), 4, 2, K)
    out = orc.moe_layer(orc.F32, x, ids, w, ex * E, shared=sh[0])
    ref = _ref_ffn(orc.F32, a, *shd[0], orc) + _ref_ffn(orc.F32, a, *dense[0], orc) * w.astype(np.float64).sum(1)[:, None]
    assert orc.rel_err(out, ref) <= 1e-6
