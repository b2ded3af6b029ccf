"""GPU edge cases of the whole path against the oracle: an empty layer,
masked-capacity drops carried through the FFN and the combine, one expert
holding every token in whole 128-row tiles (no padding), and hidden sizes
that are multiples of 128 but not of 256 (the 128-row tiled kernels decline
them and the 64-row kernels take over)."""
import numpy as np
import pytest
import torch

import oracle
import synth
from harness import (DEV, ExpertSet, check_rows, dt_code, np_of, out_as_f64, quantize_act, rdg, run_routed,
                     tolerance)

pytestmark = pytest.mark.gpu


def _cfg(dtype, H=512, I=256, N=8, K=2, wid=700):
    return dict(wid=wid, H=H, N=N, n_group=1, topk_group=1, K=K, I=I, shared_I=0, dtype=dtype, scale=1.0,
                logits="normal", name="edge_" + dtype)


def _inputs(cfg, T):
    x = synth.x(cfg, T, device=DEV)
    x_s, xo, xo_s = None, np_of(x), None
    if cfg["dtype"] in ("fp8", "fp8u"):
        x, x_s = quantize_act(x, cfg["dtype"] == "fp8u")
        if T:
            xo, xo_s = oracle.quantize_fp8(xo, 1, ue8m0=cfg["dtype"] == "fp8u")
    return x, x_s, xo, xo_s


def _compare(cfg, got, ref, what):
    err = oracle.rel_err(out_as_f64(got), out_as_f64(ref))
    check_rows(got, ref, cfg, what)
    print("%s rel_err=%.3e" % (what, err), flush=True)
    assert err <= tolerance(cfg), err


@pytest.mark.parametrize("dtype", ["f32", "bf16", "fp8"])
@pytest.mark.parametrize("kind", [0, 1])
def test_empty_layer(dtype, kind):
    m = rdg()
    cfg = _cfg(dtype)
    x, x_s, _, _ = _inputs(cfg, 0)
    ids = torch.zeros((0, cfg["K"]), dtype=torch.int32, device=DEV)
    w = torch.zeros((0, cfg["K"]), dtype=torch.float32, device=DEV)
    experts = ExpertSet(cfg, range(cfg["N"]))
    r = run_routed(cfg, x, x_s, ids, w, experts, kind, block_m=128, m_max=128 if kind else 0)
    assert m.rdg_check_status(r["L"]) == (0, 0)
    assert r["out"].shape == (0, cfg["H"])
    assert int(np_of(r["L"].counts).sum()) == 0


@pytest.mark.parametrize("dtype", ["f32", "bf16", "fp8"])
def test_masked_capacity_drop_through_the_layer(dtype):
    """Rows past m_max are dropped (status RDG_ECAPACITY, detail = largest
    count); the output is the sum over the kept rows only."""
    m = rdg()
    cfg = _cfg(dtype, N=4, K=2, wid=710)
    T, m_max = 96, 16
    rng = np.random.default_rng(3)
    ids_np = np.stack([rng.choice(cfg["N"], size=2, replace=False) for _ in range(T)]).astype(np.int32)
    w_np = rng.uniform(0.2, 0.8, size=(T, 2)).astype(np.float32)
    x, x_s, xo, xo_s = _inputs(cfg, T)
    experts = ExpertSet(cfg, range(cfg["N"]))
    r = run_routed(cfg, x, x_s, torch.from_numpy(ids_np).to(DEV), torch.from_numpy(w_np).to(DEV), experts,
                   m.RDG_MASKED, m_max=m_max)
    lay = oracle.layout(ids_np, cfg["N"], oracle.MASKED, m_max=m_max)
    assert m.rdg_check_status(r["L"]) == (lay["status"], lay["detail"]) == (m.RDG_ECAPACITY,
                                                                              int(np.bincount(ids_np.ravel()).max()))
    kept = np.where(lay["pos"].reshape(T, 2) >= 0, ids_np, -1).astype(np.int32)
    assert (kept < 0).sum() > 0
    ref = oracle.moe_layer(dt_code(cfg), xo, kept, w_np, [experts.oracle_expert(j) for j in range(cfg["N"])],
                           x_scales=xo_s)
    _compare(cfg, np_of(r["out"]), ref, "capacity drop %s" % dtype)


@pytest.mark.parametrize("dtype", ["bf16", "fp8", "fp8u"])
@pytest.mark.parametrize("T", [128, 256, 129])
def test_one_expert_whole_tiles(dtype, T):
    """Every token to expert 2 of 4 with K = 1: exactly T/128 full tiles (T=129: one row past them)."""
    m = rdg()
    cfg = _cfg(dtype, N=4, K=1, wid=720 + T)
    ids_np = np.full((T, 1), 2, np.int32)
    w_np = np.full((T, 1), 0.75, np.float32)
    x, x_s, xo, xo_s = _inputs(cfg, T)
    experts = ExpertSet(cfg, range(cfg["N"]))
    r = run_routed(cfg, x, x_s, torch.from_numpy(ids_np).to(DEV), torch.from_numpy(w_np).to(DEV), experts,
                   m.RDG_CONTIGUOUS, block_m=128)
    assert m.rdg_check_status(r["L"]) == (0, 0)
    assert np_of(r["L"].counts).tolist() == [0, 0, T, 0]
    ref = oracle.moe_layer(dt_code(cfg), xo, ids_np, w_np, [None, None, experts.oracle_expert(2), None],
                           x_scales=xo_s)
    _compare(cfg, np_of(r["out"]), ref, "one expert %s T=%d" % (dtype, T))


@pytest.mark.parametrize("dtype", ["bf16", "fp8", "fp8u"])
def test_hidden_not_a_multiple_of_256(dtype):
    m = rdg()
    cfg = dict(_cfg(dtype, H=384, I=384, N=4, K=2, wid=730), n_group=2, topk_group=1)
    T = 600
    logits = synth.logits(cfg, T)
    ri, rw = oracle.route(logits, cfg["n_group"], cfg["topk_group"], cfg["K"], cfg["scale"])
    x, x_s, xo, xo_s = _inputs(cfg, T)
    experts = ExpertSet(cfg, range(cfg["N"]))
    r = run_routed(cfg, x, x_s, torch.from_numpy(ri).to(DEV), torch.from_numpy(rw).to(DEV), experts,
                   m.RDG_CONTIGUOUS, block_m=128)
    assert m.rdg_check_status(r["L"]) == (0, 0)
    ref = oracle.moe_layer(dt_code(cfg), xo, ri, rw, [experts.oracle_expert(j) for j in range(cfg["N"])],
                           x_scales=xo_s)
    _compare(cfg, np_of(r["out"]), ref, "H=384 %s" % dtype)


@pytest.mark.parametrize("kind", [0, 1])
def test_fp8u_wide_panels(kind):
    """fp8 with power-of-two scales and enough row tiles that the 128-row
    kernels take 64 weight rows per wave (the row tiles times the 256-feature
    gate/up panels reach four times the CU count): two experts of 9000 and
    7463 rows (ragged last tiles), I = 2048, contiguous and masked; sampled
    rows, including every expert's last rows, against the oracle."""
    m = rdg()
    cfg = _cfg("fp8u", H=1024, I=2048, N=2, K=1, wid=740 + kind)
    counts = (9000, 7463)
    T = sum(counts)
    ids_np = np.concatenate([np.full(c, e, np.int32) for e, c in enumerate(counts)]).reshape(T, 1)
    ids_np = ids_np[np.random.default_rng(kind).permutation(T)]
    w_np = np.full((T, 1), 1.0, np.float32)
    x, x_s, xo, xo_s = _inputs(cfg, T)
    experts = ExpertSet(cfg, range(cfg["N"]))
    m_max = 9088 if kind == m.RDG_MASKED else 0
    r = run_routed(cfg, x, x_s, torch.from_numpy(ids_np).to(DEV), torch.from_numpy(w_np).to(DEV), experts, kind,
                   block_m=128, m_max=m_max)
    assert m.rdg_check_status(r["L"]) == (0, 0)
    last = [int(np.flatnonzero(ids_np[:, 0] == e)[-j]) for e in range(2) for j in (1, 2, 3)]
    sel = np.unique(np.concatenate([np.random.default_rng(9).choice(T, 40, replace=False), last])).astype(np.int32)
    ref = oracle.moe_layer(dt_code(cfg), xo, ids_np, w_np, [experts.oracle_expert(e) for e in range(2)],
                           x_scales=xo_s, sel=sel)
    _compare(cfg, np_of(r["out"])[sel], ref, "fp8u wide kind=%d" % kind)


@pytest.mark.parametrize("H,I", [(1536, 768), (1024, 512), (512, 768)])
def test_tiled_bf16_chunk_counts(H, I):
    """bf16 through the 128-row kernels (64-byte chunks, three ring slots) for
    reduction lengths whose chunk counts leave each remainder modulo three
    (gate/up / down: 48 / 24, 32 / 16, 16 / 24 chunks), with ragged experts;
    every output row against the oracle."""
    m = rdg()
    cfg = dict(_cfg("bf16", H=H, I=I, N=4, K=2, wid=750 + H + I), n_group=2, topk_group=1)
    T = 300
    logits = synth.logits(cfg, T)
    ri, rw = oracle.route(logits, cfg["n_group"], cfg["topk_group"], cfg["K"], cfg["scale"])
    x, x_s, xo, xo_s = _inputs(cfg, T)
    experts = ExpertSet(cfg, range(cfg["N"]))
    r = run_routed(cfg, x, x_s, torch.from_numpy(ri).to(DEV), torch.from_numpy(rw).to(DEV), experts,
                   m.RDG_CONTIGUOUS, block_m=128)
    assert m.rdg_check_status(r["L"]) == (0, 0)
    assert m.rdg_signal_rows(r["L"], m.RDG_BF16, H, I) == 128  # the row tile the FFN ran with
    ref = oracle.moe_layer(dt_code(cfg), xo, ri, rw, [experts.oracle_expert(j) for j in range(cfg["N"])],
                           x_scales=xo_s)
    _compare(cfg, np_of(r["out"]), ref, "tiled bf16 H=%d I=%d" % (H, I))


@pytest.mark.parametrize("dtype", ["fp8", "fp8u"])
@pytest.mark.parametrize("H,I", [(256, 256), (768, 512), (1280, 768)])
def test_tiled_fp8_chunk_counts(dtype, H, I):
    """fp8 (fp32 and power-of-two scales) through the 128-row kernels
    (256-byte chunks, two ring slots, direct loads issued from assembly) for
    reduction lengths of one chunk and of odd and even chunk counts (gate/up /
    down: 1 / 1, 3 / 2, 5 / 3 chunks), with ragged experts; every output row
    against the oracle."""
    m = rdg()
    cfg = dict(_cfg(dtype, H=H, I=I, N=4, K=2, wid=790 + H + I), n_group=2, topk_group=1)
    T = 300
    logits = synth.logits(cfg, T)
    ri, rw = oracle.route(logits, cfg["n_group"], cfg["topk_group"], cfg["K"], cfg["scale"])
    x, x_s, xo, xo_s = _inputs(cfg, T)
    experts = ExpertSet(cfg, range(cfg["N"]))
    r = run_routed(cfg, x, x_s, torch.from_numpy(ri).to(DEV), torch.from_numpy(rw).to(DEV), experts,
                   m.RDG_CONTIGUOUS, block_m=128)
    assert m.rdg_check_status(r["L"]) == (0, 0)
    DT = m.RDG_FP8_E4M3_UE8M0 if dtype == "fp8u" else m.RDG_FP8_E4M3
    assert m.rdg_signal_rows(r["L"], DT, H, I) == 128  # the row tile the FFN ran with
    ref = oracle.moe_layer(dt_code(cfg), xo, ri, rw, [experts.oracle_expert(j) for j in range(cfg["N"])],
                           x_scales=xo_s)
    _compare(cfg, np_of(r["out"]), ref, "tiled %s H=%d I=%d" % (dtype, H, I))


@pytest.mark.parametrize("dtype", ["f32", "bf16", "fp8"])
@pytest.mark.parametrize("kind", [0, 1])
def test_weight_streaming_experts_over_several_tiles(dtype, kind):
    """16-row tiles of the weight-streaming kernels (15 rows per expert on
    average) where experts 0 and 3 hold 40 and 20 rows: their second and third
    tiles read the same weights (cacheable loads, shared in L2), the others
    stream theirs; every output row against the oracle."""
    m = rdg()
    cfg = _cfg(dtype, H=512, I=256, N=16, K=2, wid=770)
    T = 120
    rng = np.random.default_rng(11)
    first = np.concatenate([np.zeros(40, np.int32), np.full(20, 3, np.int32),
                            rng.choice([1, 2] + list(range(4, 16)), size=T - 60).astype(np.int32)])
    ids_np = np.stack([first, (first + 1 + rng.integers(0, 14, T)) % 16], 1).astype(np.int32)
    ids_np[ids_np[:, 1] == ids_np[:, 0], 1] = (ids_np[ids_np[:, 1] == ids_np[:, 0], 0] + 5) % 16
    counts = np.bincount(ids_np.ravel(), minlength=16)
    assert counts[0] >= 40 and counts[3] >= 20 and counts.sum() == 2 * T
    w_np = rng.uniform(0.2, 0.8, size=(T, 2)).astype(np.float32)
    x, x_s, xo, xo_s = _inputs(cfg, T)
    experts = ExpertSet(cfg, range(cfg["N"]))
    m_max = 64 if kind == m.RDG_MASKED else 0
    r = run_routed(cfg, x, x_s, torch.from_numpy(ids_np).to(DEV), torch.from_numpy(w_np).to(DEV), experts, kind,
                   block_m=16, m_max=m_max)
    assert m.rdg_check_status(r["L"]) == (0, 0)
    assert m.rdg_signal_rows(r["L"], dt_code(cfg), cfg["H"], cfg["I"]) == 16  # 16-row tiles
    ref = oracle.moe_layer(dt_code(cfg), xo, ids_np, w_np, [experts.oracle_expert(j) for j in range(cfg["N"])],
                           x_scales=xo_s)
    _compare(cfg, np_of(r["out"]), ref, "experts over several tiles %s kind=%d" % (dtype, kind))
