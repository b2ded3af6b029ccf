"""GPU parity of the gathering grouped FFN (rdg_grouped_ffn_gather): the
dispatch builds the layout only (x_perm = NULL) and the gate/up GEMM reads
each layout row's token through row_src.  The permutation of rows into
expert order ([H100] "DeepGEMM integration": the contiguous grouped GEMM
takes rows sorted by expert; [DEEP] "EP": each token's vector goes to each
of its K experts) then happens in the GEMM's loads instead of a copy.

Against the permuting path on the same inputs: the layouts (counts,
offsets, pos, row_src) and every valid row of h and y bit-exact, and the
combined output bit-exact -- every kernel family (16-row weight-streaming
tiles, 32/64-row tiles, 128-row LDS tiles; fp32, bf16, fp8 with fp32 and
with power-of-two scales), contiguous and masked layouts, ragged tails.
Against the oracle: whole layers run through the gathering path."""
import numpy as np
import pytest
import torch

from harness import DEV, ExpertSet, dt_code, is_fp8, np_of, quantize_act, rdg, run_routed
import synth
from test_gpu_layer import _full_layer, _route, _small_cfg

pytestmark = pytest.mark.gpu


def _inputs(cfg, B):
    logits = synth.logits(cfg, B)
    ids, w, _, _ = _route(cfg, logits)
    x = synth.x(cfg, B, device=DEV)
    x_s = None
    if is_fp8(cfg):
        x, x_s = quantize_act(x, cfg["dtype"] == "fp8u")
    return ids, w, x, x_s


def _valid_rows(L):
    return torch.from_numpy(np.flatnonzero(np_of(L.row_src) >= 0)).to(DEV)


def _same(a, b):
    if a.dtype == torch.bfloat16:
        return torch.equal(a.view(torch.int16), b.view(torch.int16))
    if a.dtype == torch.float32:
        return torch.equal(a.view(torch.int32), b.view(torch.int32))
    return torch.equal(a, b)


def _compare(cfg, B, kind, m_max=0, experts=None):
    m = rdg()
    ids, w, x, x_s = _inputs(cfg, B)
    if experts is None:
        experts = ExpertSet(cfg, range(cfg["N"]))
    ref = run_routed(cfg, x, x_s, ids, w, experts, kind, m_max=m_max)
    got = run_routed(cfg, x, x_s, ids, w, experts, kind, m_max=m_max, gather=True)
    torch.cuda.synchronize()
    assert m.rdg_check_status(got["L"]) == m.rdg_check_status(ref["L"])
    for f in ("counts", "offsets", "masked_m", "pos", "row_src"):
        assert torch.equal(getattr(got["L"], f), getattr(ref["L"], f)), f
    rows = _valid_rows(ref["L"])
    plan = m.rdg_signal_rows(ref["L"], dt_code(cfg), cfg["H"], cfg["I"])
    print("%s B=%d kind=%d: %d valid rows, row tile %d" % (cfg["dtype"], B, kind, len(rows), plan), flush=True)
    assert _same(got["h"][rows], ref["h"][rows]), "h differs"
    if is_fp8(cfg):
        assert _same(got["h_s"][rows], ref["h_s"][rows]), "h scales differ"
    assert _same(got["y"][rows], ref["y"][rows]), "y differs"
    assert _same(got["out"], ref["out"]), "combined output differs"


# rows per expert T*K/N: 40*4/32 = 5 (16-row tiles), 300*4/32 = 37.5 (64),
# 600*4/16 = 150 (128 for bf16 / fp8; 64 for fp32)
@pytest.mark.parametrize("dtype", ["f32", "bf16", "fp8", "fp8u"])
@pytest.mark.parametrize("B,N,kind", [(40, 32, 0), (300, 32, 0), (600, 16, 0), (40, 32, 1), (600, 16, 1)])
def test_gather_equals_permuted_small(dtype, B, N, kind):
    cfg = _small_cfg(dtype, N=N, wid=900 + B + N)
    m_max = ((B + 63) // 64) * 64 if kind == rdg().RDG_MASKED else 0
    _compare(cfg, B, kind, m_max=m_max)


# the 128-row LDS-tiled kernels at shapes they run (H a multiple of the
# down panel, I of the gate/up panel), several tiles per expert and a
# ragged last tile; a token count that leaves some experts empty
@pytest.mark.parametrize("dtype", ["bf16", "fp8", "fp8u"])
@pytest.mark.parametrize("B", [1000, 1237])
def test_gather_equals_permuted_tiled(dtype, B):
    cfg = _small_cfg(dtype, N=8, n_group=4, topk_group=2, K=2, H=1024, I=512, wid=950 + B)
    _compare(cfg, B, 0)


def test_gather_with_noalloc_dispatch():
    # the layout-only dispatch through the allocation-free entry point (its
    # work area holds only the row-tile tables the GEMMs read)
    m = rdg()
    cfg = _small_cfg("bf16", N=16, wid=977)
    B = 500
    ids, w, x, _ = _inputs(cfg, B)
    experts = ExpertSet(cfg, range(cfg["N"]))
    ref = run_routed(cfg, x, None, ids, w, experts, 0)
    L = m.Layout(0, cfg["N"], B, cfg["K"], DEV, block_m=128)
    L.work = torch.zeros(m.rdg_layout_tables_bytes(cfg["N"]), dtype=torch.uint8, device=DEV)
    L.c.work = L.work.data_ptr()
    m.rdg_dispatch_noalloc(x, None, m.RDG_BF16, ids, L, None, None)
    h = torch.empty((L.m_cap, cfg["I"]), dtype=torch.bfloat16, device=DEV)
    y = torch.empty((L.m_cap, cfg["H"]), dtype=torch.bfloat16, device=DEV)
    m.rdg_grouped_ffn_gather(L, m.RDG_BF16, cfg["H"], cfg["I"], x, None, cfg["K"], experts.W1, experts.W3,
                             experts.W2, None, None, None, h, None, y)
    torch.cuda.synchronize()
    assert m.rdg_check_status(L) == (0, 0)
    assert torch.equal(L.row_src, ref["L"].row_src) and torch.equal(L.pos, ref["L"].pos)
    rows = _valid_rows(L)
    assert _same(y[rows], ref["y"][rows])


def test_gather_argument_checks():
    m = rdg()
    cfg = _small_cfg("bf16", N=16, wid=978)
    B = 64
    ids, w, x, _ = _inputs(cfg, B)
    experts = ExpertSet(cfg, range(cfg["N"]))
    L = m.Layout(0, cfg["N"], B, cfg["K"], DEV, block_m=128)
    m.rdg_dispatch(x, None, m.RDG_BF16, ids, L, None, None)
    h = torch.empty((L.m_cap, cfg["I"]), dtype=torch.bfloat16, device=DEV)
    y = torch.empty((L.m_cap, cfg["H"]), dtype=torch.bfloat16, device=DEV)
    for K in (0, 33, 3):   # out of range; a K that does not divide the layout's rows
        with pytest.raises(RuntimeError):
            m.rdg_grouped_ffn_gather(L, m.RDG_BF16, cfg["H"], cfg["I"], x, None, K, experts.W1, experts.W3,
                                     experts.W2, None, None, None, h, None, y)
    torch.cuda.synchronize()


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_gather_small_layer_vs_oracle(dtype):
    cfg = _small_cfg(dtype, N=16, wid=990)
    _full_layer(cfg, 600, 0, gather=True)


def test_gather_decode_workload_vs_oracle():
    cfg = dict(synth.WORKLOADS["decode_bf16"])
    _full_layer(cfg, cfg["B"], rdg().RDG_MASKED, m_max=cfg["m_max"], gather=True)


def test_gather_prefill_workload_vs_oracle():
    cfg = dict(synth.WORKLOADS["prefill_bf16"])
    _full_layer(cfg, cfg["B"], 0, n_sample=256, seed=5, gather=True)


# busy experts (several 128-row tiles) beside one-tile experts and empty
# ones, so that the bf16 down GEMM runs its split work order (a one-tile
# expert's panels back to back on one XCD, interleaved with the busy
# experts' panel-major items), and a tiny layer where that order does not
# fit the grid and the plain order runs; every token against the oracle,
# both payload forms
@pytest.mark.parametrize("counts", [[700, 40, 0, 300, 17, 129, 0, 64, 1, 128, 520, 33, 5, 0, 90, 256],
                                    [100, 60]])
@pytest.mark.parametrize("gather", [False, True])
def test_tiled_busy_and_one_tile_experts(counts, gather):
    import oracle
    from harness import check_rows, out_as_f64, tolerance
    from test_gpu_layer import _oracle_experts
    m = rdg()
    N = len(counts)
    cfg = _small_cfg("bf16", N=N, n_group=1, topk_group=1, K=1, H=1024, I=512, wid=1500 + N)
    B = int(sum(counts))
    rng = np.random.default_rng(N)
    ids_np = np.repeat(np.arange(N, dtype=np.int32), counts)[rng.permutation(B)].reshape(B, 1)
    w_np = np.ones((B, 1), np.float32)
    ids = torch.from_numpy(ids_np).to(DEV)
    w = torch.from_numpy(w_np).to(DEV)
    x = synth.x(cfg, B, device=DEV)
    experts = ExpertSet(cfg, range(N))
    r = run_routed(cfg, x, None, ids, w, experts, 0, gather=gather)
    torch.cuda.synchronize()
    assert m.rdg_check_status(r["L"]) == (0, 0)
    assert m.rdg_signal_rows(r["L"], m.RDG_BF16, cfg["H"], cfg["I"]) == 128  # the 128-row kernels
    used = set(np.unique(ids_np).tolist())
    ref = oracle.moe_layer(oracle.BF16, np_of(x), ids_np, w_np, _oracle_experts(experts, used))
    got = np_of(r["out"])
    err = oracle.rel_err(out_as_f64(got), out_as_f64(ref))
    row = check_rows(got, ref, cfg, "busy and one-tile experts")
    print("counts %s gather=%s rel_err=%.3e worst_row=%.3e" % (counts, gather, err, row), flush=True)
    assert err <= tolerance(cfg), err
