"""GPU parity: rdg_route against the oracle -- ids bit-exact, weights to
fp32 rounding.  Shapes: the five workloads' routers, the literal
"128 groups of 2" reading of the deep-dive's gating paragraph, tie-heavy
logits, ragged token counts and the N limits."""
import numpy as np
import pytest
import torch

import oracle
import synth
from harness import DEV, np_of, rdg

pytestmark = pytest.mark.gpu


def _run(logits_np, n_group, topk_group, K, scale=1.0):
    m = rdg()
    lg = torch.from_numpy(logits_np).to(DEV)
    B = lg.shape[0]
    ids = torch.full((B, K), -7, dtype=torch.int32, device=DEV)
    w = torch.zeros((B, K), dtype=torch.float32, device=DEV)
    m.rdg_route(lg, n_group, topk_group, K, scale, ids, w)
    torch.cuda.synchronize()
    return np_of(ids), np_of(w)


def _check(logits_np, n_group, topk_group, K, scale=1.0):
    gi, gw = _run(logits_np, n_group, topk_group, K, scale)
    ri, rw = oracle.route(logits_np, n_group, topk_group, K, scale)
    bad = np.flatnonzero((gi != ri).any(1))
    assert len(bad) == 0, ("ids differ at tokens", bad[:10], gi[bad[:3]], ri[bad[:3]])
    # the kernel sums K fp32 scores in slot order, then divides and scales in
    # fp32; the oracle rounds the fp64 value once: within (K + 2) fp32 ulps
    bound = (K + 2) * 2.0 ** -24
    assert np.max(np.abs(gw.astype(np.float64) - rw) / np.maximum(np.abs(rw), 1e-30)) <= bound


@pytest.mark.parametrize("name", ["tiny_fp32", "decode_bf16", "prefill_bf16", "prefill_bf16_balanced"])
def test_route_workloads(name):
    cfg = synth.WORKLOADS[name]
    print("route", name, flush=True)
    _check(synth.logits(cfg), cfg["n_group"], cfg["topk_group"], cfg["K"], cfg["scale"])


@pytest.mark.parametrize("name", ["decode_rank_fp8", "prefill_rank_fp8"])
def test_route_global_batches(name):
    cfg = synth.WORKLOADS[name]
    print("route", name, flush=True)
    _check(synth.logits(cfg), cfg["n_group"], cfg["topk_group"], cfg["K"], cfg["scale"])


@pytest.mark.parametrize("B,N,n_group,topk_group,K", [
    (1, 256, 8, 4, 8), (5, 256, 8, 4, 8), (131, 256, 128, 4, 8),   # 128 groups of 2
    (77, 16, 4, 2, 4), (64, 64, 1, 1, 6), (33, 64, 64, 64, 6), (50, 1024, 64, 8, 32),
    (19, 512, 16, 3, 10), (7, 40, 5, 2, 3), (300, 96, 12, 5, 7)])
def test_route_shapes_and_ties(B, N, n_group, topk_group, K):
    rng = np.random.default_rng([B, N, n_group])
    print("route shape", B, N, n_group, topk_group, K, flush=True)
    _check(rng.standard_normal((B, N)).astype(np.float32), n_group, topk_group, K, 1.0)
    _check(rng.integers(-1, 2, (B, N)).astype(np.float32), n_group, topk_group, K, 2.5)  # exact ties


def test_route_empty_batch():
    m = rdg()
    ids = torch.zeros((1, 8), dtype=torch.int32, device=DEV)
    w = torch.zeros((1, 8), dtype=torch.float32, device=DEV)
    m.rdg_route(torch.zeros((0, 256), device=DEV), 8, 4, 8, 1.0, ids, w)
    torch.cuda.synchronize()
    assert int(ids.abs().sum()) == 0


# selection-only bias (a variant not on the pages): ids bit-exact, weights from
# the plain scores to the same rounding bound
@pytest.mark.parametrize("B,N,n_group,topk_group,K,std", [
    (4096, 256, 8, 4, 8, 0.5), (333, 256, 8, 4, 8, 3.0), (77, 16, 4, 2, 4, 0.3), (50, 1024, 64, 8, 32, 0.2),
    (300, 96, 12, 5, 7, 1.0)])
def test_route_biased(B, N, n_group, topk_group, K, std):
    m = rdg()
    rng = np.random.default_rng([B, N, 5])
    for ties in (False, True):
        if ties:
            logits = rng.integers(-1, 2, (B, N)).astype(np.float32)
            bias = (rng.integers(-2, 3, N) * 0.125).astype(np.float32)
        else:
            logits = rng.standard_normal((B, N)).astype(np.float32)
            bias = rng.normal(0.0, std, N).astype(np.float32)
        ids = torch.full((B, K), -7, dtype=torch.int32, device=DEV)
        w = torch.zeros((B, K), dtype=torch.float32, device=DEV)
        m.rdg_route_biased(torch.from_numpy(logits).to(DEV), torch.from_numpy(bias).to(DEV), n_group, topk_group, K,
                           1.0, ids, w)
        gi, gw = np_of(ids), np_of(w)
        ri, rw = oracle.route(logits, n_group, topk_group, K, 1.0, bias=bias)
        bad = np.flatnonzero((gi != ri).any(1))
        print("biased route", B, N, n_group, topk_group, K, std, ties, "differing tokens", len(bad), flush=True)
        assert len(bad) == 0, (bad[:10], gi[bad[:3]], ri[bad[:3]])
        bound = (K + 2) * 2.0 ** -24
        assert np.max(np.abs(gw.astype(np.float64) - rw) / np.maximum(np.abs(rw), 1e-30)) <= bound
