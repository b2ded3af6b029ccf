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


def _sigmoid_boundary_cases(n_cases, seed=901):
    """Logits whose fp64 sigmoid lies closest to an fp32 rounding boundary
    (a 1-ulp difference between two evaluations is most likely there), each
    with a partner logit whose oracle sigmoid is the same fp32 value.  Two
    tokens per case over two experts in one group, K = 1: [partner, x] and
    [x, partner].  Both are ties under the oracle, so the lower index wins;
    a device sigmoid one ulp above the oracle's at x picks expert 1 in the
    first token, one ulp below picks expert 1 in the second."""
    rng = np.random.default_rng(seed)
    x = rng.uniform(-12.0, 12.0, 1 << 21).astype(np.float32)
    s = oracle.sigmoid(x)
    up = np.nextafter(s, np.float32(2.0))
    dn = np.nextafter(s, np.float32(-1.0))
    s64 = 1.0 / (1.0 + np.exp(-x.astype(np.float64)))
    mid_up = (s.astype(np.float64) + up) / 2
    mid_dn = (s.astype(np.float64) + dn) / 2
    ulp = (up.astype(np.float64) - s)
    dist = np.minimum(np.abs(s64 - mid_up), np.abs(s64 - mid_dn)) / ulp
    # the hardest cases of each of 16 logit ranges, so that the whole curve is covered
    bins = np.floor((x.astype(np.float64) + 12.0) / 1.5).astype(np.int64)
    order = np.lexsort((dist, bins))
    rank = np.empty_like(order)
    starts = np.searchsorted(bins[order], np.arange(16))
    rank[order] = np.arange(len(order)) - starts[bins[order]]
    pairs = []
    for i in np.argsort(rank, kind="stable"):
        xi = x[i]
        for step in (1, -1, 2, -2, 3, -3, 4, -4):
            y = xi
            for _ in range(abs(step)):
                y = np.nextafter(y, np.float32(np.inf if step > 0 else -np.inf))
            if oracle.sigmoid(np.array([y]))[0] == s[i]:
                pairs.append((y, xi, dist[i]))
                break
        if len(pairs) == n_cases:
            break
    return pairs


def test_route_sigmoid_rounding_boundaries():
    pairs = _sigmoid_boundary_cases(4096)
    assert len(pairs) == 4096
    print("sigmoid boundary cases: largest distance from a rounding boundary %.3e ulp" % pairs[-1][2], flush=True)
    lg = np.array([[y, x] for y, x, _ in pairs] + [[x, y] for y, x, _ in pairs], dtype=np.float32)
    gi, _ = _run(lg, 1, 1, 1)
    ri, _ = oracle.route(lg, 1, 1, 1)
    assert (ri == 0).all()  # every token is a tie under the oracle
    bad = np.flatnonzero(gi[:, 0] != ri[:, 0])
    assert len(bad) == 0, ("device sigmoid differs from the oracle's at logits", lg[bad[:8]])
