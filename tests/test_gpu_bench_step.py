"""GPU parity of the benchmark's own step: the launch configuration bench.py
times (streams, the shared expert on a second stream, weight rotation, the
rank shares' remap, the signalled down GEMM with the polling combine, a
replayed HIP graph) against the oracle's definition of the layer.

For each workload one Bench is built exactly as bench.py builds it and its
step is run; the output is then compared with the oracle on every token for
the small and decode layers, and on a covering sample elsewhere (each
expert's first and last row and the first row of each of its 128-row tiles,
plus seeded random tokens).  Integers (routing ids, the received rows of a
rank share) bit-exact; outputs within max|out-ref|/max|ref| <= 1e-5 (fp32),
2e-2 (bf16), 6e-2 (fp8), and per-token L2 error bounds."""
import numpy as np
import pytest
import torch

import oracle
import synth
from harness import DEV, check_rows, np_of, out_as_f64, tolerance

pytestmark = pytest.mark.gpu


def _bench(name, **kw):
    import bench
    return bench.Bench(name, DEV, **kw)


def _cover(ids, n_local, n, seed, tile=128):
    from test_gpu_layer import _cover as cover
    return cover(ids, n_local, n, seed, tile)


def _check(cfg, got, ref, what):
    err = oracle.rel_err(out_as_f64(got), out_as_f64(ref))
    row = check_rows(got, ref, cfg, what)
    print("%s rel_err=%.3e worst_token=%.3e" % (what, err, row), flush=True)
    assert err <= tolerance(cfg), err


def _full_reference(b, sel):
    cfg = b.cfg
    ri, rw = oracle.route(b.logits_np, cfg["n_group"], cfg["topk_group"], cfg["K"], cfg["scale"])
    assert np.array_equal(np_of(b.ids), ri), "routing ids differ from the oracle"
    used = set(np.unique(ri[sel]).tolist())
    experts = [{k: np_of(v) for k, v in synth.expert_weights(cfg, e, device=DEV).items()} if e in used else None
               for e in range(cfg["N"])]
    shared = {k: np_of(v) for k, v in synth.expert_weights(cfg, 0, device=DEV, shared=True).items()}
    dt = oracle.F32 if cfg["dtype"] == "f32" else oracle.BF16
    return oracle.moe_layer(dt, np_of(b.x), ri, rw, experts, shared=shared, sel=sel), ri


@pytest.mark.parametrize("name,n_sample", [("tiny_fp32", None), ("decode_bf16", None), ("prefill_bf16", 256)])
def test_bench_step_full_layers(name, n_sample):
    b = _bench(name)
    print("bench step %s: %d weight sets, shared expert on a side stream: %s" %
          (name, len(b.weight_sets), b.overlap_shared), flush=True)
    for _ in range(2):            # the second step uses the next weight set where there are several
        b.step()
    torch.cuda.synchronize()
    assert b.rdg.rdg_check_status(b.L) == (0, 0)
    B = b.T
    ri, _ = oracle.route(b.logits_np, b.cfg["n_group"], b.cfg["topk_group"], b.cfg["K"], b.cfg["scale"])
    sel = np.arange(B) if n_sample is None else _cover(ri, b.cfg["N"], n_sample, 7)
    print("%s: comparing %d of %d tokens" % (name, len(sel), B), flush=True)
    ref, _ = _full_reference(b, sel)
    _check(b.cfg, np_of(b.out)[sel], ref, "bench step " + name)


def test_bench_graph_replay_decode():
    # the decode step captured in a HIP graph as bench.py --graph does;
    # every replay equals the oracle on every token
    b = _bench("decode_bf16")
    b.step()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        b.step()
    torch.cuda.synchronize()
    ref = None
    for rep in range(3):
        b.rdg.rdg_fill_i32(b.out.view(torch.int32), -1)
        g.replay()
        torch.cuda.synchronize()
        if ref is None:
            ref, _ = _full_reference(b, np.arange(b.T))
        _check(b.cfg, np_of(b.out), ref, "graph replay %d" % rep)


def _rank_reference(b, sel):
    cfg, plan = b.cfg, b.plan
    # the rank's received rows, recomputed from the oracle's routing of the global batch
    lg = synth.logits(cfg)
    ri, rw = oracle.route(lg, cfg["n_group"], cfg["topk_group"], cfg["K"], cfg["scale"])
    gidx = np.arange(ri.shape[0], dtype=np.int64)
    rows = [int((oracle.eplb_remap(ri, gidx, plan["log2phy"], plan["n_replica"], r * plan["n_local"],
                                   plan["n_local"]) >= 0).sum()) for r in range(cfg["n_ranks"])]
    assert int(np.argmax(rows)) == plan["rank"], "measured rank differs from the oracle's choice"
    rloc = oracle.eplb_remap(ri, gidx, plan["log2phy"], plan["n_replica"], plan["phys_begin"], plan["n_local"])
    toks, keep = synth.take_rank_rows(rloc, cfg["rows"])
    ids = ri[toks].copy()
    ids[~keep & (rloc[toks] >= 0)] = -1
    assert np.array_equal(np_of(b.ids), ids), "received rows differ from the oracle's"
    loc = oracle.eplb_remap(ids, gidx[toks], plan["log2phy"], plan["n_replica"], plan["phys_begin"], plan["n_local"])
    assert np.array_equal(np_of(b.local), loc), "remap differs from the oracle"
    xb = synth.x(cfg, len(toks), device=DEV)
    xq, xs = oracle.quantize_fp8(np_of(xb), 1, ue8m0=b.ue8m0)
    assert np.array_equal(np_of(b.x), xq) and np.array_equal(np_of(b.x_s), xs)
    experts = []
    for e in b.local_logical:
        wt = synth.expert_weights(cfg, e, device=DEV)
        ex = {}
        for k, key in (("W1", "1"), ("W3", "3"), ("W2", "2")):
            q, s = oracle.quantize_fp8(np_of(wt[k]), 128, ue8m0=b.ue8m0)
            ex["W" + key], ex["s" + key] = q, s
        experts.append(ex)
    dt = oracle.FP8_UE8M0 if b.ue8m0 else oracle.FP8
    return oracle.moe_layer(dt, xq, loc, rw[toks], experts, x_scales=xs, sel=sel), loc


@pytest.mark.parametrize("name,ue8m0,replicas", [("decode_rank_fp8", False, None), ("prefill_rank_fp8", False, None),
                                                  ("prefill_rank_fp8", True, None),
                                                  ("decode_rank_fp8", False, "one_each")])
def test_bench_step_rank_shares(name, ue8m0, replicas):
    b = _bench(name, ue8m0=ue8m0, replicas=replicas)
    print("bench step %s ue8m0=%s replicas=%s: %d tokens, %d weight sets" %
          (name, ue8m0, b.plan["rule"], b.T, len(b.weight_sets)), flush=True)
    modes = ["signalled", "sequential"] if b.signals is not None else ["plain"]
    outs = {}
    for mode in modes:
        if mode != "plain":
            b.sbo_mode = mode
        for _ in range(2):
            b.rdg.rdg_fill_i32(b.out.view(torch.int32), -1)   # NaN: a token the step skipped cannot pass
            b.step()
        torch.cuda.synchronize()
        assert b.rdg.rdg_check_status(b.L) == (0, 0)
        outs[mode] = b.out.clone()
    if len(outs) == 2:
        assert torch.equal(outs["signalled"].view(torch.int16), outs["sequential"].view(torch.int16)), \
            "the overlapped step differs from the sequential one"
    n = None if name == "decode_rank_fp8" else 256
    T = b.T
    ids = np_of(b.local)
    assert int((ids >= 0).sum()) == b.cfg["rows"], "the share must hold exactly the configured rows"
    sel = np.arange(T) if n is None else _cover(ids, b.cfg["n_local"], n, 9)
    print("%s: comparing %d of %d tokens" % (name, len(sel), T), flush=True)
    ref, _ = _rank_reference(b, sel)
    cfg = dict(b.cfg, dtype="fp8u" if ue8m0 else "fp8")
    _check(cfg, np_of(outs[modes[0]])[sel], ref, "bench step " + name)
    if b.cfg.get("shared_I"):
        # the shared expert on the rank's own tokens
        xo = synth.x(b.cfg, b.cfg["own_tokens"], device=DEV, tensor=10)
        q, s = oracle.quantize_fp8(np_of(xo), 1, ue8m0=b.ue8m0)
        wt = synth.expert_weights(b.cfg, 0, device=DEV, shared=True)
        sh = {}
        for k, key in (("W1", "1"), ("W3", "3"), ("W2", "2")):
            qq, ss = oracle.quantize_fp8(np_of(wt[k]), 128, ue8m0=b.ue8m0)
            sh["W" + key], sh["s" + key] = qq, ss
        own = b.cfg["own_tokens"]
        sel2 = np.unique(np.concatenate([np.arange(8), np.arange(own - 8, own),
                                         np.random.default_rng(3).choice(own, 48, replace=False)]))
        dt = oracle.FP8_UE8M0 if b.ue8m0 else oracle.FP8
        ref2 = oracle.moe_layer(dt, q, np.full((own, 1), -1, np.int32), np.zeros((own, 1), np.float32), [None],
                                shared=sh, x_scales=s, sel=sel2)
        _check(cfg, np_of(b.ys)[sel2], ref2, "bench shared expert " + name)
