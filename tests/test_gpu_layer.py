"""GPU parity of the whole hot path (route -> [remap] -> dispatch -> grouped
FFN -> combine, plus the shared expert) against the oracle's definition of
the layer.  Integers (ids, layouts) bit-exact; outputs within
max|out-ref|/max|ref| <= 1e-5 (fp32), 2e-2 (bf16), 6e-2 (fp8).

Small workloads are compared on every token; the five full-size workloads
on every integer output and on a seeded sample of tokens."""
import numpy as np
import pytest
import torch

import oracle
import synth
from harness import (DEV, ExpertSet, check_layout, check_rows, dt_code, is_fp8, np_of, out_as_f64, quantize_act, rdg,
                     run_routed, run_shared, tolerance)

pytestmark = pytest.mark.gpu


def _route(cfg, logits_np):
    m = rdg()
    B = logits_np.shape[0]
    K = cfg["K"]
    ids = torch.empty((B, K), dtype=torch.int32, device=DEV)
    w = torch.empty((B, K), dtype=torch.float32, device=DEV)
    m.rdg_route(torch.from_numpy(logits_np).to(DEV), cfg["n_group"], cfg["topk_group"], K, cfg["scale"], ids, w)
    ri, rw = oracle.route(logits_np, cfg["n_group"], cfg["topk_group"], K, cfg["scale"])
    assert np.array_equal(np_of(ids), ri), "routing ids differ from the oracle"
    return ids, w, ri, rw


def _oracle_experts(es, used):
    return [es.oracle_expert(j) if j in used else None for j in range(len(es.ids))]


def _sample(T, n, seed):
    if T <= n:
        return np.arange(T)
    rng = np.random.default_rng(seed)
    mid = rng.choice(np.arange(8, T - 8), size=n - 16, replace=False)
    return np.unique(np.concatenate([np.arange(8), mid, np.arange(T - 8, T)]))


def _cover(ids, n_local, n, seed, tile=128):
    """Tokens to compare at full size: for every expert with rows, the
    tokens of its first row, of its last row and of the first row of each of
    its 128-row tiles (rows are stable by flat index t*K+k, so an expert's
    j-th row belongs to its j-th token in index order), then seeded random
    tokens up to n."""
    T = ids.shape[0]
    flat = ids.ravel()
    keep = set()
    for e in range(n_local):
        toks = np.flatnonzero(flat == e) // ids.shape[1]
        if len(toks) == 0:
            continue
        keep.update(toks[::tile].tolist())
        keep.add(int(toks[-1]))
    rng = np.random.default_rng(seed)
    rest = np.setdiff1d(np.arange(T), np.array(sorted(keep), dtype=np.int64))
    extra = max(0, n - len(keep))
    if extra:
        keep.update(rng.choice(rest, size=min(extra, len(rest)), replace=False).tolist())
    return np.array(sorted(keep), dtype=np.int64)


def _full_layer(cfg, B, kind, block_m=128, m_max=0, n_sample=None, seed=0, gather=False):
    """Workloads where this GPU holds every expert (the tiny, decode and prefill layers)."""
    m = rdg()
    dt = dt_code(cfg)
    logits = synth.logits(cfg, B)
    ids, w, ri, rw = _route(cfg, logits)
    x = synth.x(cfg, B, device=DEV)
    x_s = None
    xo = np_of(x)
    xo_s = None
    if is_fp8(cfg):
        pow2 = cfg["dtype"] == "fp8u"
        xq, x_s = quantize_act(x, pow2)
        rq, rs = oracle.quantize_fp8(np_of(x), 1, ue8m0=pow2)
        assert np.array_equal(np_of(xq), rq) and np.array_equal(np_of(x_s), rs)
        x, xo, xo_s = xq, rq, rs
    N = cfg["N"]
    experts = ExpertSet(cfg, range(N))
    shared = ExpertSet(cfg, [0], shared=True) if cfg["shared_I"] else None
    sh_out = run_shared(cfg, x, x_s, shared) if shared else None
    r = run_routed(cfg, x, x_s, ids, w, experts, kind, block_m=block_m, m_max=m_max, shared_out=sh_out,
                   gather=gather)
    st = m.rdg_check_status(r["L"])
    ref_l = oracle.layout(ri, N, kind, block_m=block_m, m_max=m_max)
    assert st == (ref_l["status"], ref_l["detail"])
    check_layout(r["L"], ref_l, ri.shape)
    sel = _cover(ri, N, n_sample, seed) if n_sample else np.arange(B)
    print("%s comparing %d of %d tokens with the oracle" % (cfg.get("name", ""), len(sel), B), flush=True)
    used = set(np.unique(ri[sel]).tolist())
    ref = oracle.moe_layer(dt, xo, ri, rw, _oracle_experts(experts, used),
                           shared=shared.oracle_expert(0) if shared else None, x_scales=xo_s, sel=sel)
    got = np_of(r["out"])[sel]
    err = oracle.rel_err(out_as_f64(got), out_as_f64(ref))
    row = check_rows(got, ref, cfg, cfg.get("name", ""))
    print("%s B=%d kind=%d rel_err=%.3e worst_row=%.3e" % (cfg.get("name", cfg["wid"]), B, kind, err, row), flush=True)
    assert err <= tolerance(cfg), err
    return err


def _small_cfg(dtype, N=32, n_group=4, topk_group=2, K=4, H=512, I=256, wid=100):
    return dict(wid=wid, H=H, N=N, n_group=n_group, topk_group=topk_group, K=K, I=I, shared_I=I, dtype=dtype,
                scale=1.0, logits="normal", name="small_" + dtype)


# row tiles 16 / 32 / 64 are picked from the rows per expert (T*K/N): 40*4/32=5,
# 300*4/32=37.5, 600*4/16=150; the ragged token counts leave partial tiles
@pytest.mark.parametrize("dtype", ["f32", "bf16", "fp8", "fp8u"])
@pytest.mark.parametrize("B,N,kind", [(40, 32, 0), (300, 32, 0), (600, 16, 0), (40, 32, 1), (300, 32, 1),
                                      (600, 16, 1)])
def test_small_layers(dtype, B, N, kind):
    cfg = _small_cfg(dtype, N=N, wid=100 + B + N)
    m_max = 0
    if kind == rdg().RDG_MASKED:
        m_max = ((B + 63) // 64) * 64  # never overflows: a token hits an expert once
    _full_layer(cfg, B, kind, block_m=128, m_max=m_max)


# a dense expert of T rows (the shared expert): T <= 256 takes the skinny
# kernels with 1, 2 or 4 16-row tiles per workgroup (several row groups and a
# ragged tail at T = 100 and 256 - 3); larger T the 128-row tiled kernels
@pytest.mark.parametrize("dtype", ["f32", "bf16", "fp8", "fp8u"])
@pytest.mark.parametrize("T", [1, 16, 29, 64, 100, 253, 300])
def test_dense_expert(dtype, T):
    m = rdg()
    cfg = _small_cfg(dtype, H=1024, I=512, wid=400 + T)
    x = synth.x(cfg, T, device=DEV)
    x_s, xo, xo_s = None, np_of(x), None
    if is_fp8(cfg):
        x, x_s = quantize_act(x, dtype == "fp8u")
        xo, xo_s = oracle.quantize_fp8(xo, 1, ue8m0=dtype == "fp8u")
        assert np.array_equal(np_of(x), xo) and np.array_equal(np_of(x_s), xo_s)
    shared = ExpertSet(cfg, [0], shared=True)
    got = np_of(run_shared(cfg, x, x_s, shared))
    ids = np.full((T, 1), -1, dtype=np.int32)
    ref = oracle.moe_layer(dt_code(cfg), xo, ids, np.zeros((T, 1), np.float32), [None],
                           shared=shared.oracle_expert(0), x_scales=xo_s)
    err = oracle.rel_err(out_as_f64(got), out_as_f64(ref))
    check_rows(got, ref, cfg, "dense %s T=%d" % (dtype, T))
    print("dense expert %s T=%d rel_err=%.3e" % (dtype, T, err), flush=True)
    assert err <= tolerance(cfg), err


def test_tiny_fp32_workload():
    cfg = dict(synth.WORKLOADS["tiny_fp32"], name="tiny_fp32")
    _full_layer(cfg, cfg["B"], rdg().RDG_CONTIGUOUS, block_m=16)


def test_decode_bf16_workload():
    cfg = dict(synth.WORKLOADS["decode_bf16"], name="decode_bf16")
    _full_layer(cfg, cfg["B"], rdg().RDG_MASKED, m_max=cfg["m_max"])   # every token


def test_prefill_bf16_workload():
    cfg = dict(synth.WORKLOADS["prefill_bf16"], name="prefill_bf16")
    _full_layer(cfg, cfg["B"], rdg().RDG_CONTIGUOUS, block_m=128, n_sample=256, seed=3)


def test_prefill_bf16_balanced_workload():
    # the "simulated perfect EPLB" distribution of the H100 deployment
    # article's prefill evaluation: random group-limited choices
    cfg = dict(synth.WORKLOADS["prefill_bf16_balanced"], name="prefill_bf16_balanced")
    _full_layer(cfg, cfg["B"], rdg().RDG_CONTIGUOUS, block_m=128, n_sample=256, seed=4)


# ---------------------------------------------------------------- rank shares
def rank_share(cfg):
    """One rank's received tokens under the EPLB placement: route the global
    batch (checked bit-exact), remap onto the rank that receives the most rows, and take the
    tokens that send it rows, in global order, until exactly cfg['rows'] rows
    (the last token's surplus local rows are marked -1: not sent)."""
    m = rdg()
    plan = synth.eplb_plan(cfg)
    logits = synth.logits(cfg)
    ids, w, ri, rw = _route(cfg, logits)
    Tg, K = ri.shape
    gidx = np.arange(Tg, dtype=np.int64)
    l2p, nrep = plan["log2phy"], plan["n_replica"]
    rows = [int((oracle.eplb_remap(ri, gidx, l2p, nrep, r * plan["n_local"], plan["n_local"]) >= 0).sum())
            for r in range(cfg["n_ranks"])]
    plan = synth.measured_rank(plan, rows)
    loc = torch.empty((Tg, K), dtype=torch.int32, device=DEV)
    m.rdg_eplb_remap(ids, torch.from_numpy(gidx).to(DEV), torch.from_numpy(l2p).to(DEV),
                     torch.from_numpy(nrep).to(DEV), plan["phys_begin"], plan["n_local"], loc)
    rloc = oracle.eplb_remap(ri, gidx, l2p, nrep, plan["phys_begin"], plan["n_local"])
    assert np.array_equal(np_of(loc), rloc), "remap differs from the oracle"
    toks, keep = synth.take_rank_rows(rloc, cfg["rows"])
    recv_ids = ri[toks].copy()
    recv_ids[~keep & (rloc[toks] >= 0)] = -1   # surplus rows of the last token are not sent
    taken = int(keep.sum())
    phys2log = np.full(cfg["n_ranks"] * cfg["n_local"], -1)
    for e in range(cfg["N"]):
        for r_ in range(nrep[e]):
            phys2log[l2p[e, r_]] = e
    local_logical = [int(phys2log[plan["phys_begin"] + s]) for s in range(plan["n_local"])]
    return dict(plan=plan, tokens=toks, ids=recv_ids.astype(np.int32), w=rw[toks], gidx=gidx[toks],
                rows=taken, local_logical=local_logical, w_dev=w[torch.from_numpy(toks).to(DEV)].contiguous())


def _rank_layer(cfg, kind, m_max=0, block_m=128, signals=False, concurrent=False, n_sample=256, seed=0):
    m = rdg()
    share = rank_share(cfg)
    assert share["rows"] == cfg["rows"]
    T = len(share["tokens"])
    plan = share["plan"]
    x_bf = synth.x(cfg, T, device=DEV)
    pow2 = cfg["dtype"] == "fp8u"
    xq, x_s = quantize_act(x_bf, pow2)
    rq, rs = oracle.quantize_fp8(np_of(x_bf), 1, ue8m0=pow2)
    assert np.array_equal(np_of(xq), rq) and np.array_equal(np_of(x_s), rs)
    ids_d = torch.from_numpy(share["ids"]).to(DEV)
    loc = torch.empty_like(ids_d)
    m.rdg_eplb_remap(ids_d, torch.from_numpy(share["gidx"]).to(DEV), torch.from_numpy(plan["log2phy"]).to(DEV),
                     torch.from_numpy(plan["n_replica"]).to(DEV), plan["phys_begin"], plan["n_local"], loc)
    rloc = oracle.eplb_remap(share["ids"], share["gidx"], plan["log2phy"], plan["n_replica"], plan["phys_begin"],
                             plan["n_local"])
    assert np.array_equal(np_of(loc), rloc)
    assert int((rloc >= 0).sum()) == cfg["rows"]
    experts = ExpertSet(cfg, share["local_logical"])
    r = run_routed(cfg, xq, x_s, loc, share["w_dev"], experts, kind, block_m=block_m, m_max=m_max,
                   signals=signals, concurrent=concurrent, max_blocks=64 if concurrent else 0)
    st = m.rdg_check_status(r["L"])
    ref_l = oracle.layout(rloc, plan["n_local"], kind, block_m=block_m, m_max=m_max)
    assert st == (ref_l["status"], ref_l["detail"])
    check_layout(r["L"], ref_l, rloc.shape)
    sel = _cover(rloc, plan["n_local"], n_sample, seed) if n_sample else np.arange(T)
    print("%s comparing %d of %d tokens with the oracle" % (cfg["name"], len(sel), T), flush=True)
    oe = [experts.oracle_expert(j) for j in range(plan["n_local"])]
    ref = oracle.moe_layer(dt_code(cfg), rq, rloc, share["w"], oe, x_scales=rs, sel=sel)
    got = np_of(r["out"])[sel]
    err = oracle.rel_err(out_as_f64(got), out_as_f64(ref))
    print("%s rows=%d tokens=%d rel_err=%.3e" % (cfg["name"], cfg["rows"], T, err), flush=True)
    row = check_rows(got, ref, cfg, cfg["name"])
    print("%s worst token relative error %.3e" % (cfg["name"], row), flush=True)
    assert err <= tolerance(cfg), err
    # for information: the error of the whole fp8 path (quantised x, W and h)
    # against the layer computed in fp64 from the unquantised weights and the
    # bf16 tokens, on 8 of the sampled tokens
    few = sel[:8]
    xb = np_of(x_bf)
    ref_u = np.zeros((len(few), cfg["H"]))
    for j, e in enumerate(share["local_logical"]):
        wt = synth.expert_weights(cfg, e, device=DEV)
        W1, W3, W2 = (wt[k].double().cpu().numpy() for k in ("W1", "W3", "W2"))
        for i, t in enumerate(few):
            for k in range(rloc.shape[1]):
                if rloc[t, k] == j:
                    a = oracle.bf16_decode(xb[t])
                    g, u = W1 @ a, W3 @ a
                    ref_u[i] += float(share["w"][t, k]) * (W2 @ (g / (1.0 + np.exp(-g)) * u))
    err_u = oracle.rel_err(out_as_f64(got[:len(few)]), ref_u)
    print("%s error against the unquantised fp64 layer (information) %.3e" % (cfg["name"], err_u), flush=True)
    return r, share, experts, (xq, x_s, loc, rloc, rq, rs, oe)


def test_decode_rank_fp8_workload():
    cfg = dict(synth.WORKLOADS["decode_rank_fp8"], name="decode_rank_fp8")
    _rank_layer(cfg, rdg().RDG_MASKED, m_max=cfg["m_max"], n_sample=None)   # every token


@pytest.mark.parametrize("name", ["decode_rank_fp8", "prefill_rank_fp8"])
def test_rank_workloads_ue8m0(name):
    # the rank shares with power-of-two block scales (scales applied inside
    # the scaled MFMA by the 128-row kernels)
    m = rdg()
    cfg = dict(synth.WORKLOADS[name], name=name + "_ue8m0", dtype="fp8u")
    if name == "decode_rank_fp8":
        _rank_layer(cfg, m.RDG_MASKED, m_max=cfg["m_max"])
    else:
        _rank_layer(cfg, m.RDG_CONTIGUOUS, block_m=128, signals=True, concurrent=True)


def _valid_rows(L):
    return np.flatnonzero(np_of(L.row_src) >= 0)


def test_prefill_rank_fp8_workload_sbo():
    m = rdg()
    cfg = dict(synth.WORKLOADS["prefill_rank_fp8"], name="prefill_rank_fp8")
    r, share, experts, (xq, x_s, loc, rloc, rq, rs, oe) = _rank_layer(cfg, m.RDG_CONTIGUOUS, block_m=128,
                                                                      signals=True, concurrent=True)
    # every row tile's counter reached the threshold exactly; unused counters stayed 0
    L = r["L"]
    rows = r["signal_rows"]
    sig = np_of(r["signals"])[:r["n_sig"]]
    off = np_of(L.offsets)
    mm = np_of(L.masked_m)
    want = np.zeros_like(sig)
    for e in range(len(mm)):
        for j in range((mm[e] + rows - 1) // rows):
            want[(off[e] + j * rows) // rows] = r["threshold"]
    assert np.array_equal(sig, want)
    # the signalled, concurrent run equals the plain sequential run bit for bit,
    # on every repeat (the overlap must not change a single bit), with the
    # polling combine alone and with the finishing form beside it
    r2 = run_routed(cfg, xq, x_s, loc, share["w_dev"], experts, m.RDG_CONTIGUOUS, block_m=128)
    for rep, finish, mb in ((0, False, 64), (1, True, 16), (2, True, 4)):
        r3 = run_routed(cfg, xq, x_s, loc, share["w_dev"], experts, m.RDG_CONTIGUOUS, block_m=128, signals=True,
                        concurrent=True, max_blocks=mb, finish=finish)
        assert m.rdg_check_status(r3["L"]) == (0, 0)
        ndiff = int((r3["out"] != r2["out"]).any(1).sum())
        print("repeat %d of the signalled run (finish=%s, %d polling workgroups): tokens differing from the "
              "sequential run: %d" % (rep, finish, mb, ndiff), flush=True)
        assert ndiff == 0
        del r3
    vr = _valid_rows(r2["L"])
    assert np.array_equal(vr, _valid_rows(L))
    same_h = torch.equal(r["h"][vr], r2["h"][vr])
    same_y = torch.equal(r["y"][vr], r2["y"][vr])
    diff_tok = np.flatnonzero((np_of(r["out"]) != np_of(r2["out"])).any(1))
    print("sbo vs sequential: h equal %s, y equal %s, tokens differing %d of %d" %
          (same_h, same_y, len(diff_tok), len(share["tokens"])), flush=True)
    if len(diff_tok):
        sel = diff_tok[:8]
        ref = oracle.moe_layer(dt_code(cfg), rq, rloc, share["w"], oe, x_scales=rs, sel=sel)
        for name, rr in (("signalled", r), ("sequential", r2)):
            got = np_of(rr["out"])[sel]
            rel = np.linalg.norm(out_as_f64(got) - out_as_f64(ref), axis=1) / np.linalg.norm(out_as_f64(ref), axis=1)
            print("  %s run, differing tokens %s: per-token rel err %s" % (name, sel.tolist(), np.round(rel, 4)),
                  flush=True)
        print("  local rows of those tokens:", (rloc[sel] >= 0).sum(1).tolist(), flush=True)
    assert same_h and same_y and len(diff_tok) == 0
    # shared expert on the rank's own tokens
    x_own = synth.x(cfg, cfg["own_tokens"], device=DEV, tensor=10)
    oq, os_ = quantize_act(x_own)
    shared = ExpertSet(cfg, [0], shared=True)
    ys = run_shared(cfg, oq, os_, shared)
    sel = _sample(cfg["own_tokens"], 16, 5)
    rq2, rs2 = oracle.quantize_fp8(np_of(x_own), 1)
    ref = oracle.moe_layer(oracle.FP8, rq2, np.full((cfg["own_tokens"], 1), -1, np.int32),
                           np.zeros((cfg["own_tokens"], 1), np.float32), [None], shared=shared.oracle_expert(0),
                           x_scales=rs2, sel=sel)
    err = oracle.rel_err(out_as_f64(np_of(ys)[sel]), out_as_f64(ref))
    print("prefill_rank_fp8 shared expert rel_err=%.3e" % err, flush=True)
    check_rows(np_of(ys)[sel], ref, cfg, "shared expert")
    assert err <= tolerance(cfg)


# Signalled down GEMM + concurrently polling combine on a small rank share:
# experts 8..15 of 32 are local, so many tokens have no local row (combined
# in the combine's second pass); the rows per local expert (about B*4/32)
# select 16-, 32-, 64- (fp32) and 128-row (bf16/fp8) tiles; contiguous and
# masked layouts.  The concurrent run must equal the sequential one bit for
# bit and the oracle within tolerance.
@pytest.mark.parametrize("dtype", ["f32", "bf16", "fp8", "fp8u"])
@pytest.mark.parametrize("B", [40, 300, 600])
@pytest.mark.parametrize("kind", [0, 1])
@pytest.mark.parametrize("finish", [False, True])
def test_sbo_small(dtype, B, kind, finish):
    _sbo_case(dtype, B, kind, finish)


# the 128-row signalled down GEMM takes the row tiles in groups of G in
# layout order, G = 4 raised until G x (column panels) is a multiple of 8:
# odd panel counts (G = 8) and tile counts that leave a partial last group
@pytest.mark.parametrize("dtype,H", [("fp8", 1280), ("fp8", 768), ("bf16", 1536), ("bf16", 1024), ("fp8u", 1280)])
@pytest.mark.parametrize("B", [1000, 1237])
def test_sbo_signal_order_groups(dtype, H, B):
    nt = _sbo_case(dtype, B, 0, True, H=H)
    panel = 512 if dtype == "bf16" else 256
    P = H // panel
    G = 4
    while (G * P) % 8:
        G += 1
    print("row tiles %d, panels %d, group %d" % (nt, P, G), flush=True)
    assert nt > G


def _sbo_case(dtype, B, kind, finish, H=512):
    m = rdg()
    cfg = _small_cfg(dtype, H=H, wid=500 + B + kind + H)
    dt = dt_code(cfg)
    logits = synth.logits(cfg, B)
    ids, w, ri, rw = _route(cfg, logits)
    p0, n_local = 8, 8
    loc_np = np.where((ri >= p0) & (ri < p0 + n_local), ri - p0, -1).astype(np.int32)
    loc = torch.from_numpy(loc_np).to(DEV)
    x = synth.x(cfg, B, device=DEV)
    x_s, xo, xo_s = None, np_of(x), None
    if is_fp8(cfg):
        x, x_s = quantize_act(x, dtype == "fp8u")
        xo, xo_s = oracle.quantize_fp8(xo, 1, ue8m0=dtype == "fp8u")
    experts = ExpertSet(cfg, range(p0, p0 + n_local))
    m_max = ((B + 127) // 128) * 128 if kind == m.RDG_MASKED else 0
    seq = run_routed(cfg, x, x_s, loc, w, experts, kind, block_m=128, m_max=m_max)
    sbo = run_routed(cfg, x, x_s, loc, w, experts, kind, block_m=128, m_max=m_max, signals=True, concurrent=True,
                     max_blocks=2 if finish else 8, finish=finish)
    assert m.rdg_check_status(sbo["L"]) == (0, 0)
    rows = sbo["signal_rows"]
    sig, off, mm = np_of(sbo["signals"])[:sbo["n_sig"]], np_of(sbo["L"].offsets), np_of(sbo["L"].masked_m)
    want = np.zeros_like(sig)
    for e in range(n_local):
        for j in range((mm[e] + rows - 1) // rows):
            want[(off[e] + j * rows) // rows] = sbo["threshold"]
    assert np.array_equal(sig, want)
    orphans = int((loc_np < 0).all(1).sum())
    ndiff = int((sbo["out"] != seq["out"]).any(1).sum())
    print("sbo small %s B=%d kind=%d finish=%s rows/signal=%d orphans=%d differing=%d"
          % (dtype, B, kind, finish, rows, orphans, ndiff), flush=True)
    assert orphans > 0 and ndiff == 0
    used = set(np.unique(loc_np[loc_np >= 0]).tolist())
    ref = oracle.moe_layer(dt, xo, loc_np, rw, [experts.oracle_expert(j) if j in used else None
                                                 for j in range(n_local)], x_scales=xo_s)
    got = np_of(sbo["out"])
    err = oracle.rel_err(out_as_f64(got), out_as_f64(ref))
    keep = np.flatnonzero((loc_np >= 0).any(1))
    check_rows(got[keep], ref[keep], cfg, "sbo small")
    assert not out_as_f64(got[(loc_np < 0).all(1)]).any(), "tokens without a local row must be zero"
    assert err <= tolerance(cfg), err
    return int(sum((int(v) + rows - 1) // rows for v in mm))


def test_sbo_timeout_is_reported_not_hung():
    """A threshold the producer can never reach: the combine gives up after
    its timeout, flags RDG_ETIMEOUT, and every kernel still exits."""
    m = rdg()
    cfg = _small_cfg("bf16", N=8, wid=77)
    B = 64
    logits = synth.logits(cfg, B)
    ids, w, ri, _ = _route(cfg, logits)
    x = synth.x(cfg, B, device=DEV)
    experts = ExpertSet(cfg, range(8))
    r = run_routed(cfg, x, None, ids, w, experts, m.RDG_CONTIGUOUS, block_m=128, signals=True)
    assert m.rdg_check_status(r["L"]) == (0, 0)
    out = torch.empty_like(r["out"])
    m.rdg_fill_i32(r["signals"][r["n_sig"]:], 0)  # the combine's unit counter starts again
    m.rdg_combine(r["y"], m.RDG_BF16, r["L"], w, B, cfg["K"], cfg["H"], None, out, m.RDG_BF16, r["signals"],
                  r["signal_rows"], r["threshold"] + 1, 2000, 4)
    code, detail = m.rdg_check_status(r["L"])
    assert code == m.RDG_ETIMEOUT
    assert 0 <= detail < r["n_sig"]
