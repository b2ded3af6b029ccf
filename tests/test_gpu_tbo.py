"""Two-batch overlap on one GPU: a batch of sequences cut by rdg_tbo_split
("Large-scale EP ..." page, TBO section), the two micro-batches run on two
streams at once, and every token's output checked against the oracle's layer
on the whole batch (the cut changes no token's result beyond rounding)."""
import numpy as np
import pytest
import torch

import oracle
import synth
from harness import DEV, ExpertSet, check_rows, dt_code, is_fp8, np_of, out_as_f64, quantize_act, rdg, run_routed, \
    tolerance

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype", ["bf16", "fp8u"])
def test_two_micro_batches(dtype):
    m = rdg()
    cfg = dict(wid=760, H=512, N=16, n_group=4, topk_group=2, K=4, I=256, shared_I=256, dtype=dtype, scale=1.0,
               logits="normal", name="tbo_" + dtype)
    lens = [90, 130, 40, 110]
    cut = sum(lens[:m.rdg_tbo_split(lens)])
    assert cut == 220   # 220 | 150 is the boundary closest to half of 370
    B = sum(lens)
    logits = synth.logits(cfg, B)
    ri, rw = oracle.route(logits, cfg["n_group"], cfg["topk_group"], cfg["K"], cfg["scale"])
    x = synth.x(cfg, B, device=DEV)
    x_s, xo, xo_s = None, np_of(x), None
    if is_fp8(cfg):
        x, x_s = quantize_act(x, dtype == "fp8u")
        xo, xo_s = oracle.quantize_fp8(xo, 1, ue8m0=dtype == "fp8u")
    experts = ExpertSet(cfg, range(cfg["N"]))
    ids = torch.from_numpy(ri).to(DEV)
    w = torch.from_numpy(rw).to(DEV)
    main, other = torch.cuda.current_stream(), torch.cuda.Stream()
    other.wait_stream(main)
    outs = []
    for (t0, t1), st in (((0, cut), main), ((cut, B), other)):
        with torch.cuda.stream(st):
            xs = x_s[t0:t1] if x_s is not None else None
            outs.append(run_routed(cfg, x[t0:t1], xs, ids[t0:t1], w[t0:t1], experts, m.RDG_CONTIGUOUS,
                                   block_m=128)["out"])
    main.wait_stream(other)
    got = np.concatenate([np_of(o) for o in outs])
    ref = oracle.moe_layer(dt_code(cfg), xo, ri, rw, [experts.oracle_expert(j) for j in range(cfg["N"])],
                           x_scales=xo_s)
    err = oracle.rel_err(out_as_f64(got), out_as_f64(ref))
    check_rows(got, ref, cfg, "tbo %s" % dtype)
    print("two micro-batches %s cut=%d rel_err=%.3e" % (dtype, cut, err), flush=True)
    assert err <= tolerance(cfg), err
