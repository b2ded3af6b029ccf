"""Benchmark of the MoE-layer hot path on one MI355X.

A step is one pass of the whole hot path over one batch: route -> dispatch
-> grouped gate/up GEMM (+SiLU-gated product) -> grouped down GEMM ->
combine, plus the shared expert, for the DeepSeek-V3-shaped decode layer with
every expert on this GPU (128 tokens, H=7168, 256 experts in 8 groups of 32,
4 groups kept, top-8, I=2048, shared expert I=2048, bf16, masked layout with
256 rows per expert).  Inputs are seeded synthetic tensors already resident
in HBM.  Prints one JSON line.

Extra fields: "roofline" for the dominant kernel (the grouped gate/up GEMM,
timed with HIP events on its own stream) and "cpu_baseline" (the CPU oracle
timed on a bounded sample of the same workload on this host).
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default="decode_bf16", choices=["decode_bf16"])
    p.add_argument("--cpu-tokens", type=int, default=16, help="tokens in the CPU-oracle sample (0: skip)")
    return p.parse_args()


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU's share of the layer; multi-GPU runs (--gpus %d) are not part of this "
              "build (the expert-parallel sharding is described, not implemented)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import routing_dispatch_grouped_amd as rdg
    import synth

    dev = "cuda:0"
    torch.cuda.set_device(0)
    cfg = synth.WORKLOADS[args.workload]
    B, H, N, K, I, shI = cfg["B"], cfg["H"], cfg["N"], cfg["K"], cfg["I"], cfg["shared_I"]
    m_max = cfg["m_max"]
    DT = rdg.RDG_BF16

    # ---------------------------------------------------------------- inputs (HBM-resident)
    logits_np = synth.logits(cfg)
    logits = torch.from_numpy(logits_np).to(dev)
    x = synth.x(cfg, B, device=dev)
    # weights are packed once into the grouped GEMMs' tile order (load time, not timed)
    W1 = torch.empty((N, I, H), dtype=torch.bfloat16, device=dev)
    W3 = torch.empty((N, I, H), dtype=torch.bfloat16, device=dev)
    W2 = torch.empty((N, H, I), dtype=torch.bfloat16, device=dev)
    for e in range(N):
        w = synth.expert_weights(cfg, e, device=dev)
        rdg.rdg_pack_weights(w["W1"], DT, W1[e]); rdg.rdg_pack_weights(w["W3"], DT, W3[e])
        rdg.rdg_pack_weights(w["W2"], DT, W2[e])
        del w
    sh = synth.expert_weights(cfg, 0, device=dev, shared=True)
    sW1, sW3, sW2 = (torch.empty_like(sh[k]).unsqueeze(0) for k in ("W1", "W3", "W2"))
    for k, dst in (("W1", sW1), ("W3", sW3), ("W2", sW2)):
        rdg.rdg_pack_weights(sh[k], DT, dst[0])

    # ---------------------------------------------------------------- buffers
    ids = torch.empty((B, K), dtype=torch.int32, device=dev)
    tw = torch.empty((B, K), dtype=torch.float32, device=dev)
    L = rdg.Layout(rdg.RDG_MASKED, N, B, K, dev, m_max=m_max)
    x_perm = torch.empty((L.m_cap, H), dtype=torch.bfloat16, device=dev)
    h = torch.empty((L.m_cap, I), dtype=torch.bfloat16, device=dev)
    y = torch.empty((L.m_cap, H), dtype=torch.bfloat16, device=dev)
    Ls = rdg.Layout(rdg.RDG_CONTIGUOUS, 1, B, 1, dev, block_m=16, m_cap=B)
    hs = torch.empty((B, shI), dtype=torch.bfloat16, device=dev)
    ys = torch.empty((B, H), dtype=torch.bfloat16, device=dev)
    out = torch.empty((B, H), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream()
    ev = []

    def step(timed=False):
        rdg.rdg_route(logits, cfg["n_group"], cfg["topk_group"], K, cfg["scale"], ids, tw)
        rdg.rdg_dispatch(x, None, DT, ids, L, x_perm)
        rdg.rdg_layout_dense(B, Ls)
        rdg.rdg_grouped_ffn(Ls, DT, H, shI, x, None, sW1, sW3, sW2, None, None, None, hs, None, ys)
        if timed:
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
        rdg.rdg_grouped_gate_up(L, DT, H, I, x_perm, None, W1, W3, None, None, h, None)
        if timed:
            e1.record(stream)
            ev.append((e0, e1))
        rdg.rdg_grouped_down(L, DT, H, I, h, None, W2, None, y)
        rdg.rdg_combine(y, DT, L, tw, B, K, H, ys, out, DT)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    code, detail = rdg.rdg_check_status(L)
    if code != 0:
        raise RuntimeError("device status %d (%s), detail %d" % (code, rdg.strerror(code), detail))
    active = int((L.masked_m > 0).sum().item())
    rows = int(L.masked_m.sum().item())

    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(timed=True)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms = (t1 - t0) * 1e3 / args.steps
    gate_ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))

    # algorithmic bytes of one gate/up launch: W1 and W3 of every active expert,
    # the routed rows of x_perm read once, h written once
    gate_bytes = active * 2 * I * H * 2 + rows * H * 2 + rows * I * 2
    achieved = gate_bytes / (gate_ms * 1e-3) / 1e9

    line = {
        "metric": "MoE-layer tokens/s on 1 MI355X",
        "value": B / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": args.workload, "tokens": B, "H": H, "experts": N, "n_group": cfg["n_group"],
                   "topk_group": cfg["topk_group"], "K": K, "I": I, "shared_I": shI, "layout": "masked",
                   "m_max": m_max, "active_experts": active, "routed_rows": rows},
        "roofline": {"kernel": "grouped gate/up GEMM (k_ffn, bf16, gated)", "bound": "hbm",
                     "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS,
                     "traffic": None, "avg_ms": gate_ms, "algorithmic_bytes": gate_bytes},
    }

    if args.cpu_tokens > 0:
        line["cpu_baseline"] = cpu_baseline(cfg, args.cpu_tokens, logits_np, x, sh, dev)
    print(json.dumps(line), flush=True)


def cpu_baseline(cfg, n_tok, logits_np, x, sh, dev):
    """The CPU oracle, as it stands, on a bounded sample of the same workload:
    routing of the whole batch and the layer output of the first n_tok tokens.
    Host copies of the needed inputs are made before the clock starts."""
    import numpy as np
    import torch

    import oracle

    def u16(t):
        return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)

    ri, rw = oracle.route(logits_np, cfg["n_group"], cfg["topk_group"], cfg["K"], cfg["scale"])
    sel = np.arange(n_tok, dtype=np.int32)
    used = set(np.unique(ri[sel]).tolist())
    import synth
    experts = [{k: u16(v) for k, v in synth.expert_weights(cfg, e, device=dev).items()} if e in used else None
               for e in range(cfg["N"])]
    shared = {k: u16(v) for k, v in sh.items()}
    xh = u16(x)
    t0 = time.perf_counter()
    ids, w = oracle.route(logits_np, cfg["n_group"], cfg["topk_group"], cfg["K"], cfg["scale"])
    oracle.layout(ids, cfg["N"], oracle.MASKED, m_max=cfg["m_max"])
    oracle.moe_layer(oracle.BF16, xh, ids, w, experts, shared=shared, sel=sel)
    dt = time.perf_counter() - t0
    return {"value": n_tok / dt, "unit": "tokens/s", "cores": oracle.num_threads(), "kind": "oracle",
            "seconds": dt,
            "sample": "route all %d tokens, layout, and the fp64 layer output (8 routed experts + shared) of "
                      "the first %d tokens" % (logits_np.shape[0], n_tok)}


if __name__ == "__main__":
    main()
