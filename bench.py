"""Benchmark of the MoE-layer hot path on one MI355X.

A step is one pass of the whole hot path over one batch of seeded synthetic
input already resident in HBM.  The default workload -- the one the JSON
line's value reports -- is the largest layer that runs on one GPU: the
DeepSeek-V3-shaped prefill layer with every expert on this GPU, 4096 tokens
(two 2048-token sequences), H=7168, 256 experts in 8 groups of 32, 4 groups
kept, top-8, I=2048, shared expert I=2048, bf16, expert popularity Zipf(1.1),
contiguous layout padded to 128 rows.  Its step: route -> dispatch ->
grouped gate/up GEMM (+SiLU-gated product) -> grouped down GEMM -> combine,
with the shared expert on a second stream overlapping everything before the
combine.

--workload selects another layer (tiny fp32, the 128-token decode layer, the
balanced prefill layer, and the fp8 decode / prefill rank shares with EPLB
remap; the prefill share overlaps its signalled down GEMM and the shared
expert with a polling combine on a second stream).

Extra fields: "roofline" for the dominant kernel (the grouped gate/up GEMM,
timed with HIP events on the stream it is launched on), "layer" (the whole
step against HBM), "cpu_baseline" (the CPU oracle timed on a bounded sample
of the same workload on this host), for the prefill layer "heavy_experts"
(the gate/up and down GEMMs over the experts with at least 315 rows, where
the bf16 MFMA rate can show), for the prefill rank share "sbo" (the step
with the signalled down GEMM and polling combine against the same step run
sequentially), and with the default workload "workloads": the same figures
for every other configuration, each measured in this run.
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
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0, "f32": 157.3}
DEFAULT_WORKLOAD = "prefill_bf16"
ALL_WORKLOADS = ["tiny_fp32", "decode_bf16", "prefill_bf16", "prefill_bf16_balanced", "decode_rank_fp8",
                 "prefill_rank_fp8"]
# tokens of the CPU oracle's FFN sample per workload (routing / remap and the
# layout always cover the whole batch); chosen for a few to about 20 seconds
# of oracle time on 16 host threads
CPU_TOKENS = {"tiny_fp32": -1, "decode_bf16": -1, "prefill_bf16": 192, "prefill_bf16_balanced": 96,
              "decode_rank_fp8": 256, "prefill_rank_fp8": 256}
# polling-combine workgroups of the signalled step (prefill rank share)
POLL_BLOCKS = 8
SUMMARY_CPU_TOKENS = {"tiny_fp32": -1, "decode_bf16": 32, "prefill_bf16_balanced": 0, "decode_rank_fp8": 64,
                      "prefill_rank_fp8": 64, "prefill_bf16": 48}


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default=DEFAULT_WORKLOAD, choices=ALL_WORKLOADS)
    p.add_argument("--summary", choices=["auto", "on", "off"], default="auto",
                   help="also measure every other workload and report it under 'workloads' (auto: with the "
                        "default workload and no variant flags)")
    p.add_argument("--extras", choices=["on", "off"], default="on",
                   help="the measurements after the timed steps: heavy_experts (prefill layers), the two "
                        "dispatch forms on their own, and the sbo comparison (prefill rank share); off for a "
                        "kernel trace of the timed steps alone")
    p.add_argument("--payload", choices=["gather", "copy"], default="gather",
                   help="dispatch payload: gather (the dispatch builds the layout only and the gate/up GEMM reads "
                        "each row's token through row_src) or copy (rows permuted into x_perm by the dispatch)")
    p.add_argument("--graph", action="store_true",
                   help="time replays of the step captured in a HIP graph (full-layer workloads); the gate/up "
                        "kernel's own time then comes from as many eager steps run after them")
    p.add_argument("--ue8m0", action="store_true",
                   help="fp8 workloads with power-of-two block scales (scaled-MFMA path)")
    p.add_argument("--eplb-replicas", choices=["greedy", "one_each"], default=None,
                   help="rank shares: the EPLB plan's replica rule (default greedy: each of the 32 redundant "
                        "copies to the expert with the largest expected load per copy)")
    p.add_argument("--side-cus", type=int, default=0,
                   help="full layers: the shared expert's stream may use only this many CUs, spread evenly over "
                        "the GPU (a CU-masked stream); 0: all CUs")
    p.add_argument("--tbo", action="store_true",
                   help="prefill layers as two micro-batches cut at a sequence boundary, on two streams "
                        "(the roofline then covers micro-batch A's gate/up)")
    p.add_argument("--poll-blocks", type=int, default=POLL_BLOCKS,
                   help="polling-combine workgroups in the signalled step (prefill rank share)")
    p.add_argument("--cpu-tokens", type=int, default=None,
                   help="tokens in the CPU-oracle FFN sample (-1: the whole batch; 0: skip; default per workload)")
    p.add_argument("--calibrate-copy", action="store_true",
                   help="after the timed region, copy 1 GiB device-to-device twice (a plain copy kernel of known "
                        "size, for scaling the FETCH_SIZE / WRITE_SIZE counters of a profiling run)")
    return p.parse_args()


# Files whose contents determine the dominant kernel's memory traffic (the
# kernel, its device helpers and the packed weight layout); the committed
# counter figures apply only while their hash is unchanged.
# the sources that decide the dominant kernel's memory traffic: its kernel
# file (the 16-64-row kernels for the decode and tiny layers, the 128-row
# tiles for the prefill layers and the rank shares), the shared helpers, the
# weight packing, and the kernel choice in the C ABI
TRAFFIC_COMMON = ["routing_dispatch_grouped_amd/csrc/rdg_internal.h", "routing_dispatch_grouped_amd/csrc/pack.hip",
                  "routing_dispatch_grouped_amd/csrc/abi.hip"]
TRAFFIC_KERNEL = {"decode_bf16": "routing_dispatch_grouped_amd/csrc/ffn.hip",
                  "tiny_fp32": "routing_dispatch_grouped_amd/csrc/ffn.hip"}


def traffic_sources(workload):
    return [TRAFFIC_KERNEL.get(workload, "routing_dispatch_grouped_amd/csrc/ffn_tiled.hip")] + TRAFFIC_COMMON


def source_hash(workload):
    import hashlib
    h = hashlib.sha256()
    for f in traffic_sources(workload):
        h.update(open(os.path.join(ROOT, f), "rb").read())
    return h.hexdigest()[:16]


def measured_traffic(workload):
    """HBM bytes per launch of the dominant kernel from the committed
    rocprofv3 counter summary (profiles/traffic_<workload>.txt), or None when
    it is missing or was taken on other kernel sources."""
    path = os.path.join(ROOT, "profiles", "traffic_%s.txt" % workload)
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("source_hash") != source_hash(workload):
        return None
    try:
        return float(kv["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cu_masked_stream(n_cus):
    """A stream whose kernels may run only on n_cus of the GPU's CUs, spread
    evenly (hipExtStreamCreateWithCUMask, default priority), as a torch
    external stream."""
    import ctypes

    import torch
    # the HIP runtime already loaded in this process (torch's), not a second copy
    path = "libamdhip64.so"
    for line in open("/proc/self/maps"):
        if "libamdhip64" in line:
            path = line.split()[-1]
            break
    hip = ctypes.CDLL(path)
    hip.hipExtStreamCreateWithCUMask.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint32,
                                                 ctypes.POINTER(ctypes.c_uint32)]
    total = torch.cuda.get_device_properties(0).multi_processor_count
    n_cus = max(1, min(n_cus, total))
    words = (ctypes.c_uint32 * ((total + 31) // 32))()
    for j in range(n_cus):
        cu = j * total // n_cus
        words[cu // 32] |= 1 << (cu % 32)
    stream = ctypes.c_void_p()
    rc = hip.hipExtStreamCreateWithCUMask(ctypes.byref(stream), len(words), words)
    if rc != 0:
        raise RuntimeError("hipExtStreamCreateWithCUMask failed (%d)" % rc)
    return torch.cuda.ExternalStream(stream.value)


def layer_bytes(cfg, T, R, A, esz, gather=False):
    """Algorithmic HBM bytes of one whole step (every kernel's reads and
    writes counted once: no padding, no unused masked capacity): routing (or,
    for a rank's share, the replica remap), the stable ranks and the row
    permutation, the routed gate/up and down GEMMs, the shared expert where
    there is one, and the combine.  fp8 block scales are 4-byte floats.
    gather: the permutation only publishes pos and row_src, and the gate/up
    GEMM reads the R rows' tokens through them (counted with the GEMM)."""
    H, I, K, N = cfg["H"], cfg["I"], cfg["K"], cfg["N"]
    ysz = 4 if cfg["dtype"] == "f32" else 2
    sc = 4 if cfg["dtype"] == "fp8" else 0
    rank = "B_global" in cfg
    shI = cfg.get("shared_I", 0)
    Tsh = cfg.get("own_tokens", T) if rank else T
    b = T * K * 8 + T * 8 if rank else T * N * 4 + T * K * 8            # remap / route
    b += T * K * 8                                                       # stable ranks
    if gather:
        b += T * K * 4 + R * 4                                           # publish pos, row_src
    else:
        b += T * H * esz + R * H * esz + (T + R) * (H // 128) * sc       # permute rows
    b += A * 2 * I * H * esz + A * 2 * (I // 128) * (H // 128) * sc + R * (H + I) * esz + R * (H + I) // 128 * sc
    b += A * I * H * esz + A * (I // 128) * (H // 128) * sc + R * (I * esz + H * ysz) + R * (I // 128) * sc
    if shI:
        b += 3 * shI * H * esz + 3 * (shI // 128) * (H // 128) * sc + Tsh * (2 * H + 2 * shI) * esz
        b += Tsh * H * (ysz - esz)
    b += R * H * ysz + T * H * ysz + (T * H * ysz if (shI and not rank) else 0)  # combine
    return b


class Bench:
    """Buffers and the step of one workload."""

    def __init__(self, name, dev, ue8m0=False, tbo=False, replicas=None, side_cus=0, side_stream=None,
                 payload="gather"):
        import torch

        import routing_dispatch_grouped_amd as rdg
        import synth
        self.torch, self.rdg, self.synth = torch, rdg, synth
        self.name, self.dev = name, dev
        self.cfg = cfg = dict(synth.WORKLOADS[name])
        if replicas and "B_global" in cfg:
            cfg["replicas"] = replicas
        # prefill rank share: "signalled" (down GEMM publishes row tiles, a
        # polling combine overlaps it) or "sequential" (plain down GEMM, then
        # a plain combine on the same stream)
        self.sbo_mode = "signalled"
        self.DT = {"f32": rdg.RDG_F32, "bf16": rdg.RDG_BF16, "fp8": rdg.RDG_FP8_E4M3}[cfg["dtype"]]
        # fp8 with power-of-two block scales: same codes and layouts, scales
        # applied inside the scaled MFMA by the 128-row kernels
        self.ue8m0 = ue8m0 and cfg["dtype"] == "fp8"
        self.fp8 = cfg["dtype"] == "fp8"
        self.quant = rdg.rdg_quantize_fp8_ue8m0 if self.ue8m0 else rdg.rdg_quantize_fp8
        if self.ue8m0:
            self.DT = rdg.RDG_FP8_E4M3_UE8M0
        self.sdt = {"f32": torch.float32, "bf16": torch.bfloat16, "fp8": torch.uint8}[cfg["dtype"]]
        self.ydt = torch.float32 if cfg["dtype"] == "f32" else torch.bfloat16
        self.YDT = rdg.RDG_F32 if cfg["dtype"] == "f32" else rdg.RDG_BF16
        self.events = []
        # gather: the dispatch builds the layout only and the gate/up GEMM
        # reads the tokens through row_src; copy: rows permuted into x_perm
        self.gather = payload == "gather"
        self.stream = torch.cuda.current_stream()
        self.rank = "B_global" in cfg
        self.tbo = None
        self.side_cus = side_cus
        if self.rank:
            self._setup_rank()
        else:
            self._setup_full()
            if side_cus:
                self.side = side_stream if side_stream is not None else cu_masked_stream(side_cus)
            if tbo:
                self._setup_tbo()
        self._setup_rotation()

    # ------------------------------------------------------------ weights
    def _experts(self, ids, shared=False):
        """Packed device weights for the listed logical experts (+ fp8 scales)."""
        torch, rdg, synth, cfg = self.torch, self.rdg, self.synth, self.cfg
        H = cfg["H"]
        I = cfg["shared_I"] if shared else cfg["I"]
        n = len(ids)
        W = {k: torch.empty(shape, dtype=self.sdt, device=self.dev)
             for k, shape in (("W1", (n, I, H)), ("W3", (n, I, H)), ("W2", (n, H, I)))}
        S = {}
        if self.fp8:
            S = {k: torch.empty(shape, dtype=torch.float32, device=self.dev)
                 for k, shape in (("W1", (n, I // 128, H // 128)), ("W3", (n, I // 128, H // 128)),
                                  ("W2", (n, H // 128, I // 128)))}
        for j, e in enumerate(ids):
            w = synth.expert_weights(cfg, e, device=self.dev, shared=shared)
            for k in ("W1", "W3", "W2"):
                src = w[k]
                if S:
                    q = torch.empty(src.shape, dtype=torch.uint8, device=self.dev)
                    self.quant(src, rdg.RDG_F32, 128, q, S[k][j])
                    src = q
                rdg.rdg_pack_weights(src, self.DT, W[k][j])
            del w
        return W, S

    def _setup_rotation(self):
        """Weights that fit the 256 MB last-level cache would be served from it
        by the next step: such workloads get copies of their expert weights
        (at least four, together at least 1 GiB), used in turn, one per step,
        so that every step reads its weights from HBM."""
        torch = self.torch
        sets = [(self.W, self.S, getattr(self, "Wsh", {}), getattr(self, "Ssh", {}))]
        nbytes = sum(t.numel() * t.element_size() for d in sets[0] for t in d.values())
        n_sets = 1
        if nbytes < (1 << 30):
            n_sets = max(4, -(-(1 << 30) // nbytes))
        for _ in range(n_sets - 1):
            sets.append(tuple({k: v.clone() for k, v in d.items()} for d in sets[0]))
        torch.cuda.synchronize()
        self.weight_sets, self.weight_set_bytes, self.step_index = sets, nbytes, 0

    def _next_weights(self):
        sets = self.weight_sets
        self.W, self.S, Wsh, Ssh = sets[self.step_index % len(sets)]
        if Wsh:
            self.Wsh, self.Ssh = Wsh, Ssh
        self.step_index += 1

    def _quant(self, x):
        torch, rdg = self.torch, self.rdg
        q = torch.empty(x.shape, dtype=torch.uint8, device=self.dev)
        s = torch.empty((x.shape[0], x.shape[1] // 128), dtype=torch.float32, device=self.dev)
        self.quant(x, rdg.RDG_BF16, 1, q, s)
        return q, s

    def _buffers(self, T, K, n_local, kind, block_m=128, m_max=0):
        torch, rdg, cfg = self.torch, self.rdg, self.cfg
        H, I = cfg["H"], cfg["I"]
        self.L = rdg.Layout(kind, n_local, T, K, self.dev, block_m=block_m, m_max=m_max)
        m_cap = self.L.m_cap
        self.h = torch.empty((m_cap, I), dtype=self.sdt, device=self.dev)
        self.y = torch.empty((m_cap, H), dtype=self.ydt, device=self.dev)
        fp8 = self.fp8
        self.x_perm = self.x_perm_s = None
        if not self.gather:
            self.x_perm = torch.empty((m_cap, H), dtype=self.sdt, device=self.dev)
            self.x_perm_s = torch.empty((m_cap, H // 128), dtype=torch.float32, device=self.dev) if fp8 else None
        self.h_s = torch.empty((m_cap, I // 128), dtype=torch.float32, device=self.dev) if fp8 else None

    def _shared_buffers(self, T):
        torch, rdg, cfg = self.torch, self.rdg, self.cfg
        shI = cfg["shared_I"]
        self.Ls = rdg.Layout(rdg.RDG_CONTIGUOUS, 1, T, 1, self.dev, block_m=16, m_cap=T)
        self.hs = torch.empty((T, shI), dtype=self.sdt, device=self.dev)
        self.hs_s = (torch.empty((T, shI // 128), dtype=torch.float32, device=self.dev)
                     if self.fp8 else None)
        self.ys = torch.empty((T, cfg["H"]), dtype=self.ydt, device=self.dev)

    def _setup_full(self):
        torch, rdg, synth, cfg = self.torch, self.rdg, self.synth, self.cfg
        B, N, K = cfg["B"], cfg["N"], cfg["K"]
        self.T = B
        self.logits_np = synth.logits(cfg)
        self.logits = torch.from_numpy(self.logits_np).to(self.dev)
        self.x = synth.x(cfg, B, device=self.dev)
        self.x_s = None
        self.W, self.S = self._experts(range(N))
        self.Wsh, self.Ssh = self._experts([0], shared=True)
        self.ids = torch.empty((B, K), dtype=torch.int32, device=self.dev)
        self.tw = torch.empty((B, K), dtype=torch.float32, device=self.dev)
        kind = rdg.RDG_MASKED if cfg["layout"] == "masked" else rdg.RDG_CONTIGUOUS
        self._buffers(B, K, N, kind, block_m=128 if kind == rdg.RDG_CONTIGUOUS else 128, m_max=cfg.get("m_max", 0))
        self._shared_buffers(B)
        self.side = torch.cuda.Stream()
        self.overlap_shared = cfg["H"] >= 1024
        self.out = torch.empty((B, cfg["H"]), dtype=self.ydt, device=self.dev)

    def _setup_tbo(self):
        """Two micro-batches cut at a sequence boundary (rdg_tbo_split), each with
        its own layout and buffers; the second runs on a stream of its own."""
        torch, rdg, cfg = self.torch, self.rdg, self.cfg
        if "seq_lens" not in cfg:
            raise SystemExit("--tbo needs a workload made of sequences (the prefill layers)")
        lens = cfg["seq_lens"]
        cut = sum(lens[:rdg.rdg_tbo_split(lens)])
        H, I, K, N = cfg["H"], cfg["I"], cfg["K"], cfg["N"]
        self.tbo = []
        for t0, t1 in ((0, cut), (cut, self.T)):
            T = t1 - t0
            L = rdg.Layout(rdg.RDG_CONTIGUOUS, N, T, K, self.dev, block_m=128)
            mb = dict(t0=t0, T=T, L=L, x=self.x[t0:t1], logits=self.logits[t0:t1], ids=self.ids[t0:t1],
                      tw=self.tw[t0:t1], out=self.out[t0:t1], ys=self.ys[t0:t1],
                      x_perm=(None if self.gather else torch.empty((L.m_cap, H), dtype=self.sdt, device=self.dev)),
                      h=torch.empty((L.m_cap, I), dtype=self.sdt, device=self.dev),
                      y=torch.empty((L.m_cap, H), dtype=self.ydt, device=self.dev))
            self.tbo.append(mb)
        self.tbo_stream = torch.cuda.Stream()
        self.L = self.tbo[0]["L"]   # statistics and the roofline: micro-batch A

    def _step_tbo(self, timed):
        """Shared expert on the side stream; micro-batch A's stages on this
        stream and B's on another, issued alternately so that each one's
        routing, dispatch and combine can run beside the other's GEMMs."""
        rdg, cfg, torch = self.rdg, self.cfg, self.torch
        H, I, K = cfg["H"], cfg["I"], cfg["K"]
        main = torch.cuda.current_stream()
        self.side.wait_stream(main)
        self.tbo_stream.wait_stream(main)
        with torch.cuda.stream(self.side):
            self._shared(self.x, None, self.T, stream=self.side)
        A, B = self.tbo
        sB = self.tbo_stream
        for mb, st in ((A, main), (B, sB)):
            with torch.cuda.stream(st):
                rdg.rdg_route(mb["logits"], cfg["n_group"], cfg["topk_group"], K, cfg["scale"], mb["ids"], mb["tw"],
                              stream=st)
                rdg.rdg_dispatch(mb["x"], None, self.DT, mb["ids"], mb["L"], mb["x_perm"], stream=st)
        for mb, st in ((A, main), (B, sB)):
            with torch.cuda.stream(st):
                if timed and mb is A:
                    e0 = torch.cuda.Event(enable_timing=True)
                    e1 = torch.cuda.Event(enable_timing=True)
                    e0.record(st)
                if self.gather:
                    rdg.rdg_grouped_gate_up_gather(mb["L"], self.DT, H, I, mb["x"], None, K, self.W["W1"],
                                                   self.W["W3"], None, None, mb["h"], None, stream=st)
                else:
                    rdg.rdg_grouped_gate_up(mb["L"], self.DT, H, I, mb["x_perm"], None, self.W["W1"], self.W["W3"],
                                            None, None, mb["h"], None, stream=st)
                if timed and mb is A:
                    e1.record(st)
                    self.events.append((e0, e1))
                rdg.rdg_grouped_down(mb["L"], self.DT, H, I, mb["h"], None, self.W["W2"], None, mb["y"], stream=st)
        for mb, st in ((A, main), (B, sB)):
            with torch.cuda.stream(st):
                st.wait_stream(self.side)
                rdg.rdg_combine(mb["y"], self.YDT, mb["L"], mb["tw"], mb["T"], K, H, mb["ys"], mb["out"], self.YDT,
                                stream=st)
        main.wait_stream(sB)

    def _setup_rank(self):
        """One rank's received share: the global batch is routed and remapped on
        the device once (setup, untimed) to find the rows this rank receives."""
        torch, rdg, synth, cfg = self.torch, self.rdg, self.synth, self.cfg
        import numpy as np
        K = cfg["K"]
        plan = synth.eplb_plan(cfg)
        self.plan = plan
        lg = torch.from_numpy(synth.logits(cfg)).to(self.dev)
        Tg = lg.shape[0]
        gids = torch.empty((Tg, K), dtype=torch.int32, device=self.dev)
        gw = torch.empty((Tg, K), dtype=torch.float32, device=self.dev)
        rdg.rdg_route(lg, cfg["n_group"], cfg["topk_group"], K, cfg["scale"], gids, gw)
        self.l2p = torch.from_numpy(plan["log2phy"]).to(self.dev)
        self.nrep = torch.from_numpy(plan["n_replica"]).to(self.dev)
        gidx = torch.arange(Tg, dtype=torch.int64, device=self.dev)
        loc = torch.empty_like(gids)
        # the measured rank: the one that receives the most rows of the global batch
        rows = []
        for r in range(cfg["n_ranks"]):
            rdg.rdg_eplb_remap(gids, gidx, self.l2p, self.nrep, r * plan["n_local"], plan["n_local"], loc)
            rows.append(int((loc >= 0).sum()))
        self.plan = plan = synth.measured_rank(plan, rows)
        self.rank_rows = rows
        rdg.rdg_eplb_remap(gids, gidx, self.l2p, self.nrep, plan["phys_begin"], plan["n_local"], loc)
        loc_np = loc.cpu().numpy()
        toks, keep = synth.take_rank_rows(loc_np, cfg["rows"])
        ids = gids.cpu().numpy()[toks]
        ids[~keep & (loc_np[toks] >= 0)] = -1
        sel = torch.from_numpy(toks).to(self.dev)
        self.T = T = len(toks)
        self.ids = torch.from_numpy(ids).to(self.dev)
        self.tw = gw[sel].contiguous()
        self.gidx = gidx[sel].contiguous()
        self.local = torch.empty_like(self.ids)
        self.x, self.x_s = self._quant(synth.x(cfg, T, device=self.dev))
        phys2log = np.full(cfg["n_ranks"] * cfg["n_local"], -1)
        for e in range(cfg["N"]):
            for r in range(plan["n_replica"][e]):
                phys2log[plan["log2phy"][e, r]] = e
        self.local_logical = [int(phys2log[plan["phys_begin"] + s]) for s in range(plan["n_local"])]
        self.W, self.S = self._experts(self.local_logical)
        kind = rdg.RDG_MASKED if cfg["layout"] == "masked" else rdg.RDG_CONTIGUOUS
        self._buffers(T, K, plan["n_local"], kind, block_m=128, m_max=cfg.get("m_max", 0))
        self.out = torch.empty((T, cfg["H"]), dtype=self.ydt, device=self.dev)
        self.signals = None
        if cfg.get("signals"):
            rows = rdg.rdg_signal_rows(self.L, self.DT, cfg["H"], cfg["I"])
            self.signal_rows = rows
            # the row tiles' counters, then the combine's unit counter and first finishing unit
            self.signals = torch.zeros(((self.L.m_cap + rows - 1) // rows + 2,), dtype=torch.int32, device=self.dev)
            self.threshold = rdg.rdg_signal_threshold(cfg["H"], self.DT)
            # the polling combine's workgroups: they take the tokens of the row
            # tiles that complete while the down GEMM runs, and the finishing
            # combine after the GEMM takes the rest
            self.poll_blocks = POLL_BLOCKS
            self.side = torch.cuda.Stream()
            self.gate_done = torch.cuda.Event()
        if cfg.get("shared_I"):
            self.x_own, self.x_own_s = self._quant(synth.x(cfg, cfg["own_tokens"], device=self.dev, tensor=10))
            self.Wsh, self.Ssh = self._experts([0], shared=True)
            self._shared_buffers(cfg["own_tokens"])

    # ------------------------------------------------------------ step
    def _gate_up(self, timed):
        rdg, cfg = self.rdg, self.cfg
        if timed:
            e0 = self.torch.cuda.Event(enable_timing=True)
            e1 = self.torch.cuda.Event(enable_timing=True)
            e0.record(self.torch.cuda.current_stream())
        if self.gather:
            rdg.rdg_grouped_gate_up_gather(self.L, self.DT, cfg["H"], cfg["I"], self.x, self.x_s, cfg["K"],
                                           self.W["W1"], self.W["W3"], self.S.get("W1"), self.S.get("W3"), self.h,
                                           self.h_s)
        else:
            rdg.rdg_grouped_gate_up(self.L, self.DT, cfg["H"], cfg["I"], self.x_perm, self.x_perm_s, self.W["W1"],
                                    self.W["W3"], self.S.get("W1"), self.S.get("W3"), self.h, self.h_s)
        if timed:
            e1.record(self.torch.cuda.current_stream())
            self.events.append((e0, e1))

    def _shared(self, x, x_s, T, stream=None):
        rdg, cfg = self.rdg, self.cfg
        rdg.rdg_layout_dense(T, self.Ls, stream=stream)
        rdg.rdg_grouped_ffn(self.Ls, self.DT, cfg["H"], cfg["shared_I"], x, x_s, self.Wsh["W1"], self.Wsh["W3"],
                            self.Wsh["W2"], self.Ssh.get("W1"), self.Ssh.get("W3"), self.Ssh.get("W2"), self.hs,
                            self.hs_s, self.ys, stream=stream)

    def step(self, timed=False):
        rdg, cfg = self.rdg, self.cfg
        H, I, K = cfg["H"], cfg["I"], cfg["K"]
        self._next_weights()
        if self.tbo:
            return self._step_tbo(timed)
        if not self.rank:
            # at DeepSeek-V3 sizes the shared expert runs on a second stream and
            # the combine waits for both streams; for the tiny layer the
            # cross-stream wait costs more than the overlap saves, so it runs in
            # line.  Decode layer: launched first, beside routing, dispatch and
            # the routed GEMMs.  Prefill layers: launched once the routed gate/up
            # is done, beside the routed down GEMM (steps 0.2-0.5% faster than
            # launched first; the gate/up then runs alone).  (The stream is the
            # current one, so that the step can also be captured.)
            main = self.torch.cuda.current_stream()
            late = self.overlap_shared and cfg["layout"] == "contiguous"
            if self.overlap_shared and not late:
                self.side.wait_stream(main)
                with self.torch.cuda.stream(self.side):
                    self._shared(self.x, None, self.T, stream=self.side)
            elif not self.overlap_shared:
                self._shared(self.x, None, self.T)
            rdg.rdg_route(self.logits, cfg["n_group"], cfg["topk_group"], K, cfg["scale"], self.ids, self.tw)
            rdg.rdg_dispatch(self.x, None, self.DT, self.ids, self.L, self.x_perm)  # gather: x_perm None
            self._gate_up(timed)
            if late:
                self.side.wait_stream(main)
                with self.torch.cuda.stream(self.side):
                    self._shared(self.x, None, self.T, stream=self.side)
            rdg.rdg_grouped_down(self.L, self.DT, H, I, self.h, self.h_s, self.W["W2"], self.S.get("W2"), self.y)
            if self.overlap_shared:
                main.wait_stream(self.side)
            rdg.rdg_combine(self.y, self.YDT, self.L, self.tw, self.T, K, H, self.ys, self.out, self.YDT)
            return
        plan = self.plan
        rdg.rdg_eplb_remap(self.ids, self.gidx, self.l2p, self.nrep, plan["phys_begin"], plan["n_local"], self.local)
        rdg.rdg_dispatch(self.x, self.x_s if not self.gather else None, self.DT, self.local, self.L, self.x_perm,
                         self.x_perm_s)
        if self.signals is None:
            self._gate_up(timed)
            rdg.rdg_grouped_down(self.L, self.DT, H, I, self.h, self.h_s, self.W["W2"], self.S.get("W2"), self.y)
            rdg.rdg_combine(self.y, self.YDT, self.L, self.tw, self.T, K, H, None, self.out, self.YDT)
            return
        # The shared expert (on the rank's own tokens) runs on the side stream
        # once the routed gate/up is done, beside the down GEMM: 3% faster
        # steps than beside the gate/up with fp32 scales, equal with
        # power-of-two scales.
        if self.sbo_mode == "sequential":
            # the same step without the overlap: down GEMM and a plain combine
            self._gate_up(timed)
            self.side.wait_stream(self.stream)
            with self.torch.cuda.stream(self.side):
                self._shared(self.x_own, self.x_own_s, cfg["own_tokens"], stream=self.side)
            rdg.rdg_grouped_down(self.L, self.DT, H, I, self.h, self.h_s, self.W["W2"], self.S.get("W2"), self.y)
            rdg.rdg_combine(self.y, self.YDT, self.L, self.tw, self.T, K, H, None, self.out, self.YDT)
            self.stream.wait_stream(self.side)
            return
        # signalled down GEMM on this stream, then the finishing combine; on
        # the side stream, once gate/up is done, the shared expert and then
        # the polling combine (it takes the row tiles that complete while it
        # runs; the finishing combine closes its counter and takes the rest)
        rdg.rdg_fill_i32(self.signals, 0)
        self._gate_up(timed)
        self.gate_done.record(self.stream)
        rdg.rdg_grouped_down(self.L, self.DT, H, I, self.h, self.h_s, self.W["W2"], self.S.get("W2"), self.y,
                             self.signals)
        rdg.rdg_combine_finish(self.y, self.YDT, self.L, self.tw, self.T, K, H, None, self.out, self.YDT, self.signals,
                               self.signal_rows)
        with self.torch.cuda.stream(self.side):
            self.side.wait_event(self.gate_done)
            self._shared(self.x_own, self.x_own_s, cfg["own_tokens"], stream=self.side)
            rdg.rdg_combine(self.y, self.YDT, self.L, self.tw, self.T, K, H, None, self.out, self.YDT, self.signals,
                            self.signal_rows, self.threshold, 1_000_000, self.poll_blocks, stream=self.side)
        self.stream.wait_stream(self.side)


def _ms_steps(b, steps, timed=True):
    """Wall-clock ms per step over `steps` steps (synchronised on both
    sides) and the mean gate/up kernel time recorded on its stream."""
    torch = b.torch
    b.events = []
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        b.step(timed=timed)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    gate = None
    if b.events:
        import numpy as np
        gate = float(np.mean([a.elapsed_time(e) for a, e in b.events]))
    return (t1 - t0) * 1e3 / steps, gate


def _stats(b):
    rdg = b.rdg
    code, detail = rdg.rdg_check_status(b.L)
    if code != 0:
        raise RuntimeError("device status %d (%s), detail %d" % (code, rdg.strerror(code), detail))
    masked_m = b.L.masked_m.cpu().numpy()
    counts = b.L.counts.cpu().numpy()
    # load balance of the local experts, mean / max of their routed rows (the
    # statistic expert-load rebalancing raises)
    balance = float(counts.mean() / counts.max()) if counts.max() > 0 else 1.0
    return int((masked_m > 0).sum()), int(masked_m.sum()), balance, masked_m


def _roofline(cfg, active, rows, gate_ms, workload):
    """Roofline of one gate/up launch: algorithmic bytes (W1 and W3 of every
    active expert, + fp8 block scales; the routed rows' tokens read once, h
    written once) and flops 4 R H I; the bound is whichever of bytes / 8 TB/s
    and flops / MFMA peak is the longer."""
    H, I = cfg["H"], cfg["I"]
    esz = {"f32": 4, "bf16": 2, "fp8": 1}[cfg["dtype"]]
    gate_bytes = active * 2 * I * H * esz + rows * H * esz + rows * I * esz
    if esz == 1:
        gate_bytes += active * 2 * (I // 128) * (H // 128) * 4 + rows * (H // 128 + I // 128) * 4
    gate_flops = 2 * 2 * rows * H * I
    gbps = gate_bytes / (gate_ms * 1e-3) / 1e9
    tflops = gate_flops / (gate_ms * 1e-3) / 1e12
    peak_f = MFMA_PEAK_TFLOPS[cfg["dtype"]]
    hbm_frac, mfma_frac = gbps / HBM_PEAK_GBPS, tflops / peak_f
    hbm_bound = gate_bytes / (HBM_PEAK_GBPS * 1e9) >= gate_flops / (peak_f * 1e12)
    return {"kernel": "grouped gate/up GEMM + SiLU-gated product (%s)" % cfg["dtype"],
            "bound": "hbm" if hbm_bound else "mfma",
            "achieved": gbps if hbm_bound else tflops, "peak": HBM_PEAK_GBPS if hbm_bound else peak_f,
            "unit": "GB/s" if hbm_bound else "TFLOP/s", "frac": hbm_frac if hbm_bound else mfma_frac,
            "traffic": measured_traffic(workload), "avg_ms": gate_ms, "algorithmic_bytes": gate_bytes,
            "algorithmic_flops": gate_flops, "source_hash": source_hash(workload),
            "hbm_frac": hbm_frac, "mfma_frac": mfma_frac}


def measure(b, args, steps, warmup, workload):
    """Warm-up, the timed steps, and the JSON fields of one workload."""
    torch, cfg = b.torch, b.cfg
    for _ in range(warmup):
        b.step()
    torch.cuda.synchronize()
    active, rows, balance, _ = _stats(b)
    if args.graph:
        if b.rank:
            raise SystemExit("--graph covers the full-layer workloads")
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            b.step()
        graph.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            graph.replay()
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1e3 / steps
        _, gate_ms = _ms_steps(b, steps)
    else:
        ms, gate_ms = _ms_steps(b, steps)
    H, I, K = cfg["H"], cfg["I"], cfg["K"]
    esz = {"f32": 4, "bf16": 2, "fp8": 1}[cfg["dtype"]]
    roof = _roofline(cfg, active, rows, gate_ms, workload)
    if b.rank:
        metric, unit = "MoE-layer token-equivalents/s (received rows / K) on 1 MI355X", "token-equivalents/s"
        value = rows / K / (ms * 1e-3)
    else:
        metric, unit = "MoE-layer tokens/s on 1 MI355X", "tokens/s"
        value = b.T / (ms * 1e-3)
    conf = {"workload": workload, "tokens": b.T, "H": H, "I": I, "K": K, "experts": cfg["N"],
            "n_group": cfg["n_group"], "topk_group": cfg["topk_group"], "shared_I": cfg["shared_I"],
            "layout": cfg["layout"], "active_experts": active, "routed_rows": rows,
            "load_balance_mean_over_max": round(balance, 4), "graph": bool(args.graph),
            "weight_sets": len(b.weight_sets),
            "dispatch_payload": "gathered by the gate/up GEMM" if b.gather else "copied into x_perm"}
    if b.tbo:
        conf["tbo_micro_batches"] = [mb["T"] for mb in b.tbo]
    if b.side_cus:
        conf["shared_expert_cus"] = b.side_cus
    if b.fp8:
        conf["fp8_scales"] = "ue8m0 (power of two)" if b.ue8m0 else "fp32"
    if "m_max" in cfg:
        conf["m_max"] = cfg["m_max"]
    if b.rank:
        conf.update(local_experts=cfg["n_local"], ranks=cfg["n_ranks"], received_rows=rows,
                    eplb_replicas=b.plan["rule"], measured_rank=b.plan["rank"],
                    rank_rows_max_over_mean=round(max(b.rank_rows) * len(b.rank_rows) / sum(b.rank_rows), 4),
                    rows_per_local_expert=b.L.masked_m.cpu().tolist())
    lb = layer_bytes(cfg, b.T, rows, active, esz, gather=b.gather)
    layer = {"algorithmic_bytes": lb, "achieved": lb / (ms * 1e-3) / 1e9, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
             "frac": lb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS}
    return {"metric": metric, "value": value, "unit": unit, "ms_per_step": ms, "dtype": cfg["dtype"],
            "config": conf, "roofline": roof, "layer": layer}


def sbo_compare(b, steps, rounds=4):
    """The prefill rank share's step with the signalled down GEMM and the
    polling combine against the same step run sequentially (plain down GEMM,
    then a plain combine), timed in alternating blocks."""
    import numpy as np
    per = max(3, steps // 2)
    res = {"signalled": [], "sequential": []}
    for _ in range(rounds):
        for mode in ("signalled", "sequential"):
            b.sbo_mode = mode
            b.step()
            ms, _ = _ms_steps(b, per, timed=False)
            res[mode].append(ms)
    b.sbo_mode = "signalled"
    sig, seq = float(np.median(res["signalled"])), float(np.median(res["sequential"]))
    # share of the combine's work units the polling workgroups claimed before
    # the finishing combine closed their counter (its first unit, per step)
    fracs = []
    n_sig = (b.L.m_cap + b.signal_rows - 1) // b.signal_rows
    n_units = b.L.m_cap + (b.T + 63) // 64
    for _ in range(per):
        b.step()
        b.torch.cuda.synchronize()
        fracs.append(int(b.signals[n_sig + 1].item()) / n_units)
    return {"signalled_ms": sig, "sequential_ms": seq, "gain_ms": seq - sig,
            "overlap_pays": seq > sig, "rounds": rounds, "steps_per_round": per,
            "polled_unit_fraction": round(float(np.median(fracs)), 4)}


def dispatch_forms(b, reps=20):
    """The dispatch of this batch on its own (nothing running beside it), in
    both payload forms: the layout only (ranks, scan, positions; the GEMM
    then gathers the rows) and the layout plus the rows copied into x_perm.
    The copy's algorithmic bytes: every token read once, every routed row
    written once (+ fp8 scales)."""
    torch, rdg, cfg = b.torch, b.rdg, b.cfg
    H, K = cfg["H"], cfg["K"]
    esz = {"f32": 4, "bf16": 2, "fp8": 1}[cfg["dtype"]]
    ids = b.local if b.rank else b.ids
    L = rdg.Layout(b.L.kind, b.L.n_local, b.T, K, b.dev, block_m=b.L.block_m, m_max=b.L.m_max)
    xp = torch.empty((L.m_cap, H), dtype=b.sdt, device=b.dev)
    xps = torch.empty((L.m_cap, H // 128), dtype=torch.float32, device=b.dev) if b.fp8 else None
    x_s = b.x_s if b.fp8 else None
    out = {}
    for name, args in (("layout_only", (None, None)), ("with_copy", (xp, xps))):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
        rdg.rdg_dispatch(b.x, x_s if args[0] is not None else None, b.DT, ids, L, *args)
        ev[0].record()
        for i in range(reps):
            rdg.rdg_dispatch(b.x, x_s if args[0] is not None else None, b.DT, ids, L, *args)
            ev[i + 1].record()
        torch.cuda.synchronize()
        out[name + "_us"] = round(1000 * ev[0].elapsed_time(ev[reps]) / reps, 2)
    rows = int(b.L.masked_m.sum().item())
    copy_bytes = b.T * H * esz + rows * H * esz + ((b.T + rows) * (H // 128) * 4 if b.fp8 else 0)
    extra_us = out["with_copy_us"] - out["layout_only_us"]
    out.update(copy_bytes=copy_bytes, copy_GBps=round(copy_bytes / (out["with_copy_us"] * 1e-6) / 1e9, 1),
               copy_frac_of_hbm=round(copy_bytes / (out["with_copy_us"] * 1e-6) / 1e9 / HBM_PEAK_GBPS, 3),
               copy_extra_us=round(extra_us, 2))
    return out


def heavy_experts(b, min_rows=315, reps=5):
    """The routed GEMMs restricted to the experts with at least `min_rows`
    rows (the rows per expert from which a bf16 tile's arithmetic outweighs
    its expert's weight bytes: 2.5 PFLOP/s / 8 TB/s), timed on their own:
    all of them in one grouped launch (the same kernels, the other experts'
    rows masked out of the dispatch), and each expert alone."""
    import numpy as np
    torch, rdg, cfg = b.torch, b.rdg, b.cfg
    H, I, K, N = cfg["H"], cfg["I"], cfg["K"], cfg["N"]
    counts = b.L.counts.cpu().numpy()
    heavy = [int(e) for e in np.flatnonzero(counts >= min_rows)]
    if not heavy:
        return None
    peak = MFMA_PEAK_TFLOPS[cfg["dtype"]]

    def run(expert_set):
        keep = torch.zeros(N, dtype=torch.bool, device=b.dev)
        keep[expert_set] = True
        ids = torch.where(keep[b.ids.long()], b.ids, torch.full_like(b.ids, -1))
        L = rdg.Layout(rdg.RDG_CONTIGUOUS, N, b.T, K, b.dev, block_m=128)
        xp = torch.empty((L.m_cap, H), dtype=b.sdt, device=b.dev)
        h = torch.empty((L.m_cap, I), dtype=b.sdt, device=b.dev)
        y = torch.empty((L.m_cap, H), dtype=b.ydt, device=b.dev)
        rdg.rdg_dispatch(b.x, None, b.DT, ids, L, xp)
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(reps + 1)]
        for e3 in ev:
            e3[0].record()
            rdg.rdg_grouped_gate_up(L, b.DT, H, I, xp, None, b.W["W1"], b.W["W3"], None, None, h, None)
            e3[1].record()
            rdg.rdg_grouped_down(L, b.DT, H, I, h, None, b.W["W2"], None, y)
            e3[2].record()
        torch.cuda.synchronize()
        rows = int(L.masked_m.cpu().sum())
        g = float(np.mean([e3[0].elapsed_time(e3[1]) for e3 in ev[1:]]))
        d = float(np.mean([e3[1].elapsed_time(e3[2]) for e3 in ev[1:]]))
        tiles = int(((L.masked_m.cpu().numpy() + 127) // 128).sum())
        fg = 4 * rows * H * I / (g * 1e-3) / 1e12
        fd = 2 * rows * H * I / (d * 1e-3) / 1e12
        return {"rows": rows, "row_tiles": tiles, "gate_up_ms": g, "gate_up_tflops": fg, "gate_up_mfma_frac": fg / peak,
                "down_ms": d, "down_tflops": fd, "down_mfma_frac": fd / peak}

    out = {"min_rows": min_rows, "experts": heavy, "together": run(heavy)}
    out["each"] = {str(e): run([e]) for e in heavy}
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU's share of the layer; runs on several GPUs (--gpus %d) are not "
              "supported (the expert-parallel sharding is described, not implemented)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    import torch

    dev = "cuda:0"
    torch.cuda.set_device(0)
    # a CU-masked stream needs a hardware queue of its own: created first
    side = cu_masked_stream(args.side_cus) if args.side_cus else None
    b = Bench(args.workload, dev, ue8m0=args.ue8m0, tbo=args.tbo, replicas=args.eplb_replicas, side_cus=args.side_cus,
              side_stream=side, payload=args.payload)
    if getattr(b, "signals", None) is not None:
        b.poll_blocks = args.poll_blocks
    res = measure(b, args, args.steps, args.warmup, args.workload)
    line = {"metric": res["metric"], "value": res["value"], "unit": res["unit"], "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": res["ms_per_step"], "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": res["dtype"], "data": "synthetic", "config": res["config"],
            "roofline": res["roofline"], "layer": res["layer"]}
    if b.rank and b.signals is not None and args.extras == "on":
        line["sbo"] = sbo_compare(b, args.steps)
        line["sbo"]["polling_workgroups"] = b.poll_blocks
    if not b.rank and b.cfg["layout"] == "contiguous" and b.cfg["H"] >= 1024 and not args.tbo and args.extras == "on":
        line["heavy_experts"] = heavy_experts(b)
    if not args.tbo and args.extras == "on":
        line["dispatch"] = dispatch_forms(b)
    n_cpu = CPU_TOKENS[args.workload] if args.cpu_tokens is None else args.cpu_tokens
    if n_cpu != 0:
        line["cpu_baseline"] = cpu_baseline(b, n_cpu)
    if args.calibrate_copy:
        src = torch.empty(1 << 29, dtype=torch.bfloat16, device=dev)  # 1 GiB
        dst = torch.empty_like(src)
        for _ in range(2):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    summary = args.summary == "on" or (args.summary == "auto" and args.workload == DEFAULT_WORKLOAD and
                                       not (args.graph or args.tbo or args.ue8m0 or args.eplb_replicas or
                                            args.side_cus))
    del b
    torch.cuda.empty_cache()
    if summary:
        line["workloads"] = summarise([w for w in ALL_WORKLOADS if w != args.workload], args)
    print(json.dumps(line), flush=True)


def summarise(names, args):
    """Every other workload measured in this run (10 timed steps each) with
    its own roofline, layer fraction, CPU-oracle baseline on a small sample,
    and for the prefill rank share its overlap comparison."""
    import torch
    out = {}
    for name in names:
        try:
            b = Bench(name, "cuda:0", payload=args.payload)
            r = measure(b, args, 10, 3, name)
            entry = {"value": r["value"], "unit": r["unit"], "ms_per_step": r["ms_per_step"], "dtype": r["dtype"],
                     "roofline": {k: r["roofline"][k] for k in ("bound", "frac", "achieved", "unit", "avg_ms",
                                                                "hbm_frac", "mfma_frac")},
                     "layer_frac": r["layer"]["frac"],
                     "config": {k: r["config"][k] for k in ("tokens", "routed_rows", "active_experts",
                                                            "load_balance_mean_over_max") if k in r["config"]}}
            if b.rank:
                entry["config"]["rows_per_local_expert"] = r["config"]["rows_per_local_expert"]
                entry["config"]["eplb_replicas"] = r["config"]["eplb_replicas"]
            if b.rank and b.signals is not None:
                entry["sbo"] = sbo_compare(b, 10, rounds=3)
                entry["sbo"]["polling_workgroups"] = b.poll_blocks
            n_cpu = SUMMARY_CPU_TOKENS.get(name, 0)
            if n_cpu != 0:
                entry["cpu_baseline"] = cpu_baseline(b, n_cpu)
                if name == "tiny_fp32":
                    import oracle
                    prev = oracle.set_num_threads(1)
                    try:
                        entry["cpu_baseline_1_thread"] = cpu_baseline(b, n_cpu)
                    finally:
                        oracle.set_num_threads(prev)
            out[name] = entry
            del b
        except Exception as ex:  # one workload's failure is reported, not fatal to the line
            out[name] = {"error": "%s: %s" % (type(ex).__name__, ex)}
        torch.cuda.empty_cache()
        print("measured %s" % name, file=sys.stderr, flush=True)
    return out


def _u16(t):
    import numpy as np
    import torch
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def cpu_baseline(b, n_tok):
    """The CPU oracle, as it stands, on the same workload.  Routing (or the
    rank share's replica remap) and the layout cover the whole batch; the
    layer output (routed experts + shared expert) is computed for the first
    n_tok tokens (-1: all of them).  The rate is scaled to the whole batch:
    time per token = routing-and-layout time / tokens + FFN time / sampled
    tokens (rank shares: per received row, reported as rows / K).  Host
    copies of the inputs (from the generator) are made before the clock."""
    import numpy as np

    import oracle
    cfg, synth = b.cfg, b.synth
    K, N = cfg["K"], cfg["N"]
    fp8 = b.fp8
    dt = {"f32": oracle.F32, "bf16": oracle.BF16, "fp8": oracle.FP8}[cfg["dtype"]]
    if b.ue8m0:
        dt = oracle.FP8_UE8M0
    if b.rank:
        ids = b.ids.cpu().numpy()
        gidx = b.gidx.cpu().numpy()
        w = b.tw.cpu().numpy()
        plan = b.plan
        T = ids.shape[0]
        n = T if n_tok < 0 else min(n_tok, T)
        loc = oracle.eplb_remap(ids, gidx, plan["log2phy"], plan["n_replica"], plan["phys_begin"], plan["n_local"])
        sel = np.arange(n, dtype=np.int32)
        local_logical = b.local_logical
        xb = synth.x(cfg, T, device=b.dev)
        xq, xs = oracle.quantize_fp8(_u16(xb), 1, ue8m0=b.ue8m0)
        experts = []
        for e in local_logical:
            wt = synth.expert_weights(cfg, e, device=b.dev)
            ex = {}
            for k, key in (("W1", "1"), ("W3", "3"), ("W2", "2")):
                q, s = oracle.quantize_fp8(wt[k].cpu().numpy(), 128, ue8m0=b.ue8m0)
                ex["W" + key], ex["s" + key] = q, s
            experts.append(ex)
        rows_total = int((loc >= 0).sum())
        rows_sample = int((loc[:n] >= 0).sum())
        t0 = time.perf_counter()
        loc2 = oracle.eplb_remap(ids, gidx, plan["log2phy"], plan["n_replica"], plan["phys_begin"], plan["n_local"])
        kind = oracle.MASKED if cfg["layout"] == "masked" else oracle.CONTIGUOUS
        oracle.layout(loc2, plan["n_local"], kind, block_m=128, m_max=cfg.get("m_max", 0))
        t1 = time.perf_counter()
        oracle.moe_layer(dt, xq, loc2, w, experts, x_scales=xs, sel=sel)
        t2 = time.perf_counter()
        per_row = (t1 - t0) / rows_total + (t2 - t1) / max(rows_sample, 1)
        return {"value": 1.0 / per_row / K, "unit": "token-equivalents/s", "cores": oracle.num_threads(),
                "kind": "oracle", "seconds": t2 - t0,
                "sample": "replica remap and layout of all %d received rows; the fp64 layer output of the first %d "
                          "tokens (%d rows); rate per received row scaled to the whole share" %
                          (rows_total, n, rows_sample)}
    B = b.logits_np.shape[0]
    n = B if n_tok < 0 else min(n_tok, B)
    ri, _ = oracle.route(b.logits_np, cfg["n_group"], cfg["topk_group"], K, cfg["scale"])
    sel = np.arange(n, dtype=np.int32)
    used = set(np.unique(ri[sel]).tolist())
    if cfg["dtype"] == "f32":
        conv = lambda t: t.detach().cpu().numpy()
    else:
        conv = _u16
    experts = [{k: conv(v) for k, v in synth.expert_weights(cfg, e, device=b.dev).items()} if e in used else None
               for e in range(N)]
    shared = {k: conv(v) for k, v in synth.expert_weights(cfg, 0, device=b.dev, shared=True).items()}
    xh = conv(b.x)
    kind = oracle.MASKED if cfg["layout"] == "masked" else oracle.CONTIGUOUS
    t0 = time.perf_counter()
    ids, w = oracle.route(b.logits_np, cfg["n_group"], cfg["topk_group"], K, cfg["scale"])
    oracle.layout(ids, N, kind, block_m=128, m_max=cfg.get("m_max", 0))
    t1 = time.perf_counter()
    oracle.moe_layer(dt, xh, ids, w, experts, shared=shared, sel=sel)
    t2 = time.perf_counter()
    per_tok = (t1 - t0) / B + (t2 - t1) / n
    return {"value": 1.0 / per_tok, "unit": "tokens/s", "cores": oracle.num_threads(), "kind": "oracle",
            "seconds": t2 - t0,
            "sample": ("the whole batch: routing, layout and the fp64 layer output (%d routed experts + shared) "
                       "of all %d tokens" % (K, n)) if n == B else
                      ("routing and layout of all %d tokens; the fp64 layer output (%d routed experts + shared) of "
                       "the first %d; rate per token scaled to the whole batch" % (B, K, n))}


if __name__ == "__main__":
    main()
