"""HIP-graph capture of the masked decode path.  Decode's fixed shapes (the
low-latency mode's preallocated buffers, [LEP] "DeepEP: each mode where it
belongs" and self-test answer 1) let a whole step be captured once and
replayed, which removes the per-kernel launch cost.

One step -- route, masked dispatch, grouped FFN, combine, with the shared
expert on a second stream joined before the combine -- is captured with
torch.cuda.graph.  Between replays the program does its own eager work: new
router logits and tokens are copied into the captured input buffers, the
same step runs eagerly on them, and the output buffer is poisoned with NaN.
Every replay must then reproduce the eager output bit for bit (all the
kernels are deterministic), and the last replay's output must equal the
oracle's definition of the layer on every token (max|out-ref|/max|ref| <=
2e-2, bf16)."""
import numpy as np
import pytest
import torch

import oracle
import synth
from harness import DEV, ExpertSet, check_rows, np_of, out_as_f64, rdg

pytestmark = pytest.mark.gpu


class DecodeStep:
    def __init__(self, cfg, B):
        m = rdg()
        self.m, self.cfg, self.B = m, cfg, B
        H, I, N, K = cfg["H"], cfg["I"], cfg["N"], cfg["K"]
        self.experts = ExpertSet(cfg, range(N))
        self.shared = ExpertSet(cfg, [0], shared=True)
        self.logits = torch.empty((B, N), dtype=torch.float32, device=DEV)
        self.x = torch.empty((B, H), dtype=torch.bfloat16, device=DEV)
        self.ids = torch.empty((B, K), dtype=torch.int32, device=DEV)
        self.w = torch.empty((B, K), dtype=torch.float32, device=DEV)
        self.L = m.Layout(m.RDG_MASKED, N, B, K, DEV, m_max=cfg["m_max"])
        self.xp = torch.empty((self.L.m_cap, H), dtype=torch.bfloat16, device=DEV)
        self.h = torch.empty((self.L.m_cap, I), dtype=torch.bfloat16, device=DEV)
        self.y = torch.empty((self.L.m_cap, H), dtype=torch.bfloat16, device=DEV)
        self.Ls = m.Layout(m.RDG_CONTIGUOUS, 1, B, 1, DEV, block_m=16, m_cap=B)
        m.rdg_layout_dense(B, self.Ls)
        self.hs = torch.empty((B, cfg["shared_I"]), dtype=torch.bfloat16, device=DEV)
        self.ys = torch.empty((B, H), dtype=torch.bfloat16, device=DEV)
        self.out = torch.empty((B, H), dtype=torch.bfloat16, device=DEV)
        self.side = torch.cuda.Stream()

    def load_inputs(self, index):
        cfg = dict(self.cfg, wid=self.cfg["wid"] + 1000 * index)
        self.logits_np = synth.logits(cfg, self.B)
        self.logits.copy_(torch.from_numpy(self.logits_np))
        self.x.copy_(synth.x(cfg, self.B, device=DEV))

    def oracle_out(self):
        """The layer on the current inputs by the oracle's definition (bf16 bits)."""
        cfg = self.cfg
        ri, rw = oracle.route(self.logits_np, cfg["n_group"], cfg["topk_group"], cfg["K"], cfg["scale"])
        used = set(np.unique(ri).tolist())
        experts = [self.experts.oracle_expert(j) if j in used else None for j in range(cfg["N"])]
        return oracle.moe_layer(oracle.BF16, np_of(self.x), ri, rw, experts, shared=self.shared.oracle_expert(0))

    def __call__(self):
        m, cfg, B = self.m, self.cfg, self.B
        H, I, K, sI = cfg["H"], cfg["I"], cfg["K"], cfg["shared_I"]
        main = torch.cuda.current_stream()
        self.side.wait_stream(main)
        with torch.cuda.stream(self.side):
            m.rdg_grouped_ffn(self.Ls, m.RDG_BF16, H, sI, self.x, None, self.shared.W1, self.shared.W3,
                              self.shared.W2, None, None, None, self.hs, None, self.ys, stream=self.side)
        m.rdg_route(self.logits, cfg["n_group"], cfg["topk_group"], K, cfg["scale"], self.ids, self.w)
        m.rdg_dispatch(self.x, None, m.RDG_BF16, self.ids, self.L, self.xp)
        e = self.experts
        m.rdg_grouped_ffn(self.L, m.RDG_BF16, H, I, self.xp, None, e.W1, e.W3, e.W2, None, None, None, self.h,
                          None, self.y)
        main.wait_stream(self.side)
        m.rdg_combine(self.y, m.RDG_BF16, self.L, self.w, B, K, H, self.ys, self.out, m.RDG_BF16)


def _small():
    return dict(wid=700, H=1024, N=16, n_group=4, topk_group=2, K=4, I=512, shared_I=512, dtype="bf16",
                scale=1.0, logits="normal_bias", m_max=64)


@pytest.mark.parametrize("name", ["small", "decode_bf16"])
def test_graph_replay_matches_eager(name):
    m = rdg()
    cfg = _small() if name == "small" else dict(synth.WORKLOADS["decode_bf16"])
    B = 48 if name == "small" else cfg["B"]
    step = DecodeStep(cfg, B)
    step.load_inputs(0)
    step()                       # eager warm-up: code objects loaded outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for rep in range(3):
        step.load_inputs(rep + 1)
        step()
        ref = step.out.clone()
        assert m.rdg_check_status(step.L)[0] in (m.RDG_OK, m.RDG_ECAPACITY)
        m.rdg_fill_i32(step.out.view(torch.int32), -1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = step.out.view(torch.int16)
        assert not torch.isnan(step.out.float()).any(), "replay %d left poisoned output" % rep
        assert torch.equal(got, ref.view(torch.int16)), "replay %d differs from the eager step" % rep
        print("%s replay %d bit-equal to eager" % (name, rep), flush=True)
    want = step.oracle_out()
    out = np_of(step.out)
    err = oracle.rel_err(out_as_f64(out), out_as_f64(want))
    row = check_rows(out, want, dict(cfg, dtype="bf16"), "graph replay")
    print("%s last replay against the oracle: rel_err=%.3e worst token %.3e" % (name, err, row), flush=True)
    assert err <= 2e-2
