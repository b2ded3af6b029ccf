"""Shared plumbing for the GPU parity tests: run the HIP path through the C
ABI, gather host copies, and run the oracle on the same seeded inputs.
Nothing here computes a step of the method."""
import numpy as np
import torch

import oracle
import synth

DEV = "cuda"


def rdg():
    import routing_dispatch_grouped_amd as m
    return m


def dt_code(cfg):
    m = rdg()
    return {"f32": m.RDG_F32, "bf16": m.RDG_BF16, "fp8": m.RDG_FP8_E4M3, "fp8u": m.RDG_FP8_E4M3_UE8M0}[cfg["dtype"]]


def is_fp8(cfg):
    """fp8 e4m3 layers: "fp8" (fp32 block scales) and "fp8u" (power-of-two block scales)."""
    return cfg["dtype"] in ("fp8", "fp8u")


def np_of(t):
    """Tensor -> numpy in storage form (bf16 -> uint16 bits, fp8 -> uint8 codes)."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype in (torch.float8_e4m3fn, torch.uint8):
        return t.view(torch.uint8).numpy()
    return t.numpy()


def out_as_f64(arr):
    return oracle.bf16_decode(arr) if arr.dtype == np.uint16 else arr.astype(np.float64)


def torch_dtype(dt):
    m = rdg()
    return {m.RDG_F32: torch.float32, m.RDG_BF16: torch.bfloat16, m.RDG_FP8_E4M3: torch.uint8,
            m.RDG_FP8_E4M3_UE8M0: torch.uint8}[dt]


class ExpertSet:
    """Stacked device weights of n experts, packed for the grouped GEMMs
    (rdg_pack_weights) from natural [n, I, H], [n, I, H], [n, H, I] weights.

    fp32/bf16 workloads pack the generated weights.  fp8 workloads quantise
    the generated fp32 weights on the device (rdg_quantize_fp8, 128x128
    blocks), keep those natural codes for the bit-exact check against the
    oracle's own quantisation, and pack them."""

    def __init__(self, cfg, expert_ids, device=DEV, shared=False):
        m = rdg()
        self.cfg, self.ids, self.shared = cfg, list(expert_ids), shared
        H = cfg["H"]
        I = cfg["shared_I"] if shared else cfg["I"]
        self.H, self.I = H, I
        n = len(self.ids)
        self.fp8 = is_fp8(cfg)
        self.pow2 = cfg["dtype"] == "fp8u"
        sdt = torch.uint8 if self.fp8 else synth.storage_dtype(cfg)
        code = dt_code(cfg)
        self.W1 = torch.empty((n, I, H), dtype=sdt, device=device)
        self.W3 = torch.empty((n, I, H), dtype=sdt, device=device)
        self.W2 = torch.empty((n, H, I), dtype=sdt, device=device)
        self.s1 = self.s3 = self.s2 = None
        self.codes = None
        if self.fp8:
            f = dict(dtype=torch.float32, device=device)
            self.s1 = torch.empty((n, I // 128, H // 128), **f)
            self.s3 = torch.empty((n, I // 128, H // 128), **f)
            self.s2 = torch.empty((n, H // 128, I // 128), **f)
            self.codes = {k: torch.empty_like(v) for k, v in (("W1", self.W1), ("W3", self.W3), ("W2", self.W2))}
        for j, e in enumerate(self.ids):
            w = synth.expert_weights(cfg, e, device=device, shared=shared)
            for name, dst, sc in (("W1", self.W1, self.s1), ("W3", self.W3, self.s3), ("W2", self.W2, self.s2)):
                if self.fp8:
                    nat = self.codes[name][j]
                    quant = m.rdg_quantize_fp8_ue8m0 if self.pow2 else m.rdg_quantize_fp8
                    quant(w[name], m.RDG_F32, 128, nat, sc[j])
                else:
                    nat = w[name]
                m.rdg_pack_weights(nat, code, dst[j])
            del w

    def oracle_expert(self, j, check_codes=True):
        """Expert j for the oracle, in natural layout, straight from the
        generator (fp8: the oracle's own quantisation of the same fp32
        weights, optionally checked bit for bit against the device's codes)."""
        w = synth.expert_weights(self.cfg, self.ids[j], device=self.W1.device, shared=self.shared)
        if not self.fp8:
            return {k: np_of(v) for k, v in w.items()}
        out = {}
        for name, key, dev_s in (("W1", "1", self.s1), ("W3", "3", self.s3), ("W2", "2", self.s2)):
            q, s = oracle.quantize_fp8(np_of(w[name]), 128, ue8m0=self.pow2)
            if check_codes:
                assert np.array_equal(q, np_of(self.codes[name][j])), "device weight codes differ from the oracle's"
                assert np.array_equal(s, np_of(dev_s[j])), "device weight scales differ from the oracle's"
            out["W" + key], out["s" + key] = q, s
        return out


def quantize_act(x, pow2=False):
    """Device 1x128 quantisation of activations [T, H] (pow2: power-of-two scales)."""
    m = rdg()
    T, H = x.shape
    q = torch.empty((T, H), dtype=torch.uint8, device=x.device)
    s = torch.empty((T, H // 128), dtype=torch.float32, device=x.device)
    src_dt = m.RDG_BF16 if x.dtype == torch.bfloat16 else m.RDG_F32
    (m.rdg_quantize_fp8_ue8m0 if pow2 else m.rdg_quantize_fp8)(x, src_dt, 1, q, s)
    return q, s


def run_routed(cfg, x, x_s, local_ids, topk_w, experts, kind, block_m=128, m_max=0, shared_out=None,
               signals=False, max_blocks=0, concurrent=False, timeout_us=2_000_000, gather=False, finish=False):
    """dispatch -> grouped FFN -> combine on the device.  Returns a dict of
    device tensors (layout, x_perm, h, y, out).  gather: the dispatch builds
    the layout only and the grouped FFN reads the token rows through it
    (rdg_grouped_ffn_gather; x_perm is then None).  finish (with signals):
    rdg_combine_finish after the down GEMM on its stream, beside the polling
    combine."""
    m = rdg()
    dt = dt_code(cfg)
    T, H = x.shape
    K = local_ids.shape[1]
    I = cfg["I"]
    n_local = experts.W1.shape[0]
    L = m.Layout(kind, n_local, T, K, x.device, block_m=block_m, m_max=m_max)
    sdt = torch_dtype(dt)
    if gather:
        x_perm = x_perm_s = None
        m.rdg_dispatch(x, None, dt, local_ids, L, None, None)
    else:
        x_perm = torch.empty((L.m_cap, H), dtype=sdt, device=x.device)
        x_perm_s = (torch.empty((L.m_cap, H // 128), dtype=torch.float32, device=x.device)
                    if x_s is not None else None)
        m.rdg_dispatch(x, x_s, dt, local_ids, L, x_perm, x_perm_s)

    def ffn(stream=None):
        if gather:
            m.rdg_grouped_ffn_gather(L, dt, H, I, x, x_s, K, experts.W1, experts.W3, experts.W2, experts.s1,
                                     experts.s3, experts.s2, h, h_s, y, sig, stream=stream)
        else:
            m.rdg_grouped_ffn(L, dt, H, I, x_perm, x_perm_s, experts.W1, experts.W3, experts.W2, experts.s1,
                              experts.s3, experts.s2, h, h_s, y, sig, stream=stream)
    h = torch.empty((L.m_cap, I), dtype=sdt, device=x.device)
    h_s = torch.empty((L.m_cap, I // 128), dtype=torch.float32, device=x.device) if is_fp8(cfg) else None
    ydt = torch.float32 if dt == m.RDG_F32 else torch.bfloat16
    y = torch.empty((L.m_cap, H), dtype=ydt, device=x.device)
    sig = None
    thr = 0
    rows = 0
    n_sig = 0
    if signals:
        rows = m.rdg_signal_rows(L, dt, H, I)
        n_sig = (L.m_cap + rows - 1) // rows  # the row tiles' counters, then the combine's two words
        sig = torch.empty((n_sig + 2,), dtype=torch.int32, device=x.device)
        m.rdg_fill_i32(sig, 0)
        thr = m.rdg_signal_threshold(H, dt)
    out_dt = m.RDG_F32 if dt == m.RDG_F32 else m.RDG_BF16
    out = torch.empty((T, H), dtype=ydt, device=x.device)
    if signals:
        # NaN in y and out before a signalled run: a combine that read a row
        # before its tile was published, or skipped a token, cannot pass as a
        # left-over of an earlier identical run
        m.rdg_fill_i32(y.view(torch.int32), -1)
        m.rdg_fill_i32(out.view(torch.int32), -1)
    y_dt = m.RDG_F32 if dt == m.RDG_F32 else m.RDG_BF16
    if concurrent:
        s_gemm = torch.cuda.current_stream()
        s_comb = torch.cuda.Stream()
        s_comb.wait_stream(s_gemm)  # combine starts after dispatch; it then overlaps the GEMMs
        ffn(stream=s_gemm)
        with torch.cuda.stream(s_comb):
            m.rdg_combine(y, y_dt, L, topk_w, T, K, H, shared_out, out, out_dt, sig, rows if signals else 0,
                          thr, timeout_us, max_blocks, stream=s_comb)
        if finish:
            m.rdg_combine_finish(y, y_dt, L, topk_w, T, K, H, shared_out, out, out_dt, sig, rows, stream=s_gemm)
        s_gemm.wait_stream(s_comb)
    else:
        ffn()
        m.rdg_combine(y, y_dt, L, topk_w, T, K, H, shared_out, out, out_dt, sig, rows if signals else 0, thr,
                      timeout_us, max_blocks)
        if finish:
            m.rdg_combine_finish(y, y_dt, L, topk_w, T, K, H, shared_out, out, out_dt, sig, rows)
    return dict(L=L, x_perm=x_perm, x_perm_s=x_perm_s, h=h, h_s=h_s, y=y, out=out, signals=sig, threshold=thr,
                signal_rows=rows, n_sig=n_sig)


def run_shared(cfg, x, x_s, shared):
    """The shared expert as a one-expert dense layout; returns its output [T, H]."""
    m = rdg()
    dt = dt_code(cfg)
    T, H = x.shape
    I = cfg["shared_I"]
    L = m.Layout(m.RDG_CONTIGUOUS, 1, T, 1, x.device, block_m=16, m_cap=T)
    m.rdg_layout_dense(T, L)
    sdt = torch_dtype(dt)
    h = torch.empty((T, I), dtype=sdt, device=x.device)
    h_s = torch.empty((T, I // 128), dtype=torch.float32, device=x.device) if is_fp8(cfg) else None
    ydt = torch.float32 if dt == m.RDG_F32 else torch.bfloat16
    y = torch.empty((T, H), dtype=ydt, device=x.device)
    m.rdg_grouped_ffn(L, dt, H, I, x, x_s, shared.W1, shared.W3, shared.W2, shared.s1, shared.s3, shared.s2,
                      h, h_s, y)
    return y


def check_layout(L, ref, ids_shape):
    """Bit-exact comparison of a device layout with the oracle's."""
    assert np.array_equal(np_of(L.counts), ref["counts"]), "counts"
    assert np.array_equal(np_of(L.offsets), ref["offsets"]), "offsets"
    assert np.array_equal(np_of(L.masked_m), ref["masked_m"]), "masked_m"
    n = ids_shape[0] * ids_shape[1]
    assert np.array_equal(np_of(L.pos)[:n], ref["pos"].ravel()), "pos"
    assert np.array_equal(np_of(L.row_src)[:L.m_cap], ref["row_src"]), "row_src"


def row_tolerance(cfg):
    """Per-token ||out-ref|| / ||ref|| bound: catches a missing or extra
    expert term in a token whose values are small next to the tensor's max."""
    return {"f32": 1e-5, "bf16": 2e-2, "fp8": 1e-1, "fp8u": 1e-1}[cfg["dtype"]]


def check_rows(got, ref, cfg, what=""):
    g = out_as_f64(got)
    r = out_as_f64(ref)
    num = np.linalg.norm(g - r, axis=1)
    den = np.linalg.norm(r, axis=1)
    rel = np.where(den > 0, num / np.maximum(den, 1e-300), num)
    worst = int(np.argmax(rel))
    assert rel[worst] <= row_tolerance(cfg), "%s: row %d relative error %.3e" % (what, worst, rel[worst])
    return float(rel.max())


def tolerance(cfg):
    """Max relative error max|out-ref|/max|ref| allowed per tensor."""
    return {"f32": 1e-5, "bf16": 2e-2, "fp8": 6e-2, "fp8u": 6e-2}[cfg["dtype"]]


def ue8m0_clamp_edge_rows(seed=11):
    """fp32 rows of 128 whose largest magnitude sits at the lower clamp of
    power-of-two block scales (2^-126): exactly 448 * 2^-126, one ulp either
    side of it, 448 * 2^-127 and 2^-126 (clamped), fp32-subnormal blocks,
    and an all-zero block.  Elements are random multiples of the block's
    amax, so the smallest of them are fp32 subnormals."""
    rng = np.random.default_rng(seed)
    edge = np.float32(448.0 * 2.0 ** -126)
    amaxes = [edge, np.nextafter(edge, np.float32(np.inf)), np.nextafter(edge, np.float32(0)),
              np.float32(448.0 * 2.0 ** -127), np.float32(2.0 ** -126), np.float32(2.0 ** -133),
              np.float32(2.0 ** -140), np.float32(2.0 ** -149), np.float32(1.5 * 448.0 * 2.0 ** -126),
              np.float32(0.0)]
    rows = []
    for a in amaxes:
        for rep in range(3):
            v = (rng.uniform(-1.0, 1.0, 128) * np.float64(a)).astype(np.float32)
            v[rng.integers(128)] = a if rep != 1 else -a
            rows.append(v)
    return np.array(rows, dtype=np.float32)
