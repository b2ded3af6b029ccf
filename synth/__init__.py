"""Seeded synthetic workloads for the MoE-layer hot path.

This module only draws random numbers and lays them out; it holds none of
the method's arithmetic (no scoring, selection, layout, quantisation, FFN
or combine).  Both the HIP path's tests/benchmark and the CPU oracle take
their inputs from here.

Five workloads, named by what they are:

* ``tiny_fp32``      64 tokens, H=256, 16 experts in 4 groups of 4, 2 groups
                     kept, top-4, I=128, one shared expert (I=128), fp32,
                     contiguous layout.
* ``decode_bf16``    DeepSeek-V3 decode step on one GPU holding all experts:
                     128 tokens, H=7168, 256 experts in 8 groups of 32, 4
                     groups kept, top-8, I=2048, shared expert I=2048, bf16,
                     masked layout with 256 rows per expert; logits N(0,1)
                     plus a per-expert N(0,0.5) bias.
* ``prefill_bf16``   4096 tokens (two 2048-token sequences), same shapes,
                     bf16, contiguous layout; logits make expert popularity
                     Zipf(1.1) over a seeded permutation.
* ``prefill_bf16_balanced`` the same prefill layer with i.i.d. N(0,1)
                     logits: every token's choice is a random selection that
                     follows the group-limited rule, the "simulated perfect
                     EPLB" expert distribution (balanced in expectation).
* ``decode_rank_fp8`` one decode rank's share with EPLB: 72 ranks x 4
                     physical experts (256 logical + 32 redundant copies,
                     each given greedily to the expert with the largest
                     expected load per copy; ``replicas="one_each"`` gives
                     the 32 most popular experts one extra copy each
                     instead); the rank that receives the most rows of the
                     global batch (the bottleneck) takes its first 1024
                     token-expert rows; fp8 e4m3 with 1x128 / 128x128 block
                     scales; masked layout.
* ``prefill_rank_fp8`` one prefill rank's share: 32 ranks x 9 physical
                     experts, the bottleneck rank's first 16384 received rows, shared expert on the
                     rank's own 2048 tokens; fp8; contiguous layout; the
                     down projection signals a concurrently running combine.

Seeding: every tensor comes from ``SeedSequence([2026, workload, tensor,
index])``; tensor ids: 0 logits/noise, 1 bias or Zipf permutation, 2 Gumbel,
3 x, 4 W1, 5 W3, 6 W2, 7..9 shared W1/W3/W2, 10 own-token x (shared expert).
Normals are drawn in fp32 and cast to the storage type with torch's
round-to-nearest-even casts; fp8 workloads hand out fp32 weights and bf16
activations, and each side quantises them itself.
"""
import numpy as np

WORKLOADS = {
    "tiny_fp32": dict(wid=1, B=64, H=256, N=16, n_group=4, topk_group=2, K=4, I=128, shared_I=128,
                      dtype="f32", layout="contiguous", scale=1.0, logits="normal"),
    "decode_bf16": dict(wid=2, B=128, H=7168, N=256, n_group=8, topk_group=4, K=8, I=2048, shared_I=2048,
                        dtype="bf16", layout="masked", m_max=256, scale=1.0, logits="normal_bias"),
    "prefill_bf16": dict(wid=3, B=4096, H=7168, N=256, n_group=8, topk_group=4, K=8, I=2048, shared_I=2048,
                         dtype="bf16", layout="contiguous", scale=1.0, logits="zipf", zipf_s=1.1,
                         seq_lens=[2048, 2048]),
    "prefill_bf16_balanced": dict(wid=6, B=4096, H=7168, N=256, n_group=8, topk_group=4, K=8, I=2048,
                                  shared_I=2048, dtype="bf16", layout="contiguous", scale=1.0, logits="normal",
                                  seq_lens=[2048, 2048]),
    "decode_rank_fp8": dict(wid=4, B_global=72 * 128, n_ranks=72, n_local=4, n_redundant=32, rows=1024,
                            H=7168, N=256, n_group=8, topk_group=4, K=8, I=2048, shared_I=0,
                            dtype="fp8", layout="masked", m_max=1024, scale=1.0, logits="zipf", zipf_s=1.1),
    "prefill_rank_fp8": dict(wid=5, B_global=32 * 2048, n_ranks=32, n_local=9, n_redundant=32, rows=16384,
                             own_tokens=2048, H=7168, N=256, n_group=8, topk_group=4, K=8, I=2048,
                             shared_I=2048, dtype="fp8", layout="contiguous", scale=1.0, logits="zipf",
                             zipf_s=1.1, signals=True),
}

WEIGHT_STD = 0.02


def seed_of(wid, tensor, index=0):
    return [2026, int(wid), int(tensor), int(index)]


def rng(wid, tensor, index=0):
    return np.random.default_rng(seed_of(wid, tensor, index))


def torch_seed(wid, tensor, index=0):
    return int(np.random.SeedSequence(seed_of(wid, tensor, index)).generate_state(1, np.uint64)[0] >> 1)


def zipf_probs(N, s):
    """p_r proportional to r^-s over ranks r = 1..N."""
    r = np.arange(1, N + 1, dtype=np.float64)
    p = r ** (-s)
    return p / p.sum()


def zipf_permutation(cfg):
    """rank_of[e]: popularity rank (0 = hottest) of expert e, seeded."""
    perm = rng(cfg["wid"], 1).permutation(cfg["N"])  # perm[r] = expert with rank r
    rank_of = np.empty(cfg["N"], np.int64)
    rank_of[perm] = np.arange(cfg["N"])
    return rank_of


def expected_popularity(cfg):
    """Per logical expert, the Zipf probability of its popularity rank."""
    return zipf_probs(cfg["N"], cfg["zipf_s"])[zipf_permutation(cfg)]


def logits(cfg, B=None):
    """Router logits, float32 [B, N].

    normal:      N(0, 1)
    normal_bias: N(0, 1) + b_e with b_e ~ N(0, 0.5) per expert
    zipf:        log p_rank(e) + Gumbel(0, 1) noise (Gumbel-max sampling makes
                 the top-1 choice Zipf-distributed before group limiting)
    """
    wid, N = cfg["wid"], cfg["N"]
    if B is None:
        B = cfg.get("B_global", cfg.get("B"))
    kind = cfg["logits"]
    if kind == "normal":
        return rng(wid, 0).standard_normal((B, N)).astype(np.float32)
    if kind == "normal_bias":
        z = rng(wid, 0).standard_normal((B, N))
        b = rng(wid, 1).normal(0.0, 0.5, size=N)
        return (z + b[None, :]).astype(np.float32)
    if kind == "zipf":
        u = rng(wid, 2).random((B, N))
        g = -np.log(-np.log(np.clip(u, 1e-300, None)))
        return (np.log(expected_popularity(cfg))[None, :] + g).astype(np.float32)
    raise ValueError(kind)


def _torch():
    import torch
    return torch


def normal(wid, tensor, index, shape, std, device, dtype):
    """N(0, std) in fp32 from a seeded torch generator on ``device``, then cast."""
    torch = _torch()
    gen = torch.Generator(device=device)
    gen.manual_seed(torch_seed(wid, tensor, index))
    t = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t.to(dtype)


def storage_dtype(cfg):
    torch = _torch()
    return {"f32": torch.float32, "bf16": torch.bfloat16, "fp8": torch.float32, "fp8u": torch.float32}[cfg["dtype"]]


def activation_dtype(cfg):
    torch = _torch()
    return {"f32": torch.float32, "bf16": torch.bfloat16, "fp8": torch.bfloat16, "fp8u": torch.bfloat16}[cfg["dtype"]]


def x(cfg, T, device="cpu", tensor=3):
    """Token activations [T, H] (fp32, or bf16 for the bf16 and fp8 workloads)."""
    return normal(cfg["wid"], tensor, 0, (T, cfg["H"]), 1.0, device, activation_dtype(cfg))


def expert_weights(cfg, e, device="cpu", shared=False):
    """One expert's W1, W3 [I, H] and W2 [H, I] (K-major), N(0, 0.02)."""
    H = cfg["H"]
    I = cfg["shared_I"] if shared else cfg["I"]
    base = 7 if shared else 4
    dt = storage_dtype(cfg)
    return dict(W1=normal(cfg["wid"], base, e, (I, H), WEIGHT_STD, device, dt),
                W3=normal(cfg["wid"], base + 1, e, (I, H), WEIGHT_STD, device, dt),
                W2=normal(cfg["wid"], base + 2, e, (H, I), WEIGHT_STD, device, dt))


def replica_counts(pop, n_redundant, rule="greedy"):
    """Copies of each logical expert (workload recipe, not a hot-path step).

    greedy:   n_redundant times, one more copy to the logical expert with the
              largest expected load per copy (ties: lower id) -- the replica
              rule of the EPLB workloads.
    one_each: the n_redundant most popular experts get one extra copy each
              (ties: lower id), a plainer allocation kept for comparison.
    """
    N = len(pop)
    n_rep = np.ones(N, np.int32)
    if rule == "one_each":
        for e in sorted(range(N), key=lambda e: (-pop[e], e))[:n_redundant]:
            n_rep[e] = 2
        return n_rep
    if rule != "greedy":
        raise ValueError(rule)
    for _ in range(n_redundant):
        per_copy = pop / n_rep
        best = max(per_copy)
        e = int(np.flatnonzero(per_copy == best)[0])
        n_rep[e] += 1
    return n_rep


def eplb_plan(cfg, rule=None):
    """Static placement of the logical experts into n_ranks * n_local slots.

    Workload recipe (the placement itself is not on the hot path): copies per
    expert from replica_counts (cfg["replicas"], default greedy); physical
    experts, each carrying expected popularity / copies, are taken in
    descending load (ties: lower logical id, then copy index) and each goes
    to the least-loaded rank that still has a free slot (ties: lower rank).
    Physical id = rank * n_local + slot.  Returns log2phy [N, r_max] (unused
    columns repeat the first copy), n_replica [N], the expected rank loads,
    and the rank with the highest expected load (ties lower rank) as a first
    choice of the measured rank; measured_rank replaces it by the rank that
    receives the most rows once the global batch has been routed.
    """
    N, n_ranks, n_local = cfg["N"], cfg["n_ranks"], cfg["n_local"]
    assert n_ranks * n_local == N + cfg["n_redundant"]
    rule = rule or cfg.get("replicas", "greedy")
    pop = expected_popularity(cfg)
    n_rep = replica_counts(pop, cfg["n_redundant"], rule)
    r_max = int(n_rep.max())
    units = [(pop[e] / n_rep[e], e, r) for e in range(N) for r in range(n_rep[e])]
    units.sort(key=lambda u: (-u[0], u[1], u[2]))
    load = np.zeros(n_ranks)
    used = np.zeros(n_ranks, np.int64)
    log2phy = np.full((N, r_max), -1, np.int32)
    for ld, e, r in units:
        cand = [k for k in range(n_ranks) if used[k] < n_local]
        k = min(cand, key=lambda k: (load[k], k))
        log2phy[e, r] = k * n_local + used[k]
        used[k] += 1
        load[k] += ld
    for e in range(N):
        log2phy[e, n_rep[e]:] = log2phy[e, 0]
    bottleneck = int(np.argmax(load))
    return dict(log2phy=log2phy, n_replica=n_rep, load=load, bottleneck=bottleneck,
                phys_begin=bottleneck * n_local, n_local=n_local, rule=rule)


def measured_rank(plan, rows_per_rank):
    """The rank whose share is measured: the one that receives the most
    rows of the routed global batch (the bottleneck of an expert-parallel
    step; ties: lower rank).  rows_per_rank comes from the caller's routing
    and replica remap of the global batch.  Returns the plan with that
    rank's physical range."""
    r = int(np.argmax(np.asarray(rows_per_rank)))
    return dict(plan, rank=r, phys_begin=r * plan["n_local"])


def take_rank_rows(local_ids, rows):
    """Which tokens one rank receives: given the global batch's per-slot
    local expert ids on this rank (-1: not here), take the tokens that send
    it at least one row, in global order, until exactly ``rows`` rows; the
    last token's surplus rows are marked as not sent.  Returns (token
    indices, keep mask [n_tokens, K])."""
    local_ids = np.asarray(local_ids)
    per_tok = (local_ids >= 0).sum(1)
    toks, keep, taken = [], [], 0
    for t in np.flatnonzero(per_tok > 0):
        k_loc = np.flatnonzero(local_ids[t] >= 0)
        m = np.zeros(local_ids.shape[1], bool)
        take = k_loc[:rows - taken]
        m[take] = True
        toks.append(t)
        keep.append(m)
        taken += len(take)
        if taken == rows:
            break
    return np.array(toks, dtype=np.int64), np.array(keep, dtype=bool).reshape(-1, local_ids.shape[1])
