"""bench.py's command line on the CPU: more than one GPU is refused with exit
code 2 before anything touches a device, and the defaults are one GPU, the
4096-token prefill layer (the largest configuration on one GPU), a run of
5 + 20 steps, and the summary of every other workload."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_several_gpus_are_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "8"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2
    assert "--gpus 8" in r.stderr and "one GPU" in r.stderr
    assert r.stdout == ""


def test_defaults(monkeypatch):
    sys.path.insert(0, ROOT)
    import bench
    monkeypatch.setattr(sys, "argv", ["bench.py"])
    a = bench.parse()
    assert (a.gpus, a.steps, a.warmup, a.workload, a.cpu_tokens) == (1, 20, 5, "prefill_bf16", None)
    assert a.summary == "auto" and a.eplb_replicas is None and a.payload == "gather"
    assert not (a.graph or a.ue8m0 or a.tbo or a.calibrate_copy)
    assert bench.CPU_TOKENS["prefill_bf16"] > 0 and set(bench.CPU_TOKENS) == set(bench.ALL_WORKLOADS)


def test_layer_bytes_decode():
    """The decode layer's step bytes: each of the 195 active experts' three
    weight matrices and the shared expert's, read once, plus the activations
    that move between the kernels, counted by hand here."""
    sys.path.insert(0, ROOT)
    import bench
    import synth
    cfg = synth.WORKLOADS["decode_bf16"]
    T, R, A, H, I, K, N, S = 128, 1024, 195, 7168, 2048, 8, 256, 2048
    weights = (A * 3 * I * H + 3 * S * H) * 2
    route = T * N * 4 + T * K * 8 + T * K * 8          # logits in, ids + weights out, ranks
    permute = (T + R) * H * 2
    routed = R * (H + I) * 2 + R * (I * 2 + H * 2)     # rows in and h out; h in and y out
    shared = T * (H + I) * 2 + T * (I + H) * 2
    combine = R * H * 2 + T * H * 2 + T * H * 2        # routed rows, shared output, result
    assert bench.layer_bytes(cfg, T, R, A, 2) == weights + route + permute + routed + shared + combine
    # gathering: the dispatch only publishes pos [T*K] and row_src [R]
    assert bench.layer_bytes(cfg, T, R, A, 2, gather=True) == (weights + route + T * K * 4 + R * 4 + routed + shared
                                                               + combine)


def test_layer_bytes_fp8_scales():
    """In fp8 every 128-block of weights and every 128-wide piece of a row
    carries one 4-byte scale; bf16 carries none."""
    sys.path.insert(0, ROOT)
    import bench
    import synth
    cfg = dict(synth.WORKLOADS["decode_rank_fp8"])
    T, R, A = 1013, 1024, 4
    H, I = cfg["H"], cfg["I"]
    b8 = bench.layer_bytes(cfg, T, R, A, 1)
    b16 = bench.layer_bytes(dict(cfg, dtype="bf16"), T, R, A, 2)
    w_sc = A * 3 * (I // 128) * (H // 128) * 4
    x_sc = (T + R) * (H // 128) * 4 + R * (H + I) // 128 * 4 + R * (I // 128) * 4
    # fp8 halves every token/weight byte except the bf16 output rows
    assert b8 - w_sc - x_sc < b16
    assert w_sc + x_sc > 0
