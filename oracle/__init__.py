"""CPU oracle for the MoE-layer hot path (test infrastructure).

Only the test suite, ``__graft_entry__.smoke()`` and the benchmark's
``cpu_baseline`` leg may import this package.  The product path never
touches it.  It wraps ``rdg_oracle.c`` (plain C, fp64) through ctypes and
shares no code with the HIP library.
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "rdg_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

F32, BF16, FP8, FP8_UE8M0 = 0, 1, 2, 3
CONTIGUOUS, MASKED = 0, 1
OK, EINVAL, ECAPACITY = 0, -1, -2


def build():
    """Compile the oracle with plain IEEE semantics (no contraction, no fast-math)."""
    cmd = ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-std=c11",
           "-shared", "-fPIC", "-o", _LIB + ".tmp", _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(_LIB + ".tmp", _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        L = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        i32, i64, f32 = ctypes.c_int, ctypes.c_int64, ctypes.c_float
        L.orc_num_threads.restype = i32
        L.orc_set_num_threads.argtypes = [i32]
        L.orc_set_num_threads.restype = i32
        L.orc_bf16_decode.argtypes = [ctypes.c_uint16]
        L.orc_bf16_decode.restype = ctypes.c_double
        L.orc_bf16_encode.argtypes = [ctypes.c_double]
        L.orc_bf16_encode.restype = ctypes.c_uint16
        L.orc_fp8_decode.argtypes = [ctypes.c_uint8]
        L.orc_fp8_decode.restype = ctypes.c_double
        L.orc_fp8_encode.argtypes = [ctypes.c_double]
        L.orc_fp8_encode.restype = ctypes.c_uint8
        L.orc_quantize_fp8.argtypes = [P, i32, i32, i32, i32, P, P]
        L.orc_quantize_fp8_ue8m0.argtypes = [P, i32, i32, i32, i32, P, P]
        L.orc_quantize_fp8.restype = i32
        L.orc_sigmoid.argtypes = [f32]
        L.orc_sigmoid.restype = f32
        L.orc_sigmoid_many.argtypes = [P, P, i64]
        L.orc_sigmoid_constants.argtypes = [P]
        L.orc_sigmoid_constants.restype = None
        L.orc_sigmoid_sweep.argtypes = [ctypes.c_uint32, ctypes.c_uint32, ctypes.c_uint32,
                                        ctypes.POINTER(i64), ctypes.POINTER(i64)]
        L.orc_sigmoid_sweep.restype = ctypes.c_double
        L.orc_route_biased.argtypes = [P, P, i32, i32, i32, i32, i32, f32, P, P]
        L.orc_route_biased.restype = i32
        L.orc_route.argtypes = [P, i32, i32, i32, i32, i32, f32, P, P]
        L.orc_route.restype = i32
        L.orc_eplb_remap.argtypes = [P, P, i32, i32, P, P, i32, i32, i32, i32, P]
        L.orc_eplb_remap.restype = i32
        L.orc_layout.argtypes = [P, i32, i32, i32, i32, i32, i32, i32, P, P, P, P, P, P]
        L.orc_layout.restype = i32
        L.orc_moe_layer.argtypes = [i32, i32, i32, i32, P, P, P, P, P, P, P, P, P, P,
                                    P, P, P, P, P, P, i32, P, i32, i32, P, P]
        L.orc_moe_layer.restype = i32
        L.orc_combine.argtypes = [i32, P, P, P, i32, i32, i32, P, i32, P]
        L.orc_combine.restype = i32
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data


def num_threads():
    return lib().orc_num_threads()


def set_num_threads(n):
    """Threads of the oracle's parallel loops from now on; returns the previous count."""
    return lib().orc_set_num_threads(int(n))


# ---------------------------------------------------------------- formats
def bf16_decode(bits):
    """uint16 bf16 bit patterns -> float64 (exact)."""
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def bf16_encode(v):
    v = np.ascontiguousarray(v, dtype=np.float64)
    f = lib().orc_bf16_encode
    return np.array([f(float(x)) for x in v.ravel()], dtype=np.uint16).reshape(v.shape)


def fp8_decode(codes):
    table = np.array([lib().orc_fp8_decode(c) for c in range(256)], dtype=np.float64)
    return table[np.asarray(codes, dtype=np.uint8)]


def fp8_encode(v):
    f = lib().orc_fp8_encode
    v = np.asarray(v, dtype=np.float64)
    return np.array([f(float(x)) for x in v.ravel()], dtype=np.uint8).reshape(v.shape)


def quantize_fp8(src, block_rows, ue8m0=False):
    """src: float32 [rows, cols] or uint16 bf16 bits.  Returns (codes uint8,
    scales float32); ue8m0: power-of-two scales."""
    src = np.ascontiguousarray(src)
    dt = F32 if src.dtype == np.float32 else BF16
    assert src.dtype in (np.float32, np.uint16)
    rows, cols = src.shape
    q = np.empty((rows, cols), dtype=np.uint8)
    s = np.empty(((rows + block_rows - 1) // block_rows, cols // 128), dtype=np.float32)
    f = lib().orc_quantize_fp8_ue8m0 if ue8m0 else lib().orc_quantize_fp8
    rc = f(_p(src), dt, rows, cols, block_rows, _p(q), _p(s))
    if rc != OK:
        raise ValueError("orc_quantize_fp8: %d" % rc)
    return q, s


# ---------------------------------------------------------------- routing
def sigmoid(x):
    x = np.ascontiguousarray(x, dtype=np.float32)
    y = np.empty_like(x)
    lib().orc_sigmoid_many(_p(x), _p(y), x.size)
    return y


def sigmoid_constants():
    """The oracle's sigmoid constants as derived at run time: log2(e), the
    two-part ln 2 (head, tail), then 1/k! for k = 0..13 (doubles)."""
    out = np.empty(17, dtype=np.float64)
    lib().orc_sigmoid_constants(_p(out))
    return out


def sigmoid_sweep(lo_bits, hi_bits, stride):
    n = ctypes.c_int64(0)
    nm = ctypes.c_int64(0)
    worst = lib().orc_sigmoid_sweep(lo_bits, hi_bits, stride, ctypes.byref(n), ctypes.byref(nm))
    return worst, n.value, nm.value


def route(logits, n_group, topk_group, K, scale=1.0, bias=None):
    """bias: optional float32 [N] added to the scores for the choice only."""
    logits = np.ascontiguousarray(logits, dtype=np.float32)
    B, N = logits.shape
    ids = np.empty((B, K), dtype=np.int32)
    w = np.empty((B, K), dtype=np.float32)
    if bias is None:
        rc = lib().orc_route(_p(logits), B, N, n_group, topk_group, K, scale, _p(ids), _p(w))
    else:
        bias = np.ascontiguousarray(bias, dtype=np.float32)
        rc = lib().orc_route_biased(_p(logits), _p(bias), B, N, n_group, topk_group, K, scale, _p(ids), _p(w))
    if rc != OK:
        raise ValueError("orc_route: invalid arguments")
    return ids, w


def eplb_remap(ids, gidx, log2phy, n_replica, phys_begin, n_local):
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    gidx = np.ascontiguousarray(gidx, dtype=np.int64)
    log2phy = np.ascontiguousarray(log2phy, dtype=np.int32)
    n_replica = np.ascontiguousarray(n_replica, dtype=np.int32)
    T, K = ids.shape
    out = np.empty_like(ids)
    rc = lib().orc_eplb_remap(_p(ids), _p(gidx), T, K, _p(log2phy), _p(n_replica), log2phy.shape[1],
                              log2phy.shape[0], phys_begin, n_local, _p(out))
    if rc != OK:
        raise ValueError("orc_eplb_remap: invalid arguments")
    return out


def layout(ids, n_local, kind, block_m=1, m_max=0, m_cap=None):
    """Returns dict(counts, offsets, masked_m, pos, row_src, status, detail)."""
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    T, K = ids.shape
    if m_cap is None:
        m_cap = n_local * m_max if kind == MASKED else T * K + n_local * (block_m - 1)
    counts = np.empty(n_local, np.int32)
    offsets = np.empty(n_local + 1, np.int32)
    masked_m = np.empty(n_local, np.int32)
    pos = np.empty((T, K), np.int32)
    row_src = np.empty(max(m_cap, 1), np.int32)[:m_cap]
    detail = np.zeros(1, np.int32)
    st = lib().orc_layout(_p(ids), T, K, n_local, kind, block_m, m_max, m_cap, _p(counts), _p(offsets),
                          _p(masked_m), _p(pos), _p(row_src), _p(detail))
    if st == EINVAL:
        raise ValueError("orc_layout: invalid arguments")
    return dict(counts=counts, offsets=offsets, masked_m=masked_m, pos=pos, row_src=row_src,
                status=st, detail=int(detail[0]), m_cap=m_cap)


# ---------------------------------------------------------------- FFN + combine
_DT_NP = {F32: np.float32, BF16: np.uint16, FP8: np.uint8}


def _ptr_array(lst):
    arr = (ctypes.c_void_p * max(len(lst), 1))()
    for i, a in enumerate(lst):
        arr[i] = None if a is None else a.ctypes.data
    return arr


def moe_layer(dt, x, local_ids, topk_w, experts, shared=None, x_scales=None, sel=None, out_dt=None,
              want_y=False):
    """The layer by definition for the tokens in ``sel``.

    experts: list over local experts of dict(W1, W3, W2[, s1, s3, s2]) or None
    (unused).  Arrays are numpy in storage form (fp32, uint16 bf16 bits or
    uint8 fp8 codes).  shared: the same dict for the shared expert, or None.
    Returns out [n_sel, H] (float32, or uint16 bf16 bits) and optionally the
    stored expert outputs [n_sel, K, H] (float64).
    """
    x = np.ascontiguousarray(x)
    T, H = x.shape
    local_ids = np.ascontiguousarray(local_ids, dtype=np.int32)
    topk_w = np.ascontiguousarray(topk_w, dtype=np.float32)
    K = local_ids.shape[1]
    if out_dt is None:
        out_dt = F32 if dt == F32 else BF16
    sel = np.arange(T, dtype=np.int32) if sel is None else np.ascontiguousarray(sel, dtype=np.int32)
    I = None
    W1, W3, W2, S1, S3, S2 = [], [], [], [], [], []
    keep = []
    for ex in experts:
        if ex is None:
            for l in (W1, W3, W2, S1, S3, S2):
                l.append(None)
            continue
        arrs = {k: np.ascontiguousarray(v) for k, v in ex.items()}
        keep.append(arrs)
        I = arrs["W1"].shape[0]
        W1.append(arrs["W1"]); W3.append(arrs["W3"]); W2.append(arrs["W2"])
        S1.append(arrs.get("s1")); S3.append(arrs.get("s3")); S2.append(arrs.get("s2"))
    if shared is not None:
        shared = {k: np.ascontiguousarray(v) for k, v in shared.items()}
        sh_I = shared["W1"].shape[0]
    else:
        sh_I = 0
    if I is None:
        I = max(sh_I, 128)
    pw = [_ptr_array(l) for l in (W1, W3, W2, S1, S3, S2)]
    out = np.empty((len(sel), H), dtype=np.float32 if out_dt == F32 else np.uint16)
    y_rows = np.empty((len(sel), K, H), dtype=np.float64) if want_y else None
    g = (lambda k: _p(shared[k]) if shared is not None and k in shared else None)
    rc = lib().orc_moe_layer(dt, H, I, K, _p(x), _p(x_scales), _p(local_ids), _p(topk_w),
                             *[ctypes.cast(p, ctypes.c_void_p) for p in pw],
                             g("W1"), g("W3"), g("W2"), g("s1"), g("s3"), g("s2"), sh_I,
                             _p(sel), len(sel), out_dt, _p(out), _p(y_rows))
    if rc != OK:
        raise ValueError("orc_moe_layer: invalid arguments")
    return (out, y_rows) if want_y else out


def combine(y_perm, pos, topk_w, shared_out=None, out_dt=BF16):
    y_perm = np.ascontiguousarray(y_perm)
    y_dt = F32 if y_perm.dtype == np.float32 else BF16
    pos = np.ascontiguousarray(pos, dtype=np.int32)
    topk_w = np.ascontiguousarray(topk_w, dtype=np.float32)
    T, K = pos.shape
    H = y_perm.shape[1]
    out = np.empty((T, H), dtype=np.float32 if out_dt == F32 else np.uint16)
    sh = None if shared_out is None else np.ascontiguousarray(shared_out)
    lib().orc_combine(y_dt, _p(y_perm), _p(pos), _p(topk_w), T, K, H, _p(sh), out_dt, _p(out))
    return out


def comm_bytes(b, K, H, s):
    """Logical per-rank dispatch volume of one layer: each of b tokens sends
    its H-vector of s-byte elements to K experts (DeepEP deep-dive, section
    on the traffic volume: 128 tokens, K=8, H=7168, 1 byte is about 7.3 MB)."""
    return b * K * H * s


def rel_err(out, ref):
    """max|out - ref| / max|ref| over a tensor (float64 inputs)."""
    out = np.asarray(out, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.max(np.abs(ref))
    return float(np.max(np.abs(out - ref)) / den) if den > 0 else float(np.max(np.abs(out - ref)))
