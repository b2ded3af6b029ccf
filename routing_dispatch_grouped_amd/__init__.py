"""Thin Python binding of librdg.so (include/rdg.h): argument marshalling only.

Every function carries the C entry point's name and forwards torch device
tensors as raw pointers plus torch's current HIP stream.  Nothing here
computes any step of the layer.  Importing fails loudly when the built
library is missing: there is no fallback path.
"""
import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "librdg.so")

RDG_OK, RDG_EINVAL, RDG_ECAPACITY, RDG_ETIMEOUT, RDG_EHIP, RDG_EUNSUPPORTED = 0, -1, -2, -3, -4, -5
RDG_F32, RDG_BF16, RDG_FP8_E4M3, RDG_FP8_E4M3_UE8M0 = 0, 1, 2, 3
RDG_CONTIGUOUS, RDG_MASKED = 0, 1


class RdgError(RuntimeError):
    def __init__(self, code, what):
        self.code = code
        super().__init__("%s: %s (%d)" % (what, strerror(code), code))


class rdg_layout(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("n_local", ctypes.c_int32), ("block_m", ctypes.c_int32),
                ("m_max", ctypes.c_int32), ("m_cap", ctypes.c_int32), ("n_rows", ctypes.c_int32),
                ("counts", ctypes.c_void_p), ("offsets", ctypes.c_void_p), ("masked_m", ctypes.c_void_p),
                ("pos", ctypes.c_void_p), ("row_src", ctypes.c_void_p), ("status", ctypes.c_void_p),
                ("work", ctypes.c_void_p), ("expert_load", ctypes.c_void_p)]


if not os.path.exists(LIB_PATH):
    raise ImportError("librdg.so is not built (run routing_dispatch_grouped_amd/_build.py or "
                      "__graft_entry__.build()); there is no fallback implementation")

_lib = ctypes.CDLL(LIB_PATH)
_P, _I, _I64, _F, _SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
_LP = ctypes.POINTER(rdg_layout)

_SIGS = {
    "rdg_route": ([_P, _I, _I, _I, _I, _I, _F, _P, _P, _P], _I),
    "rdg_route_biased": ([_P, _P, _I, _I, _I, _I, _I, _F, _P, _P, _P], _I),
    "rdg_eplb_place": ([_P, _I, _I, _I, _I, _I, _I, _P, _P, _P, _P], _I),
    "rdg_eplb_remap": ([_P, _P, _I, _I, _P, _P, _I, _I, _I, _I, _P, _P], _I),
    "rdg_tbo_split": ([_P, _I, _I], _I),
    "rdg_dispatch_workspace_bytes": ([_I, _I, _I], _SZ),
    "rdg_dispatch": ([_P, _P, _I, _I, _I, _P, _I, _LP, _P, _P, _P], _I),
    "rdg_dispatch_noalloc": ([_P, _P, _I, _I, _I, _P, _I, _LP, _P, _P, _P], _I),
    "rdg_layout_tables_bytes": ([_I], _SZ),
    "rdg_layout_dense": ([_I, _LP, _P], _I),
    "rdg_grouped_ffn": ([_LP, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P], _I),
    "rdg_grouped_gate_up": ([_LP, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P, _P, _P], _I),
    "rdg_grouped_down": ([_LP, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P], _I),
    "rdg_grouped_ffn_gather": ([_LP, _I, _I, _I, _P, _P, _I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P], _I),
    "rdg_grouped_gate_up_gather": ([_LP, _I, _I, _I, _P, _P, _I, _P, _P, _P, _P, _P, _P, _P], _I),
    "rdg_signal_rows": ([_LP, _I, _I, _I], _I),
    "rdg_signal_threshold": ([_I, _I], _I),
    "rdg_combine": ([_P, _I, _LP, _P, _I, _I, _I, _P, _P, _I, _P, _I, _I, _I64, _I, _P], _I),
    "rdg_combine_finish": ([_P, _I, _LP, _P, _I, _I, _I, _P, _P, _I, _P, _I, _P], _I),
    "rdg_quantize_fp8": ([_P, _I, _I, _I, _I, _P, _P, _P], _I),
    "rdg_quantize_fp8_ue8m0": ([_P, _I, _I, _I, _I, _P, _P, _P], _I),
    "rdg_fill_i32": ([_P, ctypes.c_int32, _I64, _P], _I),
    "rdg_packed_weight_bytes": ([_I, _I, _I, _I], _SZ),
    "rdg_pack_weights": ([_P, _I, _I, _I, _I, _P, _P], _I),
    "rdg_check_status": ([_P, _P, _P], _I),
    "rdg_strerror": ([_I], ctypes.c_char_p),
    "rdg_version": ([], _I),
}
for _name, (_args, _ret) in _SIGS.items():
    _fn = getattr(_lib, _name)
    _fn.argtypes = _args
    _fn.restype = _ret


def strerror(code):
    return _lib.rdg_strerror(code).decode()


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _check(rc, what):
    if rc != RDG_OK:
        raise RdgError(rc, what)


# ------------------------------------------------------------------ layout
class Layout:
    """Device buffers of an rdg_layout, allocated with torch on ``device``."""

    def __init__(self, kind, n_local, T, K, device, block_m=128, m_max=0, m_cap=None, expert_load=None):
        import torch
        self.kind, self.n_local, self.T, self.K = kind, n_local, T, K
        n_rows = T * K
        if m_cap is None:
            m_cap = n_local * m_max if kind == RDG_MASKED else n_rows + n_local * (block_m - 1)
        i32 = dict(dtype=torch.int32, device=device)
        self.counts = torch.zeros(n_local, **i32)
        self.offsets = torch.zeros(n_local + 1, **i32)
        self.masked_m = torch.zeros(n_local, **i32)
        self.pos = torch.empty(max(n_rows, 1), **i32)
        self.row_src = torch.empty(max(m_cap, 1), **i32)
        self.status = torch.zeros(2, **i32)
        wb = rdg_dispatch_workspace_bytes(T, K, n_local)
        self.work = torch.zeros(max(wb, 256), dtype=torch.uint8, device=device)
        self.c = rdg_layout(kind, n_local, block_m, m_max, m_cap, n_rows,
                            self.counts.data_ptr(), self.offsets.data_ptr(), self.masked_m.data_ptr(),
                            self.pos.data_ptr(), self.row_src.data_ptr(), self.status.data_ptr(),
                            self.work.data_ptr(), expert_load.data_ptr() if expert_load is not None else None)
        self.expert_load = expert_load  # optional int64 [n_local] accumulated by rdg_dispatch
        self.m_cap = m_cap
        self.block_m = block_m
        self.m_max = m_max

    @property
    def ref(self):
        return ctypes.byref(self.c)


# ------------------------------------------------------------------ entry points
def rdg_version():
    return _lib.rdg_version()


def rdg_dispatch_workspace_bytes(T, K, n_local):
    return int(_lib.rdg_dispatch_workspace_bytes(T, K, n_local))


def rdg_route(logits, n_group, topk_group, K, scale, topk_ids, topk_w, stream=None):
    B, N = logits.shape
    _check(_lib.rdg_route(_ptr(logits), B, N, n_group, topk_group, K, scale, _ptr(topk_ids), _ptr(topk_w),
                          _stream(stream)), "rdg_route")


def rdg_route_biased(logits, bias, n_group, topk_group, K, scale, topk_ids, topk_w, stream=None):
    B, N = logits.shape
    _check(_lib.rdg_route_biased(_ptr(logits), _ptr(bias), B, N, n_group, topk_group, K, scale, _ptr(topk_ids),
                                 _ptr(topk_w), _stream(stream)), "rdg_route_biased")


def rdg_eplb_place(load, n_groups, n_nodes, n_gpus, n_physical, r_max):
    """Host call on numpy arrays: load [n_logical] (converted to float64).
    Returns (phy2log [n_physical] int32, log2phy [n_logical, r_max] int32,
    n_replica [n_logical] int32, gpu_load [n_gpus] float64)."""
    import numpy as np
    load = np.ascontiguousarray(load, dtype=np.float64)
    n = load.shape[0]
    phy2log = np.empty(n_physical, np.int32)
    log2phy = np.empty((n, r_max), np.int32)
    n_replica = np.empty(n, np.int32)
    gpu_load = np.empty(n_gpus, np.float64)
    hp = lambda a: ctypes.c_void_p(a.ctypes.data)
    _check(_lib.rdg_eplb_place(hp(load), n, n_groups, n_nodes, n_gpus, n_physical, r_max, hp(phy2log), hp(log2phy),
                               hp(n_replica), hp(gpu_load)), "rdg_eplb_place")
    return phy2log, log2phy, n_replica, gpu_load


def rdg_tbo_split(seq_lens, decode=False):
    """Host call: seq_lens is a sequence of token counts.  Returns the number of
    sequences in the first micro-batch."""
    import numpy as np
    a = np.ascontiguousarray(seq_lens, dtype=np.int32)
    rc = _lib.rdg_tbo_split(ctypes.c_void_p(a.ctypes.data), a.shape[0], int(bool(decode)))
    if rc < 0:
        raise RdgError(rc, "rdg_tbo_split")
    return rc


def rdg_eplb_remap(ids, token_gidx, log2phy, n_replica, phys_begin, n_local, local_ids, stream=None):
    T, K = ids.shape
    n_logical, r_max = log2phy.shape
    _check(_lib.rdg_eplb_remap(_ptr(ids), _ptr(token_gidx), T, K, _ptr(log2phy), _ptr(n_replica), r_max,
                               n_logical, phys_begin, n_local, _ptr(local_ids), _stream(stream)),
           "rdg_eplb_remap")


def rdg_dispatch(x, x_scales, dtype, ids, layout, x_perm, x_perm_scales=None, stream=None):
    T, H = x.shape
    K = ids.shape[1]
    _check(_lib.rdg_dispatch(_ptr(x), _ptr(x_scales), dtype, T, H, _ptr(ids), K, layout.ref, _ptr(x_perm),
                             _ptr(x_perm_scales), _stream(stream)), "rdg_dispatch")


def rdg_layout_tables_bytes(n_local):
    return int(_lib.rdg_layout_tables_bytes(n_local))


def rdg_dispatch_noalloc(x, x_scales, dtype, ids, layout, x_perm, x_perm_scales=None, stream=None):
    """rdg_dispatch with its scratch in the library's static device array
    (layout.work then needs only rdg_layout_tables_bytes(n_local) bytes)."""
    T, H = x.shape
    K = ids.shape[1]
    _check(_lib.rdg_dispatch_noalloc(_ptr(x), _ptr(x_scales), dtype, T, H, _ptr(ids), K, layout.ref, _ptr(x_perm),
                                     _ptr(x_perm_scales), _stream(stream)), "rdg_dispatch_noalloc")


def rdg_layout_dense(T, layout, stream=None):
    _check(_lib.rdg_layout_dense(T, layout.ref, _stream(stream)), "rdg_layout_dense")


def rdg_grouped_ffn(layout, dtype, H, I, x_perm, x_perm_scales, W1, W3, W2, W1_s, W3_s, W2_s, h_ws, h_scales_ws,
                    y, signals=None, stream=None):
    _check(_lib.rdg_grouped_ffn(layout.ref, dtype, H, I, _ptr(x_perm), _ptr(x_perm_scales), _ptr(W1), _ptr(W3),
                                _ptr(W2), _ptr(W1_s), _ptr(W3_s), _ptr(W2_s), _ptr(h_ws), _ptr(h_scales_ws),
                                _ptr(y), _ptr(signals), _stream(stream)), "rdg_grouped_ffn")


def rdg_grouped_gate_up(layout, dtype, H, I, x_perm, x_perm_scales, W1, W3, W1_s, W3_s, h_ws, h_scales_ws,
                        stream=None):
    _check(_lib.rdg_grouped_gate_up(layout.ref, dtype, H, I, _ptr(x_perm), _ptr(x_perm_scales), _ptr(W1), _ptr(W3),
                                    _ptr(W1_s), _ptr(W3_s), _ptr(h_ws), _ptr(h_scales_ws), _stream(stream)),
           "rdg_grouped_gate_up")


def rdg_grouped_ffn_gather(layout, dtype, H, I, x, x_scales, K, W1, W3, W2, W1_s, W3_s, W2_s, h_ws, h_scales_ws,
                           y, signals=None, stream=None):
    _check(_lib.rdg_grouped_ffn_gather(layout.ref, dtype, H, I, _ptr(x), _ptr(x_scales), K, _ptr(W1), _ptr(W3),
                                       _ptr(W2), _ptr(W1_s), _ptr(W3_s), _ptr(W2_s), _ptr(h_ws), _ptr(h_scales_ws),
                                       _ptr(y), _ptr(signals), _stream(stream)), "rdg_grouped_ffn_gather")


def rdg_grouped_gate_up_gather(layout, dtype, H, I, x, x_scales, K, W1, W3, W1_s, W3_s, h_ws, h_scales_ws,
                               stream=None):
    _check(_lib.rdg_grouped_gate_up_gather(layout.ref, dtype, H, I, _ptr(x), _ptr(x_scales), K, _ptr(W1), _ptr(W3),
                                           _ptr(W1_s), _ptr(W3_s), _ptr(h_ws), _ptr(h_scales_ws), _stream(stream)),
           "rdg_grouped_gate_up_gather")


def rdg_grouped_down(layout, dtype, H, I, h_ws, h_scales_ws, W2, W2_s, y, signals=None, stream=None):
    _check(_lib.rdg_grouped_down(layout.ref, dtype, H, I, _ptr(h_ws), _ptr(h_scales_ws), _ptr(W2), _ptr(W2_s),
                                 _ptr(y), _ptr(signals), _stream(stream)), "rdg_grouped_down")


def rdg_signal_rows(layout, dtype, H, I):
    r = _lib.rdg_signal_rows(layout.ref, dtype, H, I)
    _check(min(r, 0), "rdg_signal_rows")
    return r


def rdg_signal_threshold(H, dtype):
    r = _lib.rdg_signal_threshold(H, dtype)
    _check(min(r, 0), "rdg_signal_threshold")
    return r


def rdg_combine(y, y_dtype, layout, topk_w, T, K, H, shared_out, out, out_dtype, signals=None, signal_rows=0,
                threshold=0, timeout_us=0, max_blocks=0, stream=None):
    _check(_lib.rdg_combine(_ptr(y), y_dtype, layout.ref, _ptr(topk_w), T, K, H, _ptr(shared_out), _ptr(out),
                            out_dtype, _ptr(signals), signal_rows, threshold, timeout_us, max_blocks,
                            _stream(stream)), "rdg_combine")


def rdg_combine_finish(y, y_dtype, layout, topk_w, T, K, H, shared_out, out, out_dtype, signals, signal_rows,
                       stream=None):
    _check(_lib.rdg_combine_finish(_ptr(y), y_dtype, layout.ref, _ptr(topk_w), T, K, H, _ptr(shared_out),
                                   _ptr(out), out_dtype, _ptr(signals), signal_rows, _stream(stream)),
           "rdg_combine_finish")


def rdg_quantize_fp8(src, src_dtype, block_rows, q, scales, stream=None):
    rows, cols = src.shape
    _check(_lib.rdg_quantize_fp8(_ptr(src), src_dtype, rows, cols, block_rows, _ptr(q), _ptr(scales),
                                 _stream(stream)), "rdg_quantize_fp8")


def rdg_quantize_fp8_ue8m0(src, src_dtype, block_rows, q, scales, stream=None):
    rows, cols = src.shape
    _check(_lib.rdg_quantize_fp8_ue8m0(_ptr(src), src_dtype, rows, cols, block_rows, _ptr(q), _ptr(scales),
                                       _stream(stream)), "rdg_quantize_fp8_ue8m0")


def rdg_pack_weights(W, dtype, W_packed, stream=None):
    """W: [n_mat, rows, cols] (or [rows, cols]) device tensor; W_packed: same byte size."""
    shape = tuple(W.shape)
    n_mat, rows, cols = (1,) + shape if len(shape) == 2 else shape
    _check(_lib.rdg_pack_weights(_ptr(W), dtype, n_mat, rows, cols, _ptr(W_packed), _stream(stream)),
           "rdg_pack_weights")


def rdg_fill_i32(p, value, stream=None):
    _check(_lib.rdg_fill_i32(_ptr(p), value, p.numel(), _stream(stream)), "rdg_fill_i32")


def rdg_check_status(layout_or_status, stream=None):
    """Waits for the stream; returns (code, detail)."""
    st = layout_or_status.status if isinstance(layout_or_status, Layout) else layout_or_status
    host = (ctypes.c_int32 * 2)()
    rc = _lib.rdg_check_status(_ptr(st), host, _stream(stream))
    if rc in (RDG_EINVAL, RDG_EHIP):  # the query itself failed (device codes are -2 / -3)
        raise RdgError(rc, "rdg_check_status")
    return int(host[0]), int(host[1])
