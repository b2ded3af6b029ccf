"""Host-side checks of the C ABI library: it loads without a GPU, exports
every entry point include/rdg.h declares, and the pure host queries
(argument validation, sizes, strings) behave as documented."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rdg.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(rdg_[a-z0-9_]+)\s*\(", src)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for must in ("rdg_route", "rdg_eplb_remap", "rdg_dispatch", "rdg_grouped_ffn", "rdg_combine"):
        assert must in names


def test_library_exports_every_declared_symbol():
    import routing_dispatch_grouped_amd as rdg
    lib = ctypes.CDLL(rdg.LIB_PATH)
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, missing


def test_host_queries_and_validation():
    import routing_dispatch_grouped_amd as rdg
    L = rdg._lib
    assert rdg.rdg_version() >= 100
    assert rdg.strerror(rdg.RDG_ECAPACITY).startswith("rows exceed")
    assert L.rdg_signal_threshold(7168, rdg.RDG_FP8_E4M3) == 7168  # counters count finished columns
    assert L.rdg_signal_threshold(100, rdg.RDG_BF16) == rdg.RDG_EINVAL
    # workspace grows with the dispatched entries and the expert count
    a = L.rdg_dispatch_workspace_bytes(128, 8, 256)
    b = L.rdg_dispatch_workspace_bytes(4096, 8, 256)
    assert 0 < a < b and b - a == 4 * (4096 - 128) * 8
    # argument errors return synchronously, before touching the device
    assert L.rdg_route(None, 4, 10, 4, 2, 2, 1.0, None, None, None) == rdg.RDG_EINVAL   # 10 % 4 != 0
    assert L.rdg_route(None, 4, 2048, 8, 4, 8, 1.0, None, None, None) == rdg.RDG_EINVAL  # N > 1024
    assert L.rdg_route(None, 0, 256, 8, 4, 8, 1.0, None, None, None) == rdg.RDG_OK      # B = 0 is a no-op
    lay = rdg.rdg_layout(rdg.RDG_MASKED, 4, 0, 256, 1000, 32, None, None, None, None, None, None, None)
    assert L.rdg_grouped_ffn(ctypes.byref(lay), rdg.RDG_BF16, 7168, 2048, *([None] * 12), None) == rdg.RDG_EINVAL
    assert L.rdg_quantize_fp8(None, rdg.RDG_F32, 4, 100, 1, None, None, None) == rdg.RDG_EINVAL


def test_layout_struct_matches_header():
    import routing_dispatch_grouped_amd as rdg
    # 6 int32 fields then 8 pointers
    assert ctypes.sizeof(rdg.rdg_layout) == 6 * 4 + 8 * 8
    assert rdg.rdg_layout.expert_load.offset == 24 + 7 * 8
    assert rdg.rdg_layout.counts.offset == 24


def test_pack_validation():
    import routing_dispatch_grouped_amd as rdg
    L = rdg._lib
    assert L.rdg_packed_weight_bytes(rdg.RDG_BF16, 256, 2048, 7168) == 256 * 2048 * 7168 * 2
    assert L.rdg_pack_weights(None, rdg.RDG_BF16, 1, 20, 128, None, None) == rdg.RDG_EINVAL   # rows % 16
    assert L.rdg_pack_weights(None, rdg.RDG_BF16, 1, 16, 100, None, None) == rdg.RDG_EINVAL   # cols % 128
    assert L.rdg_pack_weights(None, 7, 1, 16, 128, None, None) == rdg.RDG_EINVAL              # dtype


def _fake_layout(rdg, kind=0, n_local=4, block_m=128, m_max=0, m_cap=1024, n_rows=64):
    # stand-in device addresses (16-byte aligned, never dereferenced: every
    # call below fails its argument checks before anything is enqueued)
    a = [0x10000 * (i + 1) for i in range(8)]
    return rdg.rdg_layout(kind, n_local, block_m, m_max, m_cap, n_rows, *a)


def test_combine_argument_checks():
    import routing_dispatch_grouped_amd as rdg
    L = rdg._lib
    BF, F32 = rdg.RDG_BF16, rdg.RDG_F32
    y, w, out, sig = 0x100000, 0x200000, 0x300000, 0x400000
    lay = _fake_layout(rdg)                     # T = 8 tokens x K = 8 = 64 rows

    def comb(T=8, K=8, H=256, ydt=BF, odt=BF, yp=y, op=out, sh=None, s=None, sr=0, thr=0, to=0, mb=0, lay=lay):
        return L.rdg_combine(yp, ydt, ctypes.byref(lay), w, T, K, H, sh, op, odt, s, sr, thr, to, mb, None)

    assert comb(K=0) == rdg.RDG_EINVAL
    assert comb(K=33) == rdg.RDG_EINVAL
    assert comb(H=12) == rdg.RDG_EINVAL                      # H % 8
    assert comb(T=7) == rdg.RDG_EINVAL                       # T * K != the layout's rows
    assert comb(ydt=rdg.RDG_FP8_E4M3) == rdg.RDG_EUNSUPPORTED
    assert comb(ydt=F32, odt=BF) == rdg.RDG_EUNSUPPORTED     # fp32 rows are combined into fp32 only
    assert comb(yp=y + 4) == rdg.RDG_EINVAL                  # rows are read in 16-byte vectors
    assert comb(op=out + 8) == rdg.RDG_EINVAL
    assert comb(sh=out + 4) == rdg.RDG_EINVAL
    assert comb(mb=-1) == rdg.RDG_EINVAL
    # the polling form: threshold, timeout, signal rows, the unit counter's range
    assert comb(s=sig, sr=128, thr=0, to=100) == rdg.RDG_EINVAL
    assert comb(s=sig, sr=128, thr=7168, to=-1) == rdg.RDG_EINVAL
    assert comb(s=sig, sr=48, thr=7168, to=100) == rdg.RDG_EINVAL
    big = _fake_layout(rdg, m_cap=(1 << 30) - 1)
    assert comb(s=sig, sr=128, thr=7168, to=100, lay=big) == rdg.RDG_EUNSUPPORTED
    bad = _fake_layout(rdg, kind=7)
    assert comb(lay=bad) == rdg.RDG_EINVAL


def test_combine_finish_argument_checks():
    import routing_dispatch_grouped_amd as rdg
    L = rdg._lib
    BF = rdg.RDG_BF16
    y, w, out, sig = 0x100000, 0x200000, 0x300000, 0x400000
    lay = _fake_layout(rdg)

    def fin(T=8, K=8, H=256, ydt=BF, odt=BF, op=out, s=sig, sr=128, lay=lay):
        return L.rdg_combine_finish(y, ydt, ctypes.byref(lay), w, T, K, H, None, op, odt, s, sr, None)

    assert fin(s=None) == rdg.RDG_EINVAL                     # it closes the polling form's counter
    assert fin(sr=8) == rdg.RDG_EINVAL
    assert fin(T=9) == rdg.RDG_EINVAL
    assert fin(op=out + 2) == rdg.RDG_EINVAL
    assert fin(ydt=rdg.RDG_F32) == rdg.RDG_EUNSUPPORTED
    assert fin(lay=_fake_layout(rdg, m_cap=1 << 30)) == rdg.RDG_EUNSUPPORTED


def test_dispatch_and_ffn_argument_checks():
    import routing_dispatch_grouped_amd as rdg
    L = rdg._lib
    BF, F8 = rdg.RDG_BF16, rdg.RDG_FP8_E4M3
    x, xs, ids, xp, xps = 0x100000, 0x200000, 0x300000, 0x400000, 0x500000
    lay = _fake_layout(rdg)                     # 64 rows

    def disp(dt=BF, T=8, H=256, K=8, xpp=xp, xsp=None, xpsp=None, xx=x, lay=lay, fn=L.rdg_dispatch):
        return fn(xx, xsp, dt, T, H, ids, K, ctypes.byref(lay), xpp, xpsp, None)

    for fn in (L.rdg_dispatch, L.rdg_dispatch_noalloc):
        assert disp(H=200, fn=fn) == rdg.RDG_EINVAL                 # H % 16
        assert disp(dt=F8, H=1040, xsp=xs, xpsp=xps, fn=fn) == rdg.RDG_EINVAL   # fp8: H % 128
        assert disp(dt=F8, xsp=None, xpsp=xps, fn=fn) == rdg.RDG_EINVAL         # fp8 rows need their scales
        assert disp(xpp=None, xpsp=xps, fn=fn) == rdg.RDG_EINVAL    # scales out without rows out
        assert disp(xx=x + 8, fn=fn) == rdg.RDG_EINVAL              # 16-byte row copies
        assert disp(T=9, fn=fn) == rdg.RDG_EINVAL
        assert disp(K=33, fn=fn) == rdg.RDG_EINVAL
        assert disp(dt=9, fn=fn) == rdg.RDG_EINVAL
    # the allocation-free dispatch's static work area bounds the entries
    big = _fake_layout(rdg, m_cap=1 << 22, n_rows=(1 << 20) * 8)
    assert disp(T=1 << 20, lay=big, fn=L.rdg_dispatch_noalloc) == rdg.RDG_EUNSUPPORTED

    W, h, y = 0x600000, 0x700000, 0x800000
    def ffn(dt=BF, H=7168, I=2048, hp=h, yp=y, xpp=xp, lay=lay):
        return L.rdg_grouped_ffn(ctypes.byref(lay), dt, H, I, xpp, None, W, W, W, None, None, None, hp, None, yp,
                                 None, None)
    assert ffn(H=7100) == rdg.RDG_EINVAL                             # H % 128
    assert ffn(I=100) == rdg.RDG_EINVAL
    assert ffn(dt=7) == rdg.RDG_EINVAL
    assert ffn(hp=None) == rdg.RDG_EINVAL
    assert ffn(yp=y + 4) == rdg.RDG_EINVAL
    assert ffn(xpp=None) == rdg.RDG_EINVAL
    assert ffn(dt=F8) == rdg.RDG_EINVAL                              # fp8 without scales
    assert L.rdg_grouped_ffn_gather(ctypes.byref(lay), BF, 7168, 2048, x, None, 40, W, W, W, None, None, None, h,
                                    None, y, None, None) == rdg.RDG_EINVAL  # K > 32
    # an empty layout is a no-op whatever the buffers
    empty = _fake_layout(rdg, n_rows=0)
    assert ffn(lay=empty, hp=h) == rdg.RDG_OK
    assert L.rdg_fill_i32(None, 0, -1, None) == rdg.RDG_EINVAL
    assert L.rdg_check_status(None, None, None) == rdg.RDG_EINVAL
