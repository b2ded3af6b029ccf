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
