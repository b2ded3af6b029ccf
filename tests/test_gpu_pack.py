"""GPU check of rdg_pack_weights against an independent numpy statement of
the tile order: tiles of 16 rows x KS reduction elements (KS = 4 fp32, 32
bf16, 128 fp8), ordered by matrix, row group, then K; inside a tile lane
l = 16*g + r holds row r and the g-th quarter of the tile's KS elements;
an fp8 lane's 32 bytes are stored as two KiB halves."""
import numpy as np
import pytest
import torch

from harness import DEV, np_of, rdg

pytestmark = pytest.mark.gpu


def ref_pack(w, ks):
    n, rows, cols = w.shape
    q = ks // 4
    t = w.reshape(n, rows // 16, 16, cols // ks, 4, q)          # mat, rg, r, kstep, g, j
    t = t.transpose(0, 1, 3, 4, 2, 5)                            # mat, rg, kstep, g, r, j  (lane = 16g + r)
    if w.dtype == np.uint8:                                      # fp8: halves of 16 bytes
        t = t.reshape(n, rows // 16, cols // ks, 64, 2, 16).transpose(0, 1, 2, 4, 3, 5)
    return np.ascontiguousarray(t).reshape(-1)


@pytest.mark.parametrize("dt,ks,shape", [("f32", 4, (2, 32, 256)), ("bf16", 32, (3, 48, 384)),
                                         ("fp8", 128, (2, 16, 512)), ("bf16", 32, (1, 2048, 7168))])
def test_pack_order(dt, ks, shape):
    m = rdg()
    g = torch.Generator(device=DEV)
    g.manual_seed(1)
    if dt == "f32":
        w = torch.randn(shape, generator=g, device=DEV)
        code = m.RDG_F32
    elif dt == "bf16":
        w = torch.randn(shape, generator=g, device=DEV).to(torch.bfloat16)
        code = m.RDG_BF16
    else:
        w = torch.randint(0, 255, shape, generator=g, device=DEV, dtype=torch.int32).to(torch.uint8)
        code = m.RDG_FP8_E4M3
    p = torch.empty_like(w)
    m.rdg_pack_weights(w, code, p)
    torch.cuda.synchronize()
    assert np.array_equal(np_of(p).reshape(-1), ref_pack(np_of(w), ks))
