"""The C ABI on real device buffers: every validation error returns its
status and writes nothing.

Each call below fails validation (a shape, element type, block size,
alignment, axis or null-pointer error) with every other argument a real,
correctly sized device buffer filled with a sentinel; after the call and a
device synchronisation, every byte of every buffer still holds its
sentinel.  Status codes: 1 null, 2 shape, 3 unsupported, 4 alignment.
"""
import pytest
import torch

from bit_gemm_mx_amd import binding as B

pytestmark = pytest.mark.gpu

NBYTES = 1 << 20  # every buffer: 1 MiB, 256-byte aligned by the allocator


@pytest.fixture()
def bufs():
    dev = torch.device("cuda")
    b = {"x": torch.full((NBYTES // 4,), -7.25, dtype=torch.float32, device=dev),
         "y": torch.full((NBYTES // 4,), 3.5, dtype=torch.float32, device=dev),
         "codes": torch.full((NBYTES,), 0xA5, dtype=torch.uint8, device=dev),
         "scales": torch.full((NBYTES,), 0x5A, dtype=torch.uint8, device=dev),
         "bcodes": torch.full((NBYTES,), 0x3C, dtype=torch.uint8, device=dev),
         "bscales": torch.full((NBYTES,), 0x77, dtype=torch.uint8, device=dev),
         "c": torch.full((NBYTES // 4,), 1.25, dtype=torch.float32, device=dev)}
    torch.cuda.synchronize()
    ref = {k: v.clone() for k, v in b.items()}
    p = {k: v.data_ptr() for k, v in b.items()}
    yield b, p
    torch.cuda.synchronize()
    for k in b:
        assert torch.equal(b[k], ref[k]), f"buffer {k} was written by a failing call"


CODEC = [  # rows, cols, elem, block size, x offset, codes offset, status
    (4, 48, 1, 32, 0, 0, 2),      # cols not a multiple of 32
    (-1, 64, 2, 32, 0, 0, 2),     # negative rows
    (4, 64, 5, 32, 0, 0, 3),      # bad element type
    (4, 64, 1, 16, 0, 0, 3),      # block size other than 32
    (4, 64, 2, 32, 4, 0, 4),      # x not 16-byte aligned
    (4, 64, 1, 32, 0, 8, 4),      # codes not 16-byte aligned
]


@pytest.mark.parametrize("rows,cols,elem,bs,xo,co,status", CODEC)
def test_codec_errors_write_nothing(bufs, rows, cols, elem, bs, xo, co, status):
    _, p = bufs
    L = B.lib()
    assert L.mx_quantize(p["x"] + xo, p["codes"] + co, p["scales"], rows, cols, elem, bs,
                         None) == status
    assert L.mx_dequantize(p["codes"] + co, p["scales"], p["y"] + xo, rows, cols, elem, bs,
                           None) == status


@pytest.mark.parametrize("rows,cols,axis,elem,status", [
    (64, 4, 2, 1, 3), (48, 4, 0, 1, 2), (64, 4, 0, 9, 3), (4, 48, 1, 2, 2), (64, 0, 0, 1, 2)])
def test_axis_codec_errors_write_nothing(bufs, rows, cols, axis, elem, status):
    _, p = bufs
    L = B.lib()
    assert L.mx_quantize_axis(p["x"], p["codes"], p["scales"], rows, cols, axis, elem, 32,
                              None) == status
    assert L.mx_dequantize_axis(p["codes"], p["scales"], p["y"], rows, cols, axis, elem, 32,
                                None) == status


def test_fold_scale_errors_write_nothing(bufs):
    _, p = bufs
    L = B.lib()
    assert L.mx_fold_scale(p["scales"], 0, 3, None) == 2
    assert L.mx_fold_scale(p["scales"], -4, 3, None) == 2


MATMUL = [  # overrides of a valid 64 x 64 x 256 E4M3 x E2M1 call, status
    (dict(K=100), 2), (dict(M=0), 2), (dict(N=-1), 2), (dict(ae=3), 3), (dict(be=0), 3),
    (dict(bs=64), 3), (dict(ao=4), 4), (dict(bo=8), 4), (dict(co=4), 4), (dict(sa=0), 1),
    (dict(sb=0), 1)]


@pytest.mark.parametrize("over,status", MATMUL)
@pytest.mark.parametrize("acc", [0, 1])
def test_matmul_errors_write_nothing(bufs, over, status, acc):
    _, p = bufs
    L = B.lib()
    a = dict(M=64, N=64, K=256, ae=2, be=1, bs=32, ao=0, bo=0, co=0, sa=p["scales"],
             sb=p["bscales"])
    a.update(over)
    assert L.mx_block_matmul(p["codes"] + a["ao"], a["sa"], a["ae"], p["bcodes"] + a["bo"],
                             a["sb"], a["be"], p["c"] + a["co"], a["M"], a["N"], a["K"],
                             a["bs"], acc, None) == status


@pytest.mark.parametrize("over,status", [
    (dict(K=48), 2), (dict(N=0), 2), (dict(ae=4), 3), (dict(bs=16), 3), (dict(ao=2), 4),
    (dict(bo=2), 4), (dict(co=2), 4)])
def test_matmul_f32b_errors_write_nothing(bufs, over, status):
    _, p = bufs
    L = B.lib()
    a = dict(M=64, N=64, K=256, ae=1, bs=32, ao=0, bo=0, co=0)
    a.update(over)
    assert L.mx_block_matmul_f32b(p["codes"] + a["ao"], p["scales"], a["ae"], p["x"] + a["bo"],
                                  p["c"] + a["co"], a["M"], a["N"], a["K"], a["bs"], 1,
                                  None) == status


@pytest.mark.parametrize("over,status", [
    (dict(K=40), 2), (dict(M=-2), 2), (dict(ae=0), 3), (dict(be=6), 3), (dict(ao=4), 4),
    (dict(bo=4), 4), (dict(co=2), 4)])
def test_matmul_quantize_a_errors_write_nothing(bufs, over, status):
    _, p = bufs
    L = B.lib()
    a = dict(M=64, N=64, K=256, ae=2, be=1, ao=0, bo=0, co=0)
    a.update(over)
    assert L.mx_block_matmul_quantize_a(p["x"] + a["ao"], a["ae"], p["bcodes"] + a["bo"],
                                        p["bscales"], a["be"], p["c"] + a["co"], a["M"],
                                        a["N"], a["K"], 32, 0, None) == status
