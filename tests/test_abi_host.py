"""Host-side checks of the C ABI (no GPU needed, no kernel is launched).

* the shared library loads and exports every function include/libmx.h declares;
* the size helpers follow the storage arithmetic of the "Bit Layout" page;
* every validation error is returned before anything is enqueued (the
  pointers passed here are never dereferenced: each call fails validation).
"""
import os
import re

import pytest

from bit_gemm_mx_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "libmx.h")


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(B.LIB_PATH):
        from bit_gemm_mx_amd.build import build
        build()
    return B.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mx_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    assert declared_functions() == sorted([
        "mx_abi_version", "mx_block_matmul", "mx_block_matmul_f32b", "mx_block_matmul_quantize_a",
        "mx_codes_bytes",
        "mx_dequantize",
        "mx_dequantize_axis", "mx_fold_scale", "mx_num_scale_blocks", "mx_quantize",
        "mx_quantize_axis", "mx_status_string"])


def test_library_exports_every_declared_symbol(L):
    for name in declared_functions():
        assert hasattr(L, name), name


def test_abi_version(L):
    assert B.mx_abi_version() == 3


def test_size_helpers(L):
    assert B.mx_codes_bytes(256, 1024, B.MX_E2M1) == 131072
    assert B.mx_codes_bytes(256, 1024, B.MX_E4M3) == 262144
    assert B.mx_codes_bytes(4, 32, 9) == 0
    assert B.mx_num_scale_blocks(256, 1024) == 8192
    assert B.mx_num_scale_blocks(8192, 8192) == 2097152
    assert B.mx_num_scale_blocks(3, 33) == 0
    # 136 bits per block of 32 E2M1 elements ("Bit Layout", storage figure)
    bits = (B.mx_codes_bytes(1, 32, B.MX_E2M1) + B.mx_num_scale_blocks(1, 32)) * 8
    assert bits == 136


def test_status_strings(L):
    for s in range(6):
        assert isinstance(B.mx_status_string(s), str) and B.mx_status_string(s)
    assert B.mx_status_string(0) == "ok"


# Fake, never-dereferenced device addresses.
X, C, S, Y = 0x10000, 0x20000, 0x30000, 0x40000


@pytest.mark.parametrize("args,status", [
    ((0, C, S, 4, 64, 1, 32), 1),           # null x
    ((X, 0, S, 4, 64, 1, 32), 1),           # null codes
    ((X, C, 0, 4, 64, 1, 32), 1),           # null scales
    ((X, C, S, 4, 64, 3, 32), 3),           # bad element type
    ((X, C, S, 4, 64, 1, 16), 3),           # block size other than 32
    ((X, C, S, 0, 64, 1, 32), 2),           # no rows
    ((X, C, S, 4, 0, 1, 32), 2),            # no cols
    ((X, C, S, 4, 48, 1, 32), 2),           # cols not a multiple of 32
    ((X, C, S, -1, 64, 2, 32), 2),          # negative rows
    ((X + 4, C, S, 4, 64, 1, 32), 4),       # misaligned x
    ((X, C + 8, S, 4, 64, 2, 32), 4),       # misaligned codes
])
def test_codec_validation(L, args, status):
    assert L.mx_quantize(*args, None) == status
    x, c, s, r, k, e, bs = args
    assert L.mx_dequantize(c, s, x, r, k, e, bs, None) == status


@pytest.mark.parametrize("args,status", [
    ((X, C, S, 64, 4, 2, 1, 32), 3),        # axis other than 0 / 1
    ((X, C, S, 64, 4, -1, 1, 32), 3),
    ((X, C, S, 48, 4, 0, 1, 32), 2),        # axis 0: rows not a multiple of 32
    ((X, C, S, 64, 0, 0, 1, 32), 2),        # no cols
    ((X, C, S, 64, 4, 0, 5, 32), 3),        # bad element type
    ((X, C, S, 64, 4, 0, 1, 8), 3),         # block size other than 32
    ((0, C, S, 64, 4, 0, 1, 32), 1),        # null x
    ((X, C, 0, 64, 4, 0, 2, 32), 1),        # null scales
    ((X + 8, C, S, 64, 4, 0, 1, 32), 4),    # misaligned x
    ((X, C + 4, S, 64, 4, 0, 1, 32), 4),    # misaligned codes
    ((X, C, S, 4, 48, 1, 1, 32), 2),        # axis 1: cols not a multiple of 32
])
def test_axis_codec_validation(L, args, status):
    x, c, s, r, k, axis, e, bs = args
    assert L.mx_quantize_axis(x, c, s, r, k, axis, e, bs, None) == status
    assert L.mx_dequantize_axis(c, s, x, r, k, axis, e, bs, None) == status


def test_fold_scale_validation(L):
    assert L.mx_fold_scale(0, 16, 3, None) == 1
    assert L.mx_fold_scale(S, 0, 3, None) == 2
    assert L.mx_fold_scale(S, -5, 3, None) == 2


@pytest.mark.parametrize("over,status", [
    (dict(a=0), 1), (dict(sa=0), 1), (dict(b=0), 1), (dict(sb=0), 1), (dict(c=0), 1),
    (dict(ae=0), 3), (dict(be=7), 3), (dict(bs=64), 3),
    (dict(M=0), 2), (dict(N=0), 2), (dict(K=0), 2), (dict(K=100), 2), (dict(M=-3), 2),
    (dict(a=X + 1), 4), (dict(b=C + 2), 4), (dict(c=Y + 4), 4),
])
def test_matmul_validation(L, over, status):
    a = dict(a=X, sa=S, ae=1, b=C, sb=S + 4096, be=2, c=Y, M=16, N=16, K=128, bs=32, acc=0)
    a.update(over)
    assert L.mx_block_matmul(a["a"], a["sa"], a["ae"], a["b"], a["sb"], a["be"], a["c"],
                             a["M"], a["N"], a["K"], a["bs"], a["acc"], None) == status


@pytest.mark.parametrize("over,status", [
    (dict(a=0), 1), (dict(sa=0), 1), (dict(b=0), 1), (dict(c=0), 1),
    (dict(ae=3), 3), (dict(bs=16), 3),
    (dict(M=0), 2), (dict(N=0), 2), (dict(K=0), 2), (dict(K=48), 2), (dict(N=-1), 2),
    (dict(a=X + 8), 4), (dict(b=C + 2), 4), (dict(c=Y + 1), 4),
])
def test_matmul_f32b_validation(L, over, status):
    a = dict(a=X, sa=S, ae=2, b=C, c=Y, M=16, N=16, K=128, bs=32, acc=0)
    a.update(over)
    assert L.mx_block_matmul_f32b(a["a"], a["sa"], a["ae"], a["b"], a["c"], a["M"], a["N"],
                                  a["K"], a["bs"], a["acc"], None) == status


@pytest.mark.parametrize("over,status", [
    (dict(a=0), 1), (dict(b=0), 1), (dict(sb=0), 1), (dict(c=0), 1),
    (dict(ae=0), 3), (dict(be=5), 3), (dict(bs=64), 3),
    (dict(M=0), 2), (dict(N=0), 2), (dict(K=0), 2), (dict(K=40), 2), (dict(M=-2), 2),
    (dict(a=X + 4), 4), (dict(b=C + 8), 4), (dict(c=Y + 2), 4),
])
def test_matmul_quantize_a_validation(L, over, status):
    a = dict(a=X, ae=2, b=C, sb=S, be=1, c=Y, M=16, N=16, K=128, bs=32, acc=0)
    a.update(over)
    assert L.mx_block_matmul_quantize_a(a["a"], a["ae"], a["b"], a["sb"], a["be"], a["c"],
                                        a["M"], a["N"], a["K"], a["bs"], a["acc"], None) == status


def test_python_layer_rejects_cpu_tensors(L):
    import torch
    with pytest.raises(ValueError):
        B.quantize(torch.zeros(4, 64))


def _mx(rows, cols, elem, codes_n=None, scales_n=None, axis=1):
    """An MXTensor of CPU buffers, with the right sizes unless overridden."""
    import torch
    sr, sc = (rows, cols) if axis == 1 else (cols, rows)
    cn = sr * sc // 2 if elem == B.MX_E2M1 else sr * sc
    codes = torch.zeros(cn if codes_n is None else codes_n, dtype=torch.uint8)
    scales = torch.zeros(sr * sc // 32 if scales_n is None else scales_n, dtype=torch.uint8)
    return B.MXTensor(codes, scales, rows, cols, elem, axis)


def test_python_layer_checks_buffer_sizes(L):
    """A buffer that does not match the shape handed to the ABI is refused
    before any pointer reaches a kernel (a short one would be read or
    written out of bounds)."""
    import torch
    size = "must hold|must have shape"
    with pytest.raises(ValueError, match=size):                   # quantize into a short out
        B.quantize(torch.zeros(4, 64), B.MX_E2M1, out=_mx(4, 64, B.MX_E2M1, codes_n=100))
    with pytest.raises(ValueError, match=size):
        B.quantize(torch.zeros(4, 64), B.MX_E4M3, out=_mx(4, 64, B.MX_E4M3, scales_n=7))
    with pytest.raises(ValueError, match=size):                   # rows/cols that lie
        B.dequantize(_mx(4, 64, B.MX_E2M1, codes_n=96))
    with pytest.raises(ValueError, match=size):
        B.dequantize(_mx(4, 64, B.MX_E2M1), out=torch.zeros(4, 32))
    with pytest.raises(ValueError, match=size):                   # axis-0 storage
        B.dequantize(_mx(64, 4, B.MX_E4M3, codes_n=64 * 3, axis=0))
    with pytest.raises(ValueError, match=size):
        B.fold_scale(_mx(4, 64, B.MX_E2M1, scales_n=9), 1)
    a, bt = _mx(8, 64, B.MX_E4M3), _mx(16, 64, B.MX_E2M1)
    with pytest.raises(ValueError, match=size):                   # C of the wrong shape
        B.block_matmul(a, bt, out=torch.zeros(8, 15))
    with pytest.raises(ValueError, match=size):
        B.block_matmul(_mx(8, 64, B.MX_E4M3, codes_n=8 * 63), bt)
    with pytest.raises(ValueError, match=size):
        B.block_matmul(a, _mx(16, 64, B.MX_E2M1, scales_n=31))
    with pytest.raises(ValueError, match=size):
        B.block_matmul_f32b(a, torch.zeros(64, 5), out=torch.zeros(8, 6))
    with pytest.raises(ValueError, match=size):                   # fused quantize + matmul
        B.block_matmul_quantize_a(torch.zeros(8, 64), B.MX_E4M3, bt, out=torch.zeros(8, 17))
    with pytest.raises(ValueError, match=size):
        B.block_matmul_quantize_a(torch.zeros(8, 64), B.MX_E4M3, _mx(16, 64, B.MX_E2M1,
                                                                      codes_n=16 * 31))
    with pytest.raises(ValueError, match="K mismatch"):
        B.block_matmul_quantize_a(torch.zeros(8, 96), B.MX_E4M3, bt)
    with pytest.raises(ValueError, match="element type"):
        B.dequantize(B.MXTensor(torch.zeros(4), torch.zeros(4), 1, 32, 7))


def test_build_rejects_kernels_that_spill():
    """The build parses the compiler's resource-usage remarks and names every
    kernel with scratch memory (the tiled matmul's hand-counted load waits
    are only valid without spills)."""
    from bit_gemm_mx_amd import build
    remarks = "\n".join([
        "a.hip:1:1: remark: Function Name: k_ok [-Rpass-analysis=kernel-resource-usage]",
        "a.hip:1:1: remark:     ScratchSize [bytes/lane]: 0 [-Rpass-analysis=kernel-resource-usage]",
        "a.hip:9:1: remark: Function Name: k_spill [-Rpass-analysis=kernel-resource-usage]",
        "a.hip:9:1: remark:     VGPRs Spill: 12 [-Rpass-analysis=kernel-resource-usage]",
        "a.hip:9:1: remark:     ScratchSize [bytes/lane]: 48 [-Rpass-analysis=kernel-resource-usage]",
    ])
    assert build._scratch_kernels(remarks) == ["k_spill (48 bytes/lane)"]
    assert build._scratch_kernels("") == []
