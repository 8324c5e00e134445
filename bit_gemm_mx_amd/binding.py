"""ctypes binding of libmx (argument marshalling only).

Every computation runs in the HIP kernels behind the C ABI declared in
``include/libmx.h``; this module only checks tensor dtypes, sizes, devices and
contiguity, allocates outputs with ``torch.empty`` on the tensors' device and passes raw
pointers plus the current HIP stream.  There is no CPU path: if the shared
library is missing or fails to load, every call raises.
"""

from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmx.so")

MX_E2M1 = 1
MX_E4M3 = 2
BLOCK = 32
ELEM_NAMES = {MX_E2M1: "E2M1", MX_E4M3: "E4M3"}

_STATUS = {0: "MX_OK", 1: "MX_ERR_NULL", 2: "MX_ERR_SHAPE", 3: "MX_ERR_UNSUPPORTED",
           4: "MX_ERR_ALIGN", 5: "MX_ERR_HIP"}

_lib = None


class LibMXError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{_STATUS.get(status, status)}: {message}")
        self.status = status


def lib() -> ctypes.CDLL:
    """Load libmx.so (once) and declare its signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run `python -m bit_gemm_mx_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    p, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
    L.mx_quantize.argtypes = [p, p, p, i64, i64, i32, i32, p]
    L.mx_quantize.restype = i32
    L.mx_dequantize.argtypes = [p, p, p, i64, i64, i32, i32, p]
    L.mx_dequantize.restype = i32
    L.mx_block_matmul.argtypes = [p, p, i32, p, p, i32, p, i64, i64, i64, i32, i32, p]
    L.mx_block_matmul.restype = i32
    L.mx_block_matmul_f32b.argtypes = [p, p, i32, p, p, i64, i64, i64, i32, i32, p]
    L.mx_block_matmul_f32b.restype = i32
    L.mx_block_matmul_quantize_a.argtypes = [p, i32, p, p, i32, p, i64, i64, i64, i32, i32, p]
    L.mx_block_matmul_quantize_a.restype = i32
    L.mx_quantize_axis.argtypes = [p, p, p, i64, i64, i32, i32, i32, p]
    L.mx_quantize_axis.restype = i32
    L.mx_dequantize_axis.argtypes = [p, p, p, i64, i64, i32, i32, i32, p]
    L.mx_dequantize_axis.restype = i32
    L.mx_fold_scale.argtypes = [p, i64, i32, p]
    L.mx_fold_scale.restype = i32
    L.mx_codes_bytes.argtypes = [i64, i64, i32]
    L.mx_codes_bytes.restype = sz
    L.mx_num_scale_blocks.argtypes = [i64, i64, i32]
    L.mx_num_scale_blocks.restype = i64
    L.mx_status_string.argtypes = [i32]
    L.mx_status_string.restype = ctypes.c_char_p
    L.mx_abi_version.argtypes = []
    L.mx_abi_version.restype = i32
    _lib = L
    return L


def _check(status: int) -> None:
    if status != 0:
        raise LibMXError(status, lib().mx_status_string(status).decode())


# ----------------------------------------------------------------- raw ABI
def mx_quantize(x_ptr, codes_ptr, scales_ptr, rows, cols, elem, block_size=BLOCK, stream=None):
    _check(lib().mx_quantize(x_ptr, codes_ptr, scales_ptr, rows, cols, elem, block_size, stream))


def mx_dequantize(codes_ptr, scales_ptr, y_ptr, rows, cols, elem, block_size=BLOCK, stream=None):
    _check(lib().mx_dequantize(codes_ptr, scales_ptr, y_ptr, rows, cols, elem, block_size, stream))


def mx_quantize_axis(x_ptr, codes_ptr, scales_ptr, rows, cols, axis, elem, block_size=BLOCK,
                     stream=None):
    _check(lib().mx_quantize_axis(x_ptr, codes_ptr, scales_ptr, rows, cols, axis, elem,
                                  block_size, stream))


def mx_dequantize_axis(codes_ptr, scales_ptr, y_ptr, rows, cols, axis, elem, block_size=BLOCK,
                       stream=None):
    _check(lib().mx_dequantize_axis(codes_ptr, scales_ptr, y_ptr, rows, cols, axis, elem,
                                    block_size, stream))


def mx_fold_scale(scales_ptr, n_scales, j, stream=None):
    _check(lib().mx_fold_scale(scales_ptr, n_scales, j, stream))


def mx_block_matmul(a_codes, a_scales, a_elem, b_codes, b_scales, b_elem, c, M, N, K,
                    block_size=BLOCK, accumulate=0, stream=None):
    _check(lib().mx_block_matmul(a_codes, a_scales, a_elem, b_codes, b_scales, b_elem, c,
                                 M, N, K, block_size, accumulate, stream))


def mx_block_matmul_f32b(a_codes, a_scales, a_elem, b, c, M, N, K, block_size=BLOCK,
                         accumulate=0, stream=None):
    _check(lib().mx_block_matmul_f32b(a_codes, a_scales, a_elem, b, c, M, N, K, block_size,
                                      accumulate, stream))


def mx_block_matmul_quantize_a(a, a_elem, b_codes, b_scales, b_elem, c, M, N, K,
                               block_size=BLOCK, accumulate=0, stream=None):
    _check(lib().mx_block_matmul_quantize_a(a, a_elem, b_codes, b_scales, b_elem, c, M, N, K,
                                            block_size, accumulate, stream))


def mx_codes_bytes(rows, cols, elem) -> int:
    return int(lib().mx_codes_bytes(rows, cols, elem))


def mx_num_scale_blocks(rows, cols, block_size=BLOCK) -> int:
    return int(lib().mx_num_scale_blocks(rows, cols, block_size))


def mx_abi_version() -> int:
    return int(lib().mx_abi_version())


def mx_status_string(status: int) -> str:
    return lib().mx_status_string(status).decode()


# ------------------------------------------------------------ torch layer
def _stream_ptr(device):
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _require(t, dtype, name, numel=None, shape=None, device=None, on_gpu=True):
    """Type, contiguity and size of one tensor argument; then its device.

    Every kernel trusts the sizes it is given, so a buffer shorter than the
    shape passed to the ABI would be read or written out of bounds: sizes
    are checked here, before any pointer reaches the library."""
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name} must hold {numel} elements, got {t.numel()}")
    if not on_gpu:
        return
    if t.device.type != "cuda":
        raise ValueError(f"{name} must live on a GPU device, got {t.device}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, the other operands on {device}")


def _require_mx(t: "MXTensor", name: str, device=None, on_gpu=True):
    """An MXTensor whose codes and scales hold exactly the bytes its rows,
    cols, element type and block axis describe, on one device."""
    if t.elem not in ELEM_NAMES:
        raise ValueError(f"{name}: unsupported element type {t.elem}")
    if t.axis not in (0, 1):
        raise ValueError(f"{name}: block axis must be 0 or 1, got {t.axis}")
    if t.rows < 0 or t.cols < 0:
        raise ValueError(f"{name}: negative shape [{t.rows}, {t.cols}]")
    import torch
    sr, sc = (t.rows, t.cols) if t.axis == 1 else (t.cols, t.rows)
    codes = sr * sc // 2 if t.elem == MX_E2M1 else sr * sc
    _require(t.codes, torch.uint8, f"{name}.codes", numel=codes, on_gpu=False)
    _require(t.scales, torch.uint8, f"{name}.scales", numel=sr * (sc // BLOCK), on_gpu=False)
    if on_gpu:
        _require(t.codes, torch.uint8, f"{name}.codes", device=device)
        _require(t.scales, torch.uint8, f"{name}.scales", device=t.codes.device)


@dataclass
class MXTensor:
    """A block-scaled [rows, cols] tensor: element codes plus E8M0 scales.

    axis = 1 (blocks along the last axis):
      codes: uint8 [rows, cols/2] (E2M1, element 2j in the low nibble of byte j)
             or uint8 [rows, cols] (E4M3);  scales: uint8 [rows, cols/32].
    axis = 0 (blocks along axis 0), block-major storage, the layout of the
      transposed matrix: codes [cols, rows/2 or rows], scales [cols, rows/32].
    """
    codes: "object"
    scales: "object"
    rows: int
    cols: int
    elem: int
    axis: int = 1

    @property
    def device(self):
        return self.codes.device


def empty_mx(rows: int, cols: int, elem: int, device, axis: int = 1) -> MXTensor:
    import torch
    # storage is that of the [rows, cols] matrix blocked along its last axis,
    # or of its transpose when blocked along axis 0
    sr, sc = (rows, cols) if axis == 1 else (cols, rows)
    nbytes = mx_codes_bytes(sr, sc, elem)
    width = nbytes // sr if sr else 0
    codes = torch.empty((sr, width), dtype=torch.uint8, device=device)
    scales = torch.empty((sr, sc // BLOCK), dtype=torch.uint8, device=device)
    return MXTensor(codes, scales, rows, cols, elem, axis)


def quantize(x, elem: int = MX_E2M1, out: MXTensor | None = None, axis: int = 1) -> MXTensor:
    """float32 [rows, cols] GPU tensor -> MXTensor blocked along `axis`
    (mx_quantize, or mx_quantize_axis for axis 0)."""
    import torch
    if not isinstance(x, torch.Tensor) or x.dim() != 2:
        raise ValueError("x must be a 2-D [rows, cols] tensor")
    rows, cols = x.shape
    if out is None:
        out = empty_mx(rows, cols, elem, x.device, axis)
    if (out.rows, out.cols, out.elem, out.axis) != (rows, cols, elem, axis):
        raise ValueError("out does not describe x's shape, element type and block axis")
    _require_mx(out, "out")
    _require(x, torch.float32, "x", device=out.codes.device)
    mx_quantize_axis(x.data_ptr(), out.codes.data_ptr(), out.scales.data_ptr(), rows, cols,
                     axis, elem, BLOCK, _stream_ptr(x.device))
    return out


def dequantize(t: MXTensor, out=None):
    """MXTensor -> float32 [rows, cols] GPU tensor (mx_dequantize_axis)."""
    import torch
    _require_mx(t, "t", on_gpu=False)
    if out is not None:
        _require(out, torch.float32, "out", shape=(t.rows, t.cols), on_gpu=False)
    _require_mx(t, "t")
    if out is None:
        out = torch.empty((t.rows, t.cols), dtype=torch.float32, device=t.codes.device)
    _require(out, torch.float32, "out", shape=(t.rows, t.cols), device=t.codes.device)
    mx_dequantize_axis(t.codes.data_ptr(), t.scales.data_ptr(), out.data_ptr(), t.rows, t.cols,
                       t.axis, t.elem, BLOCK, _stream_ptr(out.device))
    return out


def fold_scale(t: MXTensor, j: int) -> MXTensor:
    """In place: t becomes 2^j * t through its scale bytes (mx_fold_scale)."""
    _require_mx(t, "t")
    mx_fold_scale(t.scales.data_ptr(), t.scales.numel(), j, _stream_ptr(t.scales.device))
    return t


def block_matmul(a: MXTensor, bt: MXTensor, out=None, accumulate: bool = False):
    """C = [C +] A . B with A [M, K] blocked along K, and B given either as
    B^T [N, K] blocked along its last axis or as B [K, N] blocked along axis 0
    (the same storage) (mx_block_matmul)."""
    import torch
    if a.axis != 1:
        raise ValueError("A must be blocked along its last axis (K)")
    bn, bk = (bt.rows, bt.cols) if bt.axis == 1 else (bt.cols, bt.rows)
    if a.cols != bk:
        raise ValueError(f"K mismatch: A has {a.cols}, B has {bk}")
    M, N, K = a.rows, bn, a.cols
    _require_mx(a, "a", on_gpu=False)
    _require_mx(bt, "bt", on_gpu=False)
    if out is not None:
        _require(out, torch.float32, "out", shape=(M, N), on_gpu=False)
    _require_mx(a, "a")
    _require_mx(bt, "bt", device=a.codes.device)
    if out is None:
        if accumulate:
            raise ValueError("accumulate=True needs an existing out tensor")
        out = torch.empty((M, N), dtype=torch.float32, device=a.codes.device)
    _require(out, torch.float32, "out", shape=(M, N), device=a.codes.device)
    mx_block_matmul(a.codes.data_ptr(), a.scales.data_ptr(), a.elem, bt.codes.data_ptr(),
                    bt.scales.data_ptr(), bt.elem, out.data_ptr(), M, N, K, BLOCK,
                    1 if accumulate else 0, _stream_ptr(out.device))
    return out


def block_matmul_f32b(a: MXTensor, b, out=None, accumulate: bool = False):
    """C = [C +] A . B with A [M, K] block-scaled along K and B an ordinary
    float32 [K, N] GPU tensor (mx_block_matmul_f32b)."""
    import torch
    if a.axis != 1:
        raise ValueError("A must be blocked along its last axis (K)")
    if not isinstance(b, torch.Tensor) or b.dim() != 2 or b.shape[0] != a.cols:
        raise ValueError(f"B must be a [K={a.cols}, N] tensor")
    M, K, N = a.rows, a.cols, b.shape[1]
    _require_mx(a, "a", on_gpu=False)
    if out is not None:
        _require(out, torch.float32, "out", shape=(M, N), on_gpu=False)
    _require_mx(a, "a")
    _require(b, torch.float32, "b", shape=(K, N), device=a.codes.device)
    if out is None:
        if accumulate:
            raise ValueError("accumulate=True needs an existing out tensor")
        out = torch.empty((M, N), dtype=torch.float32, device=b.device)
    _require(out, torch.float32, "out", shape=(M, N), device=a.codes.device)
    mx_block_matmul_f32b(a.codes.data_ptr(), a.scales.data_ptr(), a.elem, b.data_ptr(),
                         out.data_ptr(), M, N, K, BLOCK, 1 if accumulate else 0,
                         _stream_ptr(out.device))
    return out


def block_matmul_quantize_a(a, a_elem: int, bt: MXTensor, out=None, accumulate: bool = False):
    """C = [C +] Q(A) . B with A an ordinary float32 [M, K] GPU tensor,
    quantized along K to a_elem inside the product exactly as quantize()
    would, and B given as B^T [N, K] blocked along its last axis or as B
    [K, N] blocked along axis 0 (mx_block_matmul_quantize_a)."""
    import torch
    if not isinstance(a, torch.Tensor) or a.dim() != 2:
        raise ValueError("A must be a 2-D float32 tensor [M, K]")
    bn, bk = (bt.rows, bt.cols) if bt.axis == 1 else (bt.cols, bt.rows)
    M, K = a.shape
    if K != bk:
        raise ValueError(f"K mismatch: A has {K}, B has {bk}")
    N = bn
    _require(a, torch.float32, "a", shape=(M, K), on_gpu=False)
    _require_mx(bt, "bt", on_gpu=False)
    if out is not None:
        _require(out, torch.float32, "out", shape=(M, N), on_gpu=False)
    _require(a, torch.float32, "a", shape=(M, K))
    _require_mx(bt, "bt", device=a.device)
    if out is None:
        if accumulate:
            raise ValueError("accumulate=True needs an existing out tensor")
        out = torch.empty((M, N), dtype=torch.float32, device=a.device)
    _require(out, torch.float32, "out", shape=(M, N), device=a.device)
    mx_block_matmul_quantize_a(a.data_ptr(), a_elem, bt.codes.data_ptr(), bt.scales.data_ptr(),
                               bt.elem, out.data_ptr(), M, N, K, BLOCK, 1 if accumulate else 0,
                               _stream_ptr(out.device))
    return out
