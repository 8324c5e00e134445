"""Helpers for the GPU parity tests: move NumPy arrays through the C ABI."""
import numpy as np
import torch

from bit_gemm_mx_amd import binding as B


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    return t.cpu().numpy()


def gpu_quantize(x: np.ndarray, elem: int):
    t = B.quantize(dev(x.astype(np.float32)), elem)
    return host(t.codes), host(t.scales)


def gpu_dequantize(codes: np.ndarray, scales: np.ndarray, elem: int, cols: int) -> np.ndarray:
    rows = scales.shape[0]
    t = B.MXTensor(dev(codes), dev(scales), rows, cols, elem)
    return host(B.dequantize(t))


def gpu_matmul(ac, asc, ae, bc, bsc, be, M, N, K, c_in=None, accumulate=False):
    a = B.MXTensor(dev(ac), dev(asc), M, K, ae)
    b = B.MXTensor(dev(bc), dev(bsc), N, K, be)
    out = dev(c_in.astype(np.float32)) if c_in is not None else None
    return host(B.block_matmul(a, b, out=out, accumulate=accumulate))


def assert_bits_equal(got: np.ndarray, want: np.ndarray, what: str = ""):
    g = got.view(np.uint32) if got.dtype == np.float32 else got
    w = want.view(np.uint32) if want.dtype == np.float32 else want
    if not np.array_equal(g, w):
        bad = np.argwhere(g != w)
        i = tuple(bad[0])
        raise AssertionError(f"{what}: {len(bad)} mismatches, first at {i}: got {g[i]!r} want {w[i]!r}")


def assert_matmul_close(got: np.ndarray, want: np.ndarray, mag: np.ndarray, rel: float = 1e-5):
    """|got - want| <= rel * sum_k |a_k b_k| (+|C_in|) per element; NaN where
    the oracle has NaN; exact (signed or unsigned) zero where the bound is 0."""
    got = got.astype(np.float64)
    want_nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), want_nan), "NaN positions differ"
    ok = ~want_nan
    err = np.abs(got[ok] - want[ok].astype(np.float64))
    bound = rel * mag[ok]
    worst = np.max(err / np.where(bound > 0, bound, 1.0)) if err.size else 0.0
    assert np.all(err <= bound), f"tolerance exceeded: worst err/bound = {worst:.3g}"
    return worst


def mfma_group_bound(a_dq: np.ndarray, b_dq: np.ndarray, rows, cols, group: int = 8) -> np.ndarray:
    """Extra error allowed by the scaled-MFMA arithmetic measured on gfx950,
    at the output elements (rows[i], cols[i]).

    Each aligned group of `group` consecutive K products is summed in fixed
    point aligned to the group's largest product, dropping bits below
    2^(E-14) (E = floor(log2 max |p|) in the group); the groups are then added
    in fp32.  Per group the error is < group * 2^(E-14) <= 2^(E-10) for
    group = 8.  Returns sum over groups of 2^(E_g - 10) per element."""
    K = a_dq.shape[1]
    out = np.zeros(len(rows))
    for s0 in range(0, len(rows), 256):
        r, c = rows[s0:s0 + 256], cols[s0:s0 + 256]
        p = np.nan_to_num(np.abs(a_dq[r] * b_dq[c]))
        gmax = p.reshape(len(r), K // group, group).max(axis=-1)
        with np.errstate(divide="ignore"):
            e = np.floor(np.log2(gmax))
        out[s0:s0 + 256] = np.where(gmax > 0, np.exp2(e - 10), 0.0).sum(axis=-1)
    return out
