"""Every entry point captured in a HIP graph (torch.cuda.graph) replays to the
same bits as the eager calls.

The kernels allocate nothing, record no memset and keep no state between
calls, so a captured sequence must reproduce the eager results on every
replay.  The graph's outputs are poisoned with NaN before each replay (so a
replay that skipped a kernel would show), eager work runs between replays,
and every replay is compared bit for bit with the eager results.
"""
import numpy as np
import pytest
import torch

from bit_gemm_mx_amd import binding as B
from bit_gemm_mx_amd import workloads as W

pytestmark = pytest.mark.gpu


def bits(t: torch.Tensor) -> np.ndarray:
    a = t.detach().cpu().numpy()
    return a.view(np.uint32) if a.dtype == np.float32 else a


def test_graph_replays_match_eager():
    rng = np.random.default_rng(2024)
    x = torch.from_numpy(W.normal_with_outliers(rng, (512, 2048), 1.0, 0.01, 30.0)).cuda()
    w = torch.from_numpy(W.normal_with_outliers(rng, (512, 2048), 0.02, 0.001, 50.0)).cuda()
    bf = torch.from_numpy(rng.standard_normal((2048, 48), dtype=np.float32)).cuda()
    xs = torch.from_numpy(W.normal_with_outliers(rng, (2048, 256), 0.02, 0.001, 50.0)).cuda()
    bsq = torch.from_numpy(rng.standard_normal((256, 1024), dtype=np.float32)).cuda()
    x16 = x[:16].contiguous()

    def run(o):
        B.quantize(x, B.MX_E4M3, out=o["xa"])
        B.quantize(w, B.MX_E2M1, out=o["wq"])
        B.quantize(x16, B.MX_E2M1, out=o["x16"])
        B.dequantize(o["wq"], out=o["wd"])
        B.block_matmul(o["xa"], o["wq"], out=o["c_tiled"])            # 512 x 512 x 2048
        B.block_matmul(o["x16"], o["wq"], out=o["c_skinny"])          # 16 x 512 x 2048
        B.block_matmul_f32b(o["wq"], bf, out=o["c_f32b"])             # 512 x 48 x 2048
        B.quantize(xs, B.MX_E2M1, out=o["xs"])
        B.block_matmul_f32b(o["xs"], bsq, out=o["c_f32b_sq"])         # 2048 x 1024 x 256 (bf16 cores)
        B.block_matmul_quantize_a(x, B.MX_E4M3, o["wq"], out=o["c_fused"])  # 512 x 512 x 2048
        B.quantize(w, B.MX_E2M1, out=o["w0"], axis=0)
        B.dequantize(o["w0"], out=o["w0d"])
        B.fold_scale(o["w0"], 3)
        B.fold_scale(o["w0"], -3)

    def outputs():
        return {
            "xa": B.empty_mx(512, 2048, B.MX_E4M3, x.device),
            "wq": B.empty_mx(512, 2048, B.MX_E2M1, x.device),
            "x16": B.empty_mx(16, 2048, B.MX_E2M1, x.device),
            "wd": torch.empty(512, 2048, device="cuda"),
            "c_tiled": torch.empty(512, 512, device="cuda"),
            "c_skinny": torch.empty(16, 512, device="cuda"),
            "c_f32b": torch.empty(512, 48, device="cuda"),
            "xs": B.empty_mx(2048, 256, B.MX_E2M1, x.device),
            "c_f32b_sq": torch.empty(2048, 1024, device="cuda"),
            "c_fused": torch.empty(512, 512, device="cuda"),
            "w0": B.empty_mx(512, 2048, B.MX_E2M1, x.device, axis=0),
            "w0d": torch.empty(512, 2048, device="cuda"),
        }

    def flat(o):
        out = {}
        for k, v in o.items():
            if isinstance(v, B.MXTensor):
                out[k + ".codes"], out[k + ".scales"] = v.codes, v.scales
            else:
                out[k] = v
        return out

    eager = outputs()
    run(eager)
    torch.cuda.synchronize()
    want = {k: bits(v) for k, v in flat(eager).items()}

    graph_out = outputs()
    run(graph_out)  # warm up outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run(graph_out)
    for replay in range(3):
        for t in flat(graph_out).values():
            if t.dtype == torch.float32:
                t.fill_(float("nan"))
            else:
                t.fill_(0xA5)
        g.replay()
        run(eager)  # eager work on the same stream between replays
        torch.cuda.synchronize()
        for k, v in flat(graph_out).items():
            np.testing.assert_array_equal(bits(v), want[k], err_msg=f"replay {replay}: {k}")
