"""Build libmx.so in-tree with hipcc for gfx950.

    python -m bit_gemm_mx_amd.build

Every HIP source is compiled to an object under ``_build/`` (in parallel),
then linked into ``bit_gemm_mx_amd/libmx.so``.  Packed-FP32 instruction
selection is disabled for all device code.
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import re
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmx.so")
SOURCES = ["libmx.cpp", "quantize.hip", "dequantize.hip", "codec_axis0.hip",
           "scale_ops.hip", "block_matmul.hip", "block_matmul_f32b.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libmx)")


def common_flags() -> list[str]:
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
        "-Wall", "-Wno-unused-function",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", os.path.join(ROOT, "include"),
    ]


def _scratch_kernels(remarks: str) -> list[str]:
    """Kernels whose resource-usage remarks report private (scratch) memory."""
    bad, name = [], None
    for line in remarks.splitlines():
        m = re.search(r"remark:\s+Function Name: (\S+)", line)
        if m:
            name = m.group(1)
            continue
        m = re.search(r"remark:\s+ScratchSize \[bytes/lane\]: (\d+)", line)
        if m and name and int(m.group(1)) > 0:
            bad.append(f"{name} ({m.group(1)} bytes/lane)")
    return bad


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *common_flags(), "-Rpass-analysis=kernel-resource-usage", "-x", "hip", "-c",
           os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    # No kernel may spill: the tiled matmul counts its outstanding loads by
    # hand (s_waitcnt vmcnt), and scratch loads and stores would join that
    # count and release LDS reads before their data has landed.
    bad = _scratch_kernels(r.stderr)
    if bad:
        os.remove(obj)
        raise RuntimeError(f"{src}: kernels use scratch memory (register spills): {bad}")
    return obj


def build(verbose: bool = False) -> str:
    """Compile every source and link libmx.so; returns the library path."""
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    # --no-undefined: a kernel whose host launch stub the compiler dropped
    # must fail the build, not the first dlopen.
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-Wl,--no-undefined", *objs,
           "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
