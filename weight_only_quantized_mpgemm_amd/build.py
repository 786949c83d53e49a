"""Builds libmpgemm.so (the gfx950 HIP kernels and the C ABI) in-tree with hipcc.

    python -m weight_only_quantized_mpgemm_amd.build

Every HIP source is compiled for gfx950 only, with packed-fp32 instruction selection
switched off (those forms are avoided on this hardware) and floating-point contraction off
(the dequantization relies on an exact add followed by a single rounding multiply).  The
compiler's per-kernel resource report is checked: a kernel that spills to scratch memory
fails the build (a spill in these register-resident pipelines costs far more than it
saves, and nothing else would show it).
"""
from __future__ import annotations

import concurrent.futures
import os
import re
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmpgemm.so")
SOURCES = ["api.hip", "pack.hip", "gemm_decode.hip", "gemm_prefill.hip", "gemm_prefill_ring.hip",
           "gemm_prefill_x32.hip"]
HEADERS = ["device.hpp", "kernels.hpp"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = ["-O3", "-std=c++20", "-fPIC", f"--offload-arch={ARCH}", "-ffp-contract=off",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(ROOT, "include"), "-Wall", "-Wno-unused-function"]


def scratch_users(report: str) -> list[tuple[str, int]]:
    """(kernel, bytes per lane) for every kernel the resource report shows using scratch."""
    out, name = [], None
    for line in report.splitlines():
        m = re.search(r"remark: Function Name: (\S+)", line)
        if m:
            name = m.group(1)
        m = re.search(r"remark:\s+ScratchSize \[bytes/lane\]: (\d+)", line)
        if m and int(m.group(1)) > 0:
            out.append((name, int(m.group(1))))
    return out


def _compile(src: str, extra: list[str]) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, "-Rpass-analysis=kernel-resource-usage", *extra, "-c",
           os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{res.stderr}")
    spills = scratch_users(res.stderr)
    if spills:
        raise RuntimeError(f"{src}: kernels use scratch memory (register spills): {spills}")
    return obj


def build(verbose: bool = False, extra: list[str] | None = None) -> str:
    """Compiles every source (always; no staleness shortcuts) and links libmpgemm.so."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    extra = list(extra or [])
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(lambda s: _compile(s, extra), SOURCES))
    tmp = LIB + f".tmp{os.getpid()}"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True, extra=sys.argv[1:])
