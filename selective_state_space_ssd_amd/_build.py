"""Build ``libssd.so`` (the HIP kernels and the C ABI) for gfx950 with hipcc.

The library is built in-tree next to this file.  Each translation unit is
compiled separately (in parallel), then linked into one shared object.
"""
from __future__ import annotations

import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB_PATH = os.path.join(PKG, "libssd.so")
# measured peaks (streaming copy, matrix-core loops) for the benchmark's
# roofline lines: a library of its own, not part of the scan's
PEAKS_LIB_PATH = os.path.join(PKG, "libssd_peaks.so")
PEAKS_SOURCES = ["ssd_peaks.hip"]
OBJ_DIR = os.path.join(ROOT, "_build")
SOURCES = ["ssd_api.hip", "ssd_dt_cumsum.hip", "ssd_chunk_state.hip", "ssd_state_passing.hip",
           "ssd_chunk_scan.hip", "ssd_bf16.hip", "ssd_fused_bf16.hip",
           "ssd_fused_group_bf16.hip", "ssd_chain_bf16.hip", "ssd_decode.hip", "ssd_block.hip",
           "ssd_backward.hip"]
ARCH = "gfx950"
CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # no packed fp32 (v_pk_*_f32) instructions anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build the SSD library)")


def build(verbose: bool = False) -> str:
    """Compile every source and link ``libssd.so`` and ``libssd_peaks.so``;
    returns the path of ``libssd.so``."""
    cc = hipcc()
    os.makedirs(OBJ_DIR, exist_ok=True)

    def compile_one(src):
        obj = os.path.join(OBJ_DIR, os.path.splitext(src)[0] + ".o")
        cmd = [cc, *CFLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
        if verbose and r.stderr.strip():
            print(r.stderr)
        return obj

    every = SOURCES + PEAKS_SOURCES
    with ThreadPoolExecutor(max_workers=min(len(every), os.cpu_count() or 1)) as ex:
        objs = dict(zip(every, ex.map(compile_one, every)))
    for path, srcs in ((LIB_PATH, SOURCES), (PEAKS_LIB_PATH, PEAKS_SOURCES)):
        tmp = path + ".tmp"
        cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *[objs[s] for s in srcs],
               "-o", tmp]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
        os.replace(tmp, path)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
