"""Build libgqla.so (hand-written HIP for gfx950) in-tree with hipcc.

Usage: python -m latent_kv_cache_amd.build  [--jobs N]

Every source under csrc/ is compiled for gfx950 with packed-fp32 instruction
selection disabled, then linked into latent_kv_cache_amd/libgqla.so.  Code
objects are emitted as version 5 so that the HIP runtime bundled with
PyTorch-ROCm (which the library shares when torch is imported first; both carry
the SONAME libamdhip64.so.7) loads them.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libgqla.so")
ARCH = "gfx950"

SOURCES = ["api.hip", "decode_gqa.hip", "decode_absorb.hip", "expand_bf16.hip", "f32_path.hip", "f32_mfma.hip", "combine.hip", "append.hip", "probe.hip", "decode_sparse.hip"]

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-mcode-object-version=5",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    f"-I{os.path.join(ROOT, 'include')}",
]

# Per-source extras.  The decode kernels keep their MFMA accumulators in ordinary
# VGPRs: they rescale them with VALU, and AGPR accumulators would be copied to VGPRs
# and back every tile.
EXTRA_FLAGS = {
    "decode_gqa.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    "decode_absorb.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libgqla)")


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *HIPCC_FLAGS, *EXTRA_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{res.stdout}\n{res.stderr}")
    return obj


def build(jobs: int = 0, verbose: bool = False) -> str:
    """Compile every source and link libgqla.so; returns the library path."""
    os.makedirs(BUILD, exist_ok=True)
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 1, 8)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--jobs", type=int, default=0)
    args = ap.parse_args(argv)
    build(args.jobs, verbose=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
