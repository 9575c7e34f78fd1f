"""Build liblstm_amd.so in-tree with hipcc for gfx950."""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "liblstm_amd.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

SOURCES = ["lstm_api.cpp", "kernels.hip", "rec_f32.hip", "rec_bf16.hip", "rec_bf16_wide.hip", "backward.hip",
           "pack.hip", "noalloc.hip", "rec_wave.hip", "rec_xcd.hip",
           "rec_res.hip"]
# Packed-fp32 VALU ops stay off: the device code uses plain fp32 arithmetic.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
# Per-source flags.  rec_res.hip keeps W_hh (up to 256 registers a wave) beside
# its accumulators: with the accumulators in ordinary VGPRs the allocator puts
# W_hh in the accumulation registers instead of spilling to scratch.
SOURCE_FLAGS = {"rec_res.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _compile(src: str, verbose: bool) -> str:
    path = os.path.join(CSRC, src)
    obj = os.path.join(CSRC, os.path.splitext(src)[0] + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
           "-I", os.path.join(ROOT, "include"), *DEVICE_FLAGS, *SOURCE_FLAGS.get(src, []), *lang, "-c", path, "-o", obj]
    if verbose:
        print(" ".join(cmd), file=sys.stderr)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}")
    return obj


def build(verbose: bool = False) -> str:
    # the translation units compile independently, one process each
    from concurrent.futures import ThreadPoolExecutor
    jobs = max(1, min(len(SOURCES), int(os.environ.get("MAX_JOBS", os.cpu_count() or 1))))
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda src: _compile(src, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    subprocess.run(cmd, check=True, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
    os.replace(tmp, LIB)
    for o in objs:
        os.remove(o)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
