"""Build libqkmla.so (the C-ABI library with every HIP kernel) for gfx950.

Usage: python -m mla_latent_decode_amd.build
The library is written next to this file; objects and the device assembly go
to ./_build/.
"""
from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libqkmla.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["api.hip", "absorb_append.hip", "qprep.hip", "decode_mfma.hip",
           "decode_generic.hip", "merge_outproj.hip", "train.hip",
           "train_mfma.hip", "gemm_mfma.hip"]

# -packed-fp32-ops: never emit packed fp32 VALU ops (v_pk_*_f32).
CFLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, src.replace(".hip", ".o"))
    # -save-temps keeps the device assembly (*-gfx950.s) the code object is
    # assembled from, for the static ISA checks and the CPU emulator tests;
    # the code it produces is the same as without it.
    cmd = [HIPCC, "-save-temps=obj", *CFLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True, cwd=BUILD)
    errs = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                     if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{errs}")
    if errs.strip():
        print(errs, file=sys.stderr)
    return obj


def build() -> str:
    os.makedirs(BUILD, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
