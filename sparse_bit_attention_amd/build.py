"""Build libsagesla.so (the attention library) and libslapeak.so (the
matrix-core peak measurement kernels the benchmark quotes fractions against)
for gfx950 in-tree with hipcc.

    python -m sparse_bit_attention_amd.build
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "libsagesla.so")
PEAK_OUT = os.path.join(PKG, "libslapeak.so")
OBJ = os.path.join(PKG, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

SOURCES = ["k_quant.hip", "k_select.hip", "k_linear.hip", "k_attn.hip", "k_w8a8.hip", "k_bwd.hip",
           "sla_api.cpp"]
PEAK_SOURCES = ["peak.hip"]

FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # float32 results that decide integers must follow the written order
    "-ffp-contract=off",
    # no packed-fp32 VALU instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
    "-I", CSRC,
    "-Wno-unused-result",
]


# Per-file extra hipcc flags.  peak.hip: MFMA accumulators in ordinary
# VGPRs (in AGPRs the compiler rotates the independent chains through
# register copies every iteration, which the measurement must not contain).
EXTRA = {"peak.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _compile(src: str) -> str:
    obj = os.path.join(OBJ, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, *EXTRA.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd[-4:-4] = ["-x", "hip"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def _link(objs, out: str) -> None:
    tmp = out + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)


def build(verbose: bool = False) -> str:
    os.makedirs(OBJ, exist_ok=True)
    with ThreadPoolExecutor(len(SOURCES) + len(PEAK_SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES + PEAK_SOURCES))
    _link(objs[:len(SOURCES)], OUT)
    _link(objs[len(SOURCES):], PEAK_OUT)
    if verbose:
        print("built", OUT, "and", PEAK_OUT)
    return OUT


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
