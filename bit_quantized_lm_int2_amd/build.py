"""Build libi2h.so (the HIP kernels and the C ABI) in-tree for gfx950.

    python -m bit_quantized_lm_int2_amd.build [-v]

Every call compiles from scratch. The library lands next to this file; the Python binding
loads it from there.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libi2h.so")
ARCH = os.environ.get("I2H_OFFLOAD_ARCH", "gfx950")

SOURCES = ["pack.hip", "coarse.hip", "coarse_tile.hip", "select.hip", "select_rerank.hip", "rerank.hip", "head.hip",
           "logits.hip", "coarse4.hip", "select_tokens.hip", "variant.hip"]

COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    "-Wall", "-Wno-unused-function",
    # packed fp32 instructions stay out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{INCLUDE}", f"-I{CSRC}",
]
# The packer must be bit-exact against an eager fp32 evaluation: no contraction into FMA and
# correctly rounded division. Its inputs are finite, so min / max need no NaN quieting.
EXTRA = {"pack.hip": ["-ffp-contract=off", "-fhip-fp32-correctly-rounded-divide-sqrt", "-fno-honor-nans"],
         "variant.hip": ["-ffp-contract=off", "-fhip-fp32-correctly-rounded-divide-sqrt", "-fno-honor-nans"]}


def _hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found; the int2 head library cannot be built")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in p.stdout.splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in l)
    if p.returncode != 0:
        raise RuntimeError(f"command failed ({p.returncode}): {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out, flush=True)


def build(verbose: bool = False) -> str:
    hipcc = _hipcc()
    tmp = tempfile.mkdtemp(prefix="i2h_build_")
    try:
        objs = []
        cmds = []
        for src in SOURCES:
            obj = os.path.join(tmp, src.replace(".hip", ".o"))
            objs.append(obj)
            cmds.append([hipcc, *COMMON, *EXTRA.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj])
        with cf.ThreadPoolExecutor(min(8, len(cmds))) as ex:
            list(ex.map(lambda c: _run(c, verbose), cmds))
        out_tmp = LIB + ".tmp"
        _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", out_tmp, *objs], verbose)
        os.replace(out_tmp, LIB)
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv[1:]))
