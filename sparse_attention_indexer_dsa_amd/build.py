"""Build libdsa_index.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

Usage: ``python -m sparse_attention_indexer_dsa_amd.build`` (or ``build()`` from Python).
Objects go to ``_build/`` at the repository root; the shared library is written next to
this file so the Python binding finds it in-tree.
"""

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "libdsa_index.so")
BUILD_DIR = os.path.join(ROOT, "_build")
SOURCES = ["api.cpp", "preprocess.hip", "kpool.hip", "score.hip", "topk.hip", "softmax.hip", "attention.hip", "peak.hip",
           "noalloc.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17",
    # one rounding per fp32 operation unless a fused multiply-add is written explicitly
    "-ffp-contract=off",
    # correctly rounded fp32 division and square root, denormals kept
    "-fhip-fp32-correctly-rounded-divide-sqrt", "-fno-gpu-flush-denormals-to-zero",
    # no packed fp32 arithmetic
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
    "-Wall", "-Wno-unused-function",
]


def _compile(src):
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC] + FLAGS + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in (r.stderr or "").splitlines()
                    if "packed-fp32-ops" not in l)   # the host pass does not know the feature
    return obj, r.returncode, " ".join(cmd), err


def build(verbose=False):
    os.makedirs(BUILD_DIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 4)) as ex:
        results = list(ex.map(_compile, SOURCES))
    objs = []
    for obj, rc, cmd, err in results:
        if verbose or rc != 0:
            print(cmd)
            if err.strip():
                print(err)
        if rc != 0:
            raise RuntimeError(f"hipcc failed for {obj}")
        objs.append(obj)
    tmp = OUT + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        print(" ".join(cmd))
        print(r.stderr)
        raise RuntimeError("link failed")
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
