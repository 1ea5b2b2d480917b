"""Build libsfnn.so (HIP, gfx950) in-tree with hipcc.

Usage: python -m activation_sparse_gemv_amd.build  (or call build()).
Always recompiles; objects go to activation_sparse_gemv_amd/_build/.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libsfnn.so")
SOURCES = ["api.hip", "k_predict.hip", "k_ffn.hip", "k_ffn_f32.hip", "k_ffn_f16.hip", "k_ffn_i4.hip",
           "k_lookahead.hip", "k_la_f32.hip", "k_la_f16.hip", "k_la_i4.hip", "k_misc.hip",
           "k_mfma.hip", "k_mfma_i4.hip", "k_pred_mfma.hip", "k_isg.hip", "k_heads.hip"]
ARCH = "gfx950"

FLAGS = [
    "-O3", f"--offload-arch={ARCH}", "-fPIC", "-std=c++17",
    "-fno-gpu-rdc", "-mcode-object-version=5",
    # no packed fp32 arithmetic in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError("command failed: " + " ".join(cmd) + "\n" + r.stdout)
    return r.stdout


def build(verbose: bool = False) -> str:
    os.makedirs(OBJ, exist_ok=True)
    cc = hipcc()
    jobs = []
    for src in SOURCES:
        obj = os.path.join(OBJ, src.replace(".hip", ".o"))
        jobs.append(([cc, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj], obj))
    with cf.ThreadPoolExecutor(min(8, len(jobs))) as ex:
        outs = list(ex.map(lambda j: _run(j[0]), jobs))
    if verbose:
        for o in outs:
            if o.strip():
                print(o)
    tmp = LIB + ".tmp"
    _run([cc, "-shared", f"--offload-arch={ARCH}", "-fno-gpu-rdc", "-o", tmp, *[j[1] for j in jobs]])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
