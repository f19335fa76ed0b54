"""Build the gfx950 HIP library ``lib/libmoe_mi355x.so`` in-tree with hipcc.

    python -m sparse_mixture_experts_10_amd.build

Cross-compiles without a GPU.  Always rebuilds (each source is one hipcc job,
run in parallel); the shared object is written next to this file.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
ROOT = os.path.dirname(PKG)
INCLUDE = os.path.join(ROOT, "include")
OUT_DIR = os.path.join(PKG, "lib")
LIB_NAME = "libmoe_mi355x.so"
LIB_PATH = os.path.join(OUT_DIR, LIB_NAME)
ARCH = "gfx950"

SOURCES = ["router.hip", "dispatch.hip", "grouped_gemm.hip", "gemm_bf16_v2.hip", "gemm_bf16_persist.hip", "combine.hip",
           "stats.hip", "balance.hip", "calib.hip", "noalloc.hip", "abi.cpp"]

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    # keep the compiler from forming packed-fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def _hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build the library)")


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    msgs = [ln for ln in r.stdout.splitlines() if "packed-fp32-ops" not in ln]
    return r.returncode, "\n".join(msgs)


def build(verbose: bool = False) -> str:
    hipcc = _hipcc()
    obj_dir = os.path.join(ROOT, "_build", "obj")
    os.makedirs(obj_dir, exist_ok=True)
    os.makedirs(OUT_DIR, exist_ok=True)
    jobs = []
    for src in SOURCES:
        obj = os.path.join(obj_dir, src + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        jobs.append((obj, [hipcc] + FLAGS + lang + ["-c", os.path.join(CSRC, src), "-o", obj]))
    with ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        results = list(ex.map(lambda j: _run(j[1]), jobs))
    for (obj, cmd), (rc, out) in zip(jobs, results):
        if out.strip() and (verbose or rc):
            print(out, file=sys.stderr)
        if rc:
            raise RuntimeError(f"hipcc failed ({rc}): {' '.join(cmd)}")
    tmp = LIB_PATH + ".tmp"
    rc, out = _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + [j[0] for j in jobs])
    if rc:
        print(out, file=sys.stderr)
        raise RuntimeError("link failed")
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
