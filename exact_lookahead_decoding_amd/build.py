"""Compile the HIP sources into the in-tree C-ABI library (gfx950 only).

    python -m exact_lookahead_decoding_amd.build

produces exact_lookahead_decoding_amd/_lib/liblookahead.so.  Every call
recompiles (translation units in parallel, then one link).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT_DIR = os.path.join(PKG, "_lib")
LIB = os.path.join(OUT_DIR, "liblookahead.so")
SOURCES = ["la_gemm.hip", "la_model.hip", "la_rows.hip", "la_attn.hip", "la_verify.hip", "la_state.hip",
           "la_api.hip"]
ARCH = "gfx950"
# per-file code generation options: the attention kernel post-processes its
# MFMA results with vector ALU code (softmax, rescaling), so its accumulators
# are kept in the architectural VGPRs (no AGPR <-> VGPR copies per chunk)
EXTRA = {"la_attn.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def flags():
    return ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def build(verbose: bool = False) -> str:
    os.makedirs(OUT_DIR, exist_ok=True)
    cc = hipcc()
    objs = []

    def compile_one(src):
        obj = os.path.join(OUT_DIR, src.replace(".hip", ".o"))
        cmd = [cc] + flags() + EXTRA.get(src, []) + ["-c", os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
        if verbose and r.stderr.strip():
            print(r.stderr)
        return obj

    workers = min(len(SOURCES), max(1, min(16, len(os.sched_getaffinity(0)))))
    with ThreadPoolExecutor(workers) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [cc, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    for o in objs:
        os.remove(o)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
