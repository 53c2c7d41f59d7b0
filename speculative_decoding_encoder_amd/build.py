"""Build libwf.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

Run ``python -m speculative_decoding_encoder_amd.build``; the library lands
next to this file, where the Python binding looks for it.
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libwf.so")
SOURCES = ["engine.hip", "k_gemm.hip", "k_gemm_rk_attn.hip", "k_gemm_rk_mlp.hip",
           "k_gemm_rk_head.hip", "k_attn.hip", "k_misc.hip", "k_sample.hip", "k_draft.hip", "k_pass.hip", "encoder.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(l for l in (res.stderr or "").splitlines() if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{errs}")
    if verbose and errs.strip():
        print(errs, file=sys.stderr)


def build(verbose: bool = False, jobs: int = 0) -> str:
    """Compile every source to an object (in parallel), then link."""
    jobs = jobs or min(len(SOURCES), max(1, os.cpu_count() or 1), 16)
    inc = ["-I", os.path.join(HERE, "..", "include")]
    with tempfile.TemporaryDirectory(prefix="wf_build_") as tmpd:
        objs = [os.path.join(tmpd, os.path.splitext(s)[0] + ".o") for s in SOURCES]
        cmds = [[hipcc()] + HIPCC_FLAGS + inc + ["-c", os.path.join(CSRC, s), "-o", o]
                for s, o in zip(SOURCES, objs)]
        with concurrent.futures.ThreadPoolExecutor(jobs) as ex:
            for f in [ex.submit(_run, c, verbose) for c in cmds]:
                f.result()
        tmp = LIB + ".tmp"
        _run([hipcc()] + HIPCC_FLAGS + ["-shared"] + objs + ["-o", tmp], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
