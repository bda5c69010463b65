"""Build libquoka.so (the HIP kernels and the C ABI) for gfx950 with hipcc, and
libquoka_peaks.so (the bench's peak probes).

Usage: python -m chunked_prefill_kv_amd.build   (or build() from Python)
Objects go to _build/ at the repository root; the library lands in
chunked_prefill_kv_amd/lib/libquoka.so, next to the binding that loads it.
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJ_DIR = os.path.join(ROOT, "_build", "quoka")
LIB_DIR = os.path.join(PKG, "lib")
LIB_PATH = os.path.join(LIB_DIR, "libquoka.so")
PEAKS_SRC = os.path.join(PKG, "peaks", "peaks.hip")
PEAKS_LIB = os.path.join(LIB_DIR, "libquoka_peaks.so")
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC or install ROCm)")


def compile_flags():
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
        f"-I{INCLUDE}", f"-I{CSRC}",
        # no packed-fp32 instructions (v_pk_{add,mul,fma}_f32) in device code
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wno-unused-command-line-argument",
    ]


# Per-source extra flags. The scorer's max over the kept rows reads MFMA
# results, and in IEEE mode every fmaxf of such a value is preceded by a
# NaN-quieting v_max (16 per 16-row block, in the chain the next block's
# products wait behind); its inputs are finite by contract, so it is built in
# non-IEEE mode (rounding of adds and products is unchanged). Scorer on the
# long layer's data: 81.4 -> 77.8 us; llama8b 21.6 -> 21.0 us.
FILE_FLAGS = {"scorer.hip": ["-fno-honor-nans", "-mno-amdgpu-ieee"]}


def _run(cmd):
    p = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the packed-fp32 feature; that warning is noise
    err = "\n".join(l for l in p.stderr.splitlines() if "packed-fp32-ops" not in l)
    if p.returncode != 0:
        raise RuntimeError(f"command failed ({p.returncode}): {' '.join(cmd)}\n{err}")
    return err


def build(verbose: bool = False, jobs: int | None = None) -> str:
    """Compile every csrc/*.hip for gfx950 and link libquoka.so. Returns its path."""
    cc = hipcc()
    os.makedirs(OBJ_DIR, exist_ok=True)
    os.makedirs(LIB_DIR, exist_ok=True)
    srcs = sorted(f for f in os.listdir(CSRC) if f.endswith(".hip"))
    flags = compile_flags()

    def one(src):
        obj = os.path.join(OBJ_DIR, src[:-4] + ".o")
        cmd = [cc, *flags, *FILE_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        msg = _run(cmd)
        if verbose and msg.strip():
            print(msg, flush=True)
        return obj

    jobs = jobs or min(len(srcs), max(1, min(8, os.cpu_count() or 1)))
    with concurrent.futures.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(one, srcs))
    tmp = LIB_PATH + ".tmp"
    _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, LIB_PATH)
    # the peak probes the bench confirms the roofline denominators with
    tmp = PEAKS_LIB + ".tmp"
    _run([cc, *flags, "-shared", PEAKS_SRC, "-o", tmp])
    os.replace(tmp, PEAKS_LIB)
    if verbose:
        print(f"built {LIB_PATH} and {PEAKS_LIB}", flush=True)
    return LIB_PATH


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
