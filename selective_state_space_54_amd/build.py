"""Build the mssm HIP library (libmssm.so) for gfx950 with hipcc, in-tree."""
from __future__ import annotations

import concurrent.futures
import glob
import os
import subprocess

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_PATH = os.path.join(PKG_DIR, "libmssm.so")
# issue-rate and bandwidth probes behind the roofline figures (bench.py --probe-rates)
PROBE_SRC = os.path.join(PKG_DIR, "probe", "issue_rates.hip")
PROBE_LIB_PATH = os.path.join(PKG_DIR, "libmssm_probe.so")
OBJ_DIR = os.path.join(PKG_DIR, "_build")

# -packed-fp32-ops: no v_pk_{add,mul,fma}_f32 in the generated code.
HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def _jobs() -> int:
    try:
        n = int(os.environ.get("MAX_JOBS", "0"))
    except ValueError:
        n = 0
    return max(1, min(n or (os.cpu_count() or 1), 16))


def build(verbose: bool = False) -> str:
    """Compile every HIP source (in parallel, one object each) and link
    libmssm.so next to this file; return its path."""
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    os.makedirs(OBJ_DIR, exist_ok=True)

    def compile_one(src):
        obj = os.path.join(OBJ_DIR, os.path.basename(src) + ".o")
        cmd = [hipcc, *HIPCC_FLAGS, "-I", INCLUDE, "-I", CSRC, "-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src} ({r.returncode}):\n{r.stderr[-8000:]}")
        return obj

    with concurrent.futures.ThreadPoolExecutor(max_workers=_jobs()) as pool:
        objs = list(pool.map(compile_one, sources()))
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp,
           "-L/opt/rocm/lib", "-lrocblas", "-Wl,-rpath,/opt/rocm/lib"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed ({r.returncode}):\n{r.stderr[-8000:]}")
    os.replace(tmp, LIB_PATH)
    build_probe(hipcc, verbose)
    return LIB_PATH


def build_probe(hipcc: str, verbose: bool = False) -> str:
    """The measurement probes, a library of their own (not part of libmssm)."""
    tmp = PROBE_LIB_PATH + ".tmp"
    cmd = [hipcc, *HIPCC_FLAGS, "-shared", PROBE_SRC, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {PROBE_SRC} ({r.returncode}):\n{r.stderr[-8000:]}")
    os.replace(tmp, PROBE_LIB_PATH)
    return PROBE_LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
