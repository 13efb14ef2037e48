"""Build libfgemm.so for gfx950 with hipcc (runs on a CPU-only machine too).

The GEMM kernel template is instantiated once per (MFMA dtype, A layout, B layout)
from gemm_inst.hip with -D switches, so the eight instantiation units and the other
sources compile in parallel.  Objects go to _build/ at the repository root and the
library lands next to this file.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libfgemm.so")

HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I" + INCLUDE, "-I" + CSRC,
         # keep the compiler away from packed fp32 instructions on this device
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _units():
    units = []
    for dt in (0, 1):
        for ak in (0, 1):
            for bk in (0, 1):
                units.append((os.path.join(CSRC, "gemm_inst.hip"), f"gemm_inst_{dt}_{ak}{bk}.o",
                              [f"-DFG_DT={dt}", f"-DFG_AK={ak}", f"-DFG_BK={bk}"]))
    for src in ("gemm_f8.hip", "strassen_adds.hip", "noalloc.hip", "read_probe.hip", "quantize_mx.hip",
                "fgemm_api.cpp", "model.cpp"):
        units.append((os.path.join(CSRC, src), src.rsplit(".", 1)[0] + ".o", []))
    return units


def _compile(unit, extra=(), build_dir=BUILD):
    src, obj, defs = unit
    out = os.path.join(build_dir, obj)
    cmd = [HIPCC, *FLAGS, *extra, *defs, "-c", src, "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return out


def build(jobs: int | None = None, verbose: bool = True, extra=(), out: str = LIB,
          build_dir: str = BUILD) -> str:
    """Compile and link; `extra` adds compiler switches, `out` names the library."""
    os.makedirs(build_dir, exist_ok=True)
    units = _units()
    jobs = jobs or min(len(units), max(1, len(os.sched_getaffinity(0))))
    if verbose:
        print(f"[fgemm build] {len(units)} units, {jobs} jobs, {HIPCC}", flush=True)
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda u: _compile(u, extra, build_dir), units))
    tmp = out + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)
    if verbose:
        print(f"[fgemm build] wrote {out}", flush=True)
    return out


if __name__ == "__main__":
    build(int(sys.argv[1]) if len(sys.argv) > 1 else None)
