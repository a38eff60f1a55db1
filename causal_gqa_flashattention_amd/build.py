"""Build the HIP library in-tree: csrc/*.hip + csrc/*.cpp -> libcgqa_fa.so (gfx950)."""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG_DIR, "csrc")
LIB_NAME = "libcgqa_fa.so"
PROBE_LIB_NAME = "libcgqa_probe.so"  # matrix-core throughput probe (csrc/probe), not the attention ABI
ARCH = "gfx950"

# Packed fp32 VALU forms are switched off; the compiler would otherwise form
# them from ordinary float code.
HIP_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result",
]


def _hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


# Per-file scheduler choice.  The backward kernels run two 256-register
# waves per SIMD; LLVM's default scheduler keeps enough LDS reads in flight
# there to spill, and every spill reload then waits on the vector-memory
# counter behind the in-flight tile loads.  The occupancy-first iterative
# strategy schedules them without spills.
FILE_FLAGS = {
    "fa_bwd.hip": ["-mllvm", "-amdgpu-sched-strategy=iterative-maxocc"],
}


def _compile(src: str, obj: str) -> None:
    cmd = [_hipcc(), *HIP_FLAGS, *FILE_FLAGS.get(os.path.basename(src), []), "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")


def build_library(verbose: bool = True) -> str:
    """Compile every source for gfx950 and link the shared library; returns its path."""
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))
    bdir = os.path.join(PKG_DIR, "_build")
    os.makedirs(bdir, exist_ok=True)
    objs = [os.path.join(bdir, os.path.basename(s) + ".o") for s in srcs]
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        list(ex.map(_compile, srcs, objs))
    out = os.path.join(PKG_DIR, LIB_NAME)
    tmp = out + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)
    if verbose:
        print(f"built {out}")
    build_probe(verbose)
    return out


def build_probe(verbose: bool = True) -> str:
    """The measurement probe used by ``bench.py --mfma-ceiling``."""
    srcs = sorted(glob.glob(os.path.join(CSRC, "probe", "*.hip")))
    out = os.path.join(PKG_DIR, PROBE_LIB_NAME)
    tmp = out + ".tmp"
    cmd = [_hipcc(), *HIP_FLAGS, "-shared", *srcs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"probe build failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)
    if verbose:
        print(f"built {out}")
    return out


if __name__ == "__main__":
    build_library()
