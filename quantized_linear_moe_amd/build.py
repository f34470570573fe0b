"""Build libqe.so (HIP, gfx950) in-tree with hipcc.

Usage: python quantized_linear_moe_amd/build.py   (or load this file and call build()).
The script imports nothing from the package, so it works before libqe.so exists.
"""

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libqe.so")
SOURCES = ["qe_api.hip", "k_act.hip", "k_gemm_w4.hip", "k_decode.hip", "k_stat.hip", "k_prep.hip", "k_probe.hip",
           "k_cooc.hip", "calib_host.hip", "k_gemm_a16.hip", "k_lowrank.hip"]
ARCH = "gfx950"


def _hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found; libqe needs ROCm's hipcc to build")


def compile_flags():
    return [
        f"--offload-arch={ARCH}",
        "-O3",
        "-std=c++17",
        "-fPIC",
        "-ffp-contract=off",
        "-Wall",
        "-Wno-unused-function",
        "-Wno-unused-variable",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", os.path.join(ROOT, "include"),
    ]


def build(verbose: bool = False) -> str:
    hipcc = _hipcc()
    objdir = os.path.join(ROOT, "_build", "libqe")
    os.makedirs(objdir, exist_ok=True)
    flags = compile_flags()

    def one(src):
        obj = os.path.join(objdir, src + ".o")
        cmd = [hipcc, *flags, "-c", os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
        if verbose and r.stderr.strip():
            err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
            if err.strip():
                print(err, file=sys.stderr)
        return obj

    with ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(one, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs, "-lpthread"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
