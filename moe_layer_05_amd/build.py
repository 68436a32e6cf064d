"""Ahead-of-time build of the HIP library libmoemi.so for gfx950.

Every kernel is compiled here, once; nothing is compiled at run time.  The
library lands next to this file (in-tree), where the Python binding loads it.

    python -m moe_layer_05_amd.build          # or __graft_entry__.build()
"""

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libmoemi.so")
OBJDIR = os.path.join(ROOT, "_build")

SOURCES = ["api.hip", "router.hip", "align.hip", "front.hip", "quant.hip", "gemm_decode.hip", "gemm_tile.hip",
           "down_small.hip", "combine.hip", "rope.hip"]

ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # packed FP32 arithmetic stays off: the compiler then never emits
    # v_pk_{add,mul,fma}_f32 from ordinary float code.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    f"-I{os.path.join(ROOT, 'include')}",
]


def hipcc():
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build libmoemi.so)")


def _compile(src, verbose):
    obj = os.path.join(OBJDIR, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops" not in l and l.strip())
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{msg}")
    if verbose and msg:
        print(msg, file=sys.stderr)
    return obj


def build(verbose=False, jobs=8):
    """Compile every source for gfx950 and link libmoemi.so (always rebuilds)."""
    os.makedirs(OBJDIR, exist_ok=True)
    with ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
