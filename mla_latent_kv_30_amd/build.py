"""Build libmla.so (the gfx950 HIP kernels and the C entry points) in-tree.

Usage: python -m mla_latent_kv_30_amd.build [--jobs N] [--save-temps]
"""

from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libmla.so")
SOURCES = ["api.hip", "absorb.hip", "cache_write.hip", "decode.hip", "merge.hip", "linear.hip", "upproj.hip",
           "ceilings.hip", "decode_wide.hip"]
ARCH = "gfx950"

# -packed-fp32-ops: keep the compiler from forming packed fp32 add/mul/fma.
CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


# Extra flags per source.  The wide decode kernel keeps its latent
# accumulators in the accumulation registers itself (one-instruction
# products) and wants every compiler-built matrix product in ordinary VGPRs.
FILE_FLAGS = {"decode_wide.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def hipcc() -> str:
    for c in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def _compile(src: str, save_temps: bool) -> str:
    obj = os.path.join(OBJ, src.replace(".hip", ".o"))
    cmd = [hipcc(), *CFLAGS, *FILE_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    if save_temps:
        cmd += ["-save-temps=obj"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [ln for ln in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in ln]
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n" + "\n".join(msgs))
    if msgs:
        sys.stderr.write("\n".join(msgs) + "\n")
    return obj


def build(jobs: int = 8, save_temps: bool = False) -> str:
    os.makedirs(OBJ, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(lambda s: _compile(s, save_temps), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=min(8, os.cpu_count() or 1))
    ap.add_argument("--save-temps", action="store_true")
    args = ap.parse_args()
    print(build(args.jobs, args.save_temps))
