"""Build libmlra.so for gfx950 with hipcc (in-tree, no JIT cache).

python -m branch_rank_amd.build [--jobs N]
"""

import argparse
import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libmlra.so")

SOURCES = ["mlra_api.cpp", "kernels_generic.hip", "decode_mfma.hip", "decode_branch.hip",
           "proj_mfma.hip", "cache_append.hip", "prefill_branch.hip"]
# The split-KV decode kernels hold no NaN by construction (finite scores, -inf
# for masked tokens): without NaN semantics their max reductions need no
# canonicalising moves.
EXTRA = {"decode_mfma.hip": ["-fno-honor-nans"], "decode_branch.hip": ["-fno-honor-nans"],
         "prefill_branch.hip": ["-fno-honor-nans"]}

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unknown-warning-option",
    f"-I{os.path.join(ROOT, 'include')}",
]


def _compile(src):
    obj = os.path.join(OBJ, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, *EXTRA.get(src, []), "-x", "hip", "-c", os.path.join(CSRC, src),
           "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    return src, obj, r.returncode, r.stdout + r.stderr, cmd


def build(jobs=None, verbose=False):
    os.makedirs(OBJ, exist_ok=True)
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 1)
    objs = []
    with cf.ThreadPoolExecutor(jobs) as ex:
        for src, obj, rc, out, cmd in ex.map(_compile, SOURCES):
            if verbose or rc:
                print(" ".join(cmd))
                print(out)
            if rc:
                raise RuntimeError(f"hipcc failed on {src}")
            objs.append(obj)
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode:
        print(" ".join(cmd))
        print(r.stdout + r.stderr)
        raise RuntimeError("link failed")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=None)
    ap.add_argument("-v", "--verbose", action="store_true")
    a = ap.parse_args()
    print(build(a.jobs, a.verbose))
    sys.exit(0)
