"""Build libmlra.so for gfx950 with hipcc (in-tree, no JIT cache).

python -m branch_rank_amd.build [--jobs N] [--no-debug]

Builds libmlra.so and, from the same sources with MLRA_DEBUG_BOUNDS (device
bounds checks, see mlra_bounds_checks in include/mlra.h), libmlra_debug.so.
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
DEBUG_LIB = os.path.join(PKG, "libmlra_debug.so")
OBJ_DEBUG = os.path.join(PKG, "_build_debug")
# the benchmark's HBM read-ceiling probe (include/mlra_probe.h), a library of its own
PROBE_SRC = "probe_read.hip"
PROBE_LIB = os.path.join(PKG, "libmlra_probe.so")

SOURCES = ["mlra_api.cpp", "kernels_generic.hip", "decode_mfma.hip", "decode_branch.hip",
           "decode_wide.hip", "proj_mfma.hip", "cache_append.hip", "prefill_branch.hip",
           "prefill_mha.hip"]
# The split-KV decode kernels hold no NaN by construction (finite scores, -inf
# for masked tokens): without NaN semantics their max reductions need no
# canonicalising moves.
EXTRA = {"decode_mfma.hip": ["-fno-honor-nans"], "decode_branch.hip": ["-fno-honor-nans"],
         "decode_wide.hip": ["-fno-honor-nans", "-mllvm", "-amdgpu-mfma-vgpr-form"],
         "prefill_branch.hip": ["-fno-honor-nans"], "prefill_mha.hip": ["-fno-honor-nans"]}
# decode_wide.hip holds 200 registers of query and output per lane beside a
# second wave on its SIMD: with the MFMA results selected into VGPRs the
# register allocator keeps the loop free of spills (the default, every MFMA
# result in AGPRs, spills)

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unknown-warning-option",
    f"-I{os.path.join(ROOT, 'include')}",
]


def _compile(src, debug=False):
    obj = os.path.join(OBJ_DEBUG if debug else OBJ, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, *(["-DMLRA_DEBUG_BOUNDS"] if debug else []), *EXTRA.get(src, []),
           "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    return src, obj, r.returncode, r.stdout + r.stderr, cmd


def _link(objs, lib):
    tmp = lib + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode:
        print(" ".join(cmd))
        print(r.stdout + r.stderr)
        raise RuntimeError(f"link of {os.path.basename(lib)} failed")
    os.replace(tmp, lib)


def build(jobs=None, verbose=False, debug=True):
    os.makedirs(OBJ, exist_ok=True)
    os.makedirs(OBJ_DEBUG, exist_ok=True)
    work = [(s, False) for s in SOURCES + [PROBE_SRC]]
    if debug:
        work += [(s, True) for s in SOURCES]
    jobs = jobs or min(len(work), os.cpu_count() or 1)
    objs = {}
    with cf.ThreadPoolExecutor(jobs) as ex:
        for (src, dbg), (_, obj, rc, out, cmd) in zip(work, ex.map(lambda a: _compile(*a), work)):
            if verbose or rc:
                print(" ".join(cmd))
                print(out)
            if rc:
                raise RuntimeError(f"hipcc failed on {src}{' (debug)' if dbg else ''}")
            objs[(src, dbg)] = obj
    _link([objs[(s, False)] for s in SOURCES], LIB)
    _link([objs[(PROBE_SRC, False)]], PROBE_LIB)
    if debug:
        _link([objs[(s, True)] for s in SOURCES], DEBUG_LIB)
    return LIB


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=None)
    ap.add_argument("-v", "--verbose", action="store_true")
    ap.add_argument("--no-debug", action="store_true", help="skip libmlra_debug.so")
    a = ap.parse_args()
    print(build(a.jobs, a.verbose, debug=not a.no_debug))
    sys.exit(0)
