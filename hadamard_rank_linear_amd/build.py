"""Build the gfx950 HIP library libhlq.so in-tree with hipcc.

Each source compiles to an object of its own (in parallel), then one link."""
from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libhlq.so")
# (source, object, extra flags): the transform kernels build once per block size
SOURCES = [("hlq_tr.hip", f"hlq_tr{n}", [f"-DHLQ_TR_N={n}"]) for n in (16, 32, 64, 128)] + [
    ("hlq_gemm.hip", "hlq_gemm", []), ("hlq_lqs.hip", "hlq_lqs", []),
    ("hlq_acbp.hip", "hlq_acbp", []), ("hlq_noalloc.hip", "hlq_noalloc", []),
    ("hlq_ablation.hip", "hlq_ablation", []),
    ("hlq_api.cpp", "hlq_api", [])]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# Numerics flags: no FMA contraction (the transforms must round every add),
# IEEE division, denormals kept; packed fp32 instructions disabled.
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-ffp-contract=off", "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-fno-gpu-flush-denormals-to-zero",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed: " + " ".join(cmd[-3:]))


def build(verbose: bool = False) -> str:
    os.makedirs(OBJ, exist_ok=True)
    inc = ["-I", os.path.join(ROOT, "include")]
    objs, cmds = [], []
    for src, name, extra in SOURCES:
        o = os.path.join(OBJ, name + ".o")
        objs.append(o)
        cmds.append([HIPCC, *FLAGS, *extra, *inc, "-c", "-o", o, os.path.join(CSRC, src)])
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(cmds)) as ex:
        for f in [ex.submit(_run, c, verbose) for c in cmds]:
            f.result()
    tmp = LIB + ".tmp"
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
