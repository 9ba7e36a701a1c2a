"""Build libdbv.so (HIP, gfx950) in-tree with hipcc.

    python -m draft_block_verification_amd.build

The library is written next to this file so it travels with the source tree.
"""

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libdbv.so")
SOURCES = ["api.hip", "kernels_chain.hip", "kernels_tree.hip", "kernels_anyorder.hip", "kernels_truncate.hip",
           "kernels_ddtree.hip"]

HIP_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # Contractions are written out (fmaf) so every kernel evaluates a formula
    # identically; no implicit fusion.
    "-ffp-contract=off",
    # Packed FP32 (v_pk_*_f32) stays off in every kernel of this library.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
]


def hipcc():
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _filter(stderr):
    return "\n".join(line for line in stderr.splitlines()
                     if "packed-fp32-ops" not in line and "not a recognized feature" not in line)


def build(verbose=False, out=LIB):
    """Compile every HIP source (in parallel, one object each) and link them
    into one shared library (always recompiles)."""
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    compile_flags = [f for f in HIP_FLAGS if f != "-shared"]
    jobs = []
    for src in SOURCES:
        obj = os.path.join(objdir, src.replace(".hip", ".o"))
        cmd = [hipcc()] + compile_flags + ["-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        jobs.append((obj, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)))
    objs, errs, failed = [], [], False
    for obj, proc in jobs:
        _, err = proc.communicate()
        errs.append(_filter(err))
        failed |= proc.returncode != 0
        objs.append(obj)
    if failed:
        raise RuntimeError("hipcc failed:\n" + "\n".join(e for e in errs if e.strip()))
    tmp = out + ".tmp"
    cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC"] + objs + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("link failed:\n" + _filter(res.stderr))
    if verbose and any(e.strip() for e in errs):
        print("\n".join(e for e in errs if e.strip()), file=sys.stderr)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
