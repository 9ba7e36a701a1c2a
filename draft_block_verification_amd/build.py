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


def build(verbose=False, out=LIB):
    """Compile every HIP source into one shared library (always recompiles)."""
    tmp = out + ".tmp"
    cmd = [hipcc()] + HIP_FLAGS + [os.path.join(CSRC, s) for s in SOURCES] + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(line for line in res.stderr.splitlines()
                     if "packed-fp32-ops" not in line and "not a recognized feature" not in line)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + errs)
    if verbose and errs.strip():
        print(errs, file=sys.stderr)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
