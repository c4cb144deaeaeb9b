"""Build the HIP library (libie.so) for gfx950 with hipcc, in-tree.

Every translation unit is compiled in parallel into integer_only_dnn_amd/_build,
then linked into integer_only_dnn_amd/libie.so.
"""

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libie.so")
SOURCES = ["ie_api.hip", "ie_aux.hip", "ie_update.hip", "ie_gemm_kk.hip", "ie_gemm_im2col.hip",
           "ie_gemm_dgrad.hip", "ie_gemm_dgrad_wt.hip", "ie_gemm_wgrad.hip", "ie_gemm_pair.hip",
           "ie_gemm_pair_al.hip", "ie_pointwise.hip", "ie_gemm_batched.hip"]
# host-only C++ (planner, argument checks, workspace layout): no GPU code
HOST_SOURCES = ["ie_plan.cpp"]
CXX = os.environ.get("CXX", "g++")
HOST_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # keep the compiler from forming packed fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (res.stdout + res.stderr).splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in l)
    if res.returncode != 0:
        sys.stderr.write(out + "\n")
        raise RuntimeError("hipcc failed: " + " ".join(cmd[-3:]))
    return out


def build(verbose: bool = False) -> str:
    """Compile every source and link libie.so (always recompiles)."""
    os.makedirs(OBJ, exist_ok=True)
    jobs = []
    for s in SOURCES:
        obj = os.path.join(OBJ, s.replace(".hip", ".o"))
        jobs.append(([HIPCC, *FLAGS, "-c", os.path.join(CSRC, s), "-o", obj], obj))
    for s in HOST_SOURCES:
        obj = os.path.join(OBJ, s.replace(".cpp", ".o"))
        jobs.append(([CXX, *HOST_FLAGS, "-c", os.path.join(CSRC, s), "-o", obj], obj))
    with ThreadPoolExecutor(max_workers=min(len(jobs), os.cpu_count() or 4)) as ex:
        list(ex.map(lambda j: _run(j[0], verbose), jobs))
    tmp = LIB + ".tmp"
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *[o for _, o in jobs]], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
