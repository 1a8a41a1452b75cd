"""Build the HIP library libnvfp4.so in-tree for gfx950 with hipcc.

Every .hip file under csrc/ is compiled for gfx950 only, with packed-fp32
instructions disabled and no floating-point contraction (the producer's rounding
decisions are written out operation by operation).
"""
import glob
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libnvfp4.so")
OBJ_DIR = os.path.join(HERE, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-function", "-I", os.path.join(HERE, "..", "include")]

# Per-source additions. The producer's work-queue takes are single-lane atomics whose
# result is needed one group later; LLVM's atomic optimizer rewrites them into a form
# that reads the result (and so waits for every load in flight) right after the atomic.
EXTRA_FLAGS = {"producer.hip": ["-mllvm", "-amdgpu-atomic-optimizer-strategy=None"]}


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(OBJ_DIR, os.path.basename(src) + ".o")
    cmd = [HIPCC] + FLAGS + EXTRA_FLAGS.get(os.path.basename(src), []) + ["-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    noise = [l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l and l.strip()]
    if noise and verbose:
        print("\n".join(noise))
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(OBJ_DIR, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), srcs))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
