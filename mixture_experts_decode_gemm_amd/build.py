"""Builds libmoedecode.so (the HIP kernels and the C ABI) for gfx950, in-tree.

Every source is compiled by hipcc with --offload-arch=gfx950 -O3 and the packed-FP32
instructions disabled; router.hip (the bit-exact routing arithmetic) additionally with
-ffp-contract=off, ffn.hip without the atomic optimizer.  Objects go to _build/ next to this file; the library is linked into
this package directory.
"""
import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libmoedecode.so")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["abi.hip", "finalize.hip", "quant.hip", "router.hip", "lists.hip", "ffn.hip",
           "gemm.hip", "wgemm.hip", "norm.hip"]
COMMON = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I", CSRC, "-I", INCLUDE]
# ffn.hip: the expert passes take work tickets with one atomic add by one thread; the
# atomic optimizer would turn it into a wave-wide add whose result is read at once (a wait
# for every load in flight), so it is off there
PER_FILE = {"router.hip": ["-ffp-contract=off"],
            "ffn.hip": ["-mllvm", "-amdgpu-atomic-optimizer-strategy=None"]}


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(OBJ, src.replace(".hip", ".o"))
    cmd = [HIPCC, *COMMON, *PER_FILE.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    if verbose and r.stderr.strip():
        print(r.stderr, flush=True)
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(OBJ, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    # only the C ABI's entry points are exported (the version script hides the rest)
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs,
           "-Wl,--version-script=" + os.path.join(CSRC, "exports.map"), "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
    print(LIB)
