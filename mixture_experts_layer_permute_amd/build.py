"""Builds libmoe.so (the HIP kernels behind the C ABI in include/moe.h) for
gfx950 with hipcc, one object per source in parallel, in-tree."""
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libmoe.so")
BUILD = os.path.join(HERE, "_build")
# Debug build: device-side bounds checks on indexes that come from data
# (MOE_DEBUG_BOUNDS; a failed check traps).  Load it with
# _lib.load(DEBUG_OUT) before anything else loads the library.
DEBUG_OUT = os.path.join(HERE, "libmoe_debug_bounds.so")
DEBUG_FLAGS = ["-DMOE_DEBUG_BOUNDS"]

SOURCES = ["abi.hip", "gate.hip", "permute.hip", "combine.hip", "ggemm.hip"]
# per-file extra flags: the gate's fp32 logits must not fuse multiply-adds
EXTRA = {"gate.hip": ["-ffp-contract=off"]}
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I" + os.path.join(os.path.dirname(HERE), "include")]


def hipcc():
    return os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")


def _compile(src, debug=False):
    obj = os.path.join(BUILD, src.replace(".hip", "_debug.o" if debug else ".o"))
    cmd = [hipcc()] + FLAGS + EXTRA.get(src, []) + (DEBUG_FLAGS if debug else []) + \
        ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s" % (src, r.stderr))
    return obj


def build(jobs: int = 8, debug_bounds: bool = False) -> str:
    """Compile every source and link libmoe.so (or, with debug_bounds, the
    checked library at DEBUG_OUT); returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda src: _compile(src, debug_bounds), SOURCES))
    out = DEBUG_OUT if debug_bounds else OUT
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stderr)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build())
