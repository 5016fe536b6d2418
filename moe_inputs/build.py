"""Builds libmoe_inputs.so, the device twin of the input generator."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "csrc", "fill.hip")
OUT = os.path.join(HERE, "libmoe_inputs.so")


def build() -> str:
    hipcc = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")
    tmp = OUT + ".tmp%d" % os.getpid()
    cmd = [hipcc, "--offload-arch=gfx950", "-O3", "-fPIC", "-shared",
           "-ffp-contract=off", "-Xclang", "-target-feature", "-Xclang",
           "-packed-fp32-ops", SRC, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + r.stderr)
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build())
