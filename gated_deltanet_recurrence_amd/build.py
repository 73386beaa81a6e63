"""Builds libgdr.so (the HIP kernels and the C ABI) for gfx950 with hipcc."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libgdr.so")
SOURCES = ["gdr_api.hip", "gdr_decode.hip", "gdr_chunk.hip", "gdr_norm.hip", "gdr_conv.hip"]

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # packed-fp32 forms are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fvisibility=hidden", "-Wall",
]


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = (["hipcc"] + FLAGS + ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
           + [os.path.join(CSRC, s) for s in SOURCES] + ["-o", tmp])
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "unknown target feature"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l and "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed:\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
