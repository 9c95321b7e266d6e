"""Compile the HIP sources into the in-tree shared library libbkv.so (gfx950)."""
import glob
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libbkv.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-shared", "-fPIC",
    # packed fp32 arithmetic stays off: plain float code only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def sources():
    return sorted(glob.glob(os.path.join(HERE, "csrc", "*.hip")))


def build(verbose=False):
    """Build libbkv.so next to this file; raise on failure."""
    tmp = LIB + ".tmp"
    cmd = [HIPCC] + FLAGS + ["-I", os.path.join(ROOT, "include"),
                             "-I", os.path.join(HERE, "csrc")] + sources() + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + res.stdout + res.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
