"""Build the HIP library libzds.so in-tree for gfx950.

    python -m zero_sharded_mixed_tensor_amd.build

Every .hip file under csrc/ is compiled with hipcc and every .cpp file (host
only code) with the host C++ compiler to an object in _build/, then the
objects are linked into zero_sharded_mixed_tensor_amd/libzds.so.
Floating point: no contraction into FMAs (-ffp-contract=off) and packed fp32
instructions disabled; fp32 divide and sqrt keep HIP's correctly rounded
default.
"""

import concurrent.futures
import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libzds.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


# Host-only sources (the offloaded CPU optimizer): the host compiler, the same
# floating-point rules (no contraction; IEEE divide and sqrt; errno-free sqrt
# so it vectorises), AVX2 + F16C.
CXX = os.environ.get("CXX", "g++")
HOST_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-Wall", "-pthread",
    "-ffp-contract=off", "-fno-math-errno", "-mavx2", "-mf16c",
    "-I", INCLUDE, "-I", CSRC,
]


def _compile(src, extra):
    if src.endswith(".cpp"):
        obj = os.path.join(BUILD, os.path.basename(src).replace(".cpp", "_host.o"))
        cmd = [CXX, *HOST_FLAGS, "-c", src, "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError("host compile failed for %s:\n%s\n%s" % (src, " ".join(cmd), r.stderr))
        return obj
    obj = os.path.join(BUILD, os.path.basename(src).replace(".hip", ".o"))
    cmd = [HIPCC, *CFLAGS, *extra, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, " ".join(cmd), r.stderr))
    return obj


def build(out=LIB, extra_flags=(), verbose=False):
    """Compile and link; returns the path of the shared library."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, list(extra_flags)), srcs))
    tmp = out + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-pthread", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd), r.stderr))
    os.replace(tmp, out)
    if verbose:
        print("built", out)
    return out


if __name__ == "__main__":
    build(verbose=True, extra_flags=sys.argv[1:])
