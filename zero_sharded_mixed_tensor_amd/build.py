"""Build the HIP library libzds.so in-tree for gfx950.

    python -m zero_sharded_mixed_tensor_amd.build              # libzds.so
    python -m zero_sharded_mixed_tensor_amd.build --sanitize   # libzds_san.so

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


# Host AddressSanitizer + UndefinedBehaviorSanitizer build (host code only;
# device code is compiled as usual): `--sanitize` writes libzds_san.so next to
# the library. The host-only sources go through the ROCm clang so that one
# sanitizer runtime serves the whole library; a process loads it with that
# runtime preloaded (see sanitizer_env()).
SAN_LIB = os.path.join(PKG, "libzds_san.so")
SAN_BUILD = os.path.join(PKG, "_build_san")
CLANGXX = "/opt/rocm/llvm/bin/clang++"
SAN_HIP_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
SAN_HOST_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer"]


def sanitizer_runtime():
    """The ROCm clang's ASan runtime (UBSan included), for LD_PRELOAD."""
    libs = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not libs:
        raise RuntimeError("no libclang_rt.asan-x86_64.so under /opt/rocm/llvm")
    return libs[-1]


def sanitizer_env(base=None):
    """Environment for a process that loads libzds_san.so."""
    env = dict(os.environ if base is None else base)
    env["LD_PRELOAD"] = sanitizer_runtime()
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    env["ZDS_LIBRARY"] = SAN_LIB
    return env


def _compile(src, extra, build_dir=BUILD, sanitize=False):
    if src.endswith(".cpp"):
        obj = os.path.join(build_dir, os.path.basename(src).replace(".cpp", "_host.o"))
        if sanitize:
            flags = [f for f in HOST_FLAGS if f != "-pthread"] + ["-pthread"] + SAN_HOST_FLAGS
            cmd = [CLANGXX, *flags, "-c", src, "-o", obj]
        else:
            cmd = [CXX, *HOST_FLAGS, "-c", src, "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError("host compile failed for %s:\n%s\n%s" % (src, " ".join(cmd), r.stderr))
        return obj
    obj = os.path.join(build_dir, os.path.basename(src).replace(".hip", ".o"))
    cmd = [HIPCC, *CFLAGS, *(SAN_HIP_FLAGS if sanitize else []), *extra, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, " ".join(cmd), r.stderr))
    return obj


def build(out=None, extra_flags=(), verbose=False, sanitize=False):
    """Compile and link; returns the path of the shared library."""
    out = out or (SAN_LIB if sanitize else LIB)
    build_dir = SAN_BUILD if sanitize else BUILD
    os.makedirs(build_dir, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, list(extra_flags), build_dir, sanitize), srcs))
    tmp = out + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-pthread", *objs, "-o", tmp]
    if sanitize:
        cmd[3:3] = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                    "-shared-libsan"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd), r.stderr))
    os.replace(tmp, out)
    if verbose:
        print("built", out)
    return out


if __name__ == "__main__":
    args = sys.argv[1:]
    san = "--sanitize" in args
    build(verbose=True, extra_flags=[a for a in args if a != "--sanitize"], sanitize=san)
