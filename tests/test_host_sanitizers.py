"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

`python -m zero_sharded_mixed_tensor_amd.build --sanitize` writes
libzds_san.so: the same library with every host-side translation unit built
with -fsanitize=address,undefined (device code is compiled as usual). These
CPU tests run the host-path suites against it in a child process with the
sanitizer runtime preloaded: argument checking, geometry and plans, the
checkpoint's threaded I/O and shared mapping, the host AdamW's thread pool,
the ctypes binding, and the C99 client. Any sanitizer report aborts the child,
which fails the test.
"""

import os
import shutil
import subprocess
import sys

import pytest

from zero_sharded_mixed_tensor_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

HOST_SUITES = ["tests/test_abi_cpu.py", "tests/test_binding_cpu.py", "tests/test_checkpoint_cpu.py",
               "tests/test_cpu_offload.py"]


def _sanitized_env():
    if not os.path.exists(B.SAN_LIB):
        pytest.skip("libzds_san.so not built (python -m zero_sharded_mixed_tensor_amd.build --sanitize)")
    try:
        return B.sanitizer_env()
    except RuntimeError as e:
        pytest.skip(str(e))


def test_host_suites_under_asan_ubsan():
    env = _sanitized_env()
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu",
                        *HOST_SUITES], cwd=ROOT, env=env, capture_output=True, text=True, timeout=1200)
    tail = (r.stdout + r.stderr)[-4000:]
    assert r.returncode == 0, tail
    assert "passed" in r.stdout and "ERROR: AddressSanitizer" not in r.stderr, tail


def test_loaded_library_is_the_sanitized_build():
    env = _sanitized_env()
    code = ("from zero_sharded_mixed_tensor_amd import zds; m = open('/proc/self/maps').read(); "
            "print(zds.LIB_PATH.endswith('libzds_san.so') and 'libzds_san.so' in m and 'libclang_rt.asan' in m)")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    assert r.stdout.strip().endswith("True")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="no C compiler")
def test_c99_client_under_asan_ubsan(tmp_path):
    env = _sanitized_env()
    # the client links against a library named libzds; give it the sanitized one
    shutil.copy(B.SAN_LIB, tmp_path / "libzds.so")
    exe = str(tmp_path / "abi_smoke")
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror",
                    "-I", os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "c", "abi_smoke.c"),
                    "-L", str(tmp_path), "-lzds", "-Wl,-rpath," + str(tmp_path),
                    # the sanitizer runtime the library calls into is preloaded when it runs
                    "-Wl,--allow-shlib-undefined", "-lm", "-o", exe], check=True)
    r = subprocess.run([exe, str(tmp_path)], env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-4000:]
    assert r.stdout.strip() == "ok"
