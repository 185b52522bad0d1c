"""The boundary is a C ABI: a C99 program that includes include/zds.h,
compiled with gcc -std=c99 -Werror (no C++), links against libzds.so and
calls the entry points that need no GPU."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB_DIR = os.path.join(ROOT, "zero_sharded_mixed_tensor_amd")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="no C compiler")
def test_c99_client_compiles_links_and_runs(tmp_path):
    if not os.path.exists(os.path.join(LIB_DIR, "libzds.so")):
        pytest.skip("libzds.so not built")
    exe = str(tmp_path / "abi_smoke")
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror",
                    "-I", os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "c", "abi_smoke.c"),
                    "-L", LIB_DIR, "-lzds", "-Wl,-rpath," + LIB_DIR, "-lm", "-o", exe], check=True)
    r = subprocess.run([exe, str(tmp_path)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    assert r.stdout.strip() == "ok"
