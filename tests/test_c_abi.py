"""The C ABI from C: tests/c_abi_consumer.c, a C99 program that includes only
include/bia.h and links the built libbia.so, plans prefill and decode
batches, checks their work lists against counts it derives from the split
rule itself, and checks the status codes and messages of invalid calls. All
of it is host-side (no GPU)."""
import os
import shutil
import subprocess

import pytest

from invariant_paged_kv_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_c99_consumer(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not found")
    lib = _lib.lib_path()
    if not os.path.exists(lib):
        pytest.fail(f"{lib} is not built (python __graft_entry__.py build)")
    exe = str(tmp_path / "c_abi_consumer")
    cmd = [gcc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic",
           "-I" + os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "c_abi_consumer.c"),
           "-L" + os.path.dirname(lib), "-l:" + os.path.basename(lib),
           "-Wl,-rpath," + os.path.dirname(lib), "-o", exe]
    build = subprocess.run(cmd, capture_output=True, text=True)
    assert build.returncode == 0, build.stderr
    run = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert run.returncode == 0 and run.stdout.strip().endswith("ok"), run.stdout + run.stderr
