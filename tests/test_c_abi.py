"""The C ABI from C.

* tests/c_abi_consumer.c: a C99 program that includes only include/bia.h and
  links the built libbia.so, plans prefill and decode batches, checks their
  work lists against counts it derives from the split rule itself, and
  checks the status codes and messages of invalid calls (host-side, no GPU).
* tests/c_abi_gpu.c (GPU): a C99 program that runs a paged decode through the
  header alone, with device memory from the HIP runtime API and no Python or
  torch, on inputs whose result has a closed form (identical keys: the mean
  of the values and lse = logit + ln(kv_len)), one request spanning three
  partitions."""
import os
import shutil
import subprocess

import pytest

from invariant_paged_kv_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def _build(tmp_path, source, hip=False):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not found")
    lib = _lib.lib_path()
    if not os.path.exists(lib):
        pytest.fail(f"{lib} is not built (python __graft_entry__.py build)")
    exe = str(tmp_path / os.path.splitext(source)[0])
    cmd = [gcc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic",
           "-I" + os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", source),
           "-L" + os.path.dirname(lib), "-l:" + os.path.basename(lib)]
    rpath = [os.path.dirname(lib)]
    if hip:
        cmd[1:1] = ["-D__HIP_PLATFORM_AMD__", "-isystem", os.path.join(ROCM, "include")]
        cmd += ["-L" + os.path.join(ROCM, "lib"), "-lamdhip64", "-lm"]
        rpath.append(os.path.join(ROCM, "lib"))
    cmd += ["-Wl,-rpath," + ":".join(rpath), "-o", exe]
    build = subprocess.run(cmd, capture_output=True, text=True)
    assert build.returncode == 0, build.stderr
    return exe


def test_c99_consumer(tmp_path):
    exe = _build(tmp_path, "c_abi_consumer.c")
    run = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert run.returncode == 0 and run.stdout.strip().endswith("ok"), run.stdout + run.stderr


@pytest.mark.gpu
def test_c99_decode_on_gpu(tmp_path):
    exe = _build(tmp_path, "c_abi_gpu.c", hip=True)
    print("[gpu] C99 decode through include/bia.h", flush=True)
    run = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    print(run.stdout, run.stderr, flush=True)
    assert run.returncode == 0 and run.stdout.strip().endswith("ok"), run.stdout + run.stderr
