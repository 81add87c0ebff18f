"""CPU hygiene checks.

* The host planner (csrc/plan.cpp, plain C++) built with g++ under
  AddressSanitizer and UndefinedBehaviorSanitizer and driven through valid,
  invalid and seeded random batches (tests/plan_sanitize_driver.cpp).
* The library sources hold no atomics (every reduction has a fixed order), no
  Triton and no CUDA compatibility layer: checked in the source text and in
  the gfx950 assembly the compiler makes from it."""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "invariant_paged_kv_amd", "csrc")
INCLUDE = os.path.join(ROOT, "include")
SOURCES = [os.path.join(CSRC, f) for f in ("bia.hip", "plan.cpp", "plan.h")] + \
    [os.path.join(INCLUDE, "bia.h")]


def _strip_comments(text):
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.sub(r"//[^\n]*", "", text)


def test_planner_under_asan_and_ubsan(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    exe = str(tmp_path / "plan_sanitize")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           f"-I{INCLUDE}", f"-I{CSRC}", os.path.join(CSRC, "plan.cpp"),
           os.path.join(ROOT, "tests", "plan_sanitize_driver.cpp"), "-o", exe]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    assert run.returncode == 0, run.stdout + run.stderr
    assert "0 failures" in run.stdout
    assert "ERROR: AddressSanitizer" not in run.stderr
    assert "runtime error" not in run.stderr


FORBIDDEN_SOURCE = [
    (r"\batomic", "an atomic operation"),
    (r"__hip_atomic|__atomic_|__sync_", "an atomic builtin"),
    (r"\btriton\b", "Triton"),
    (r"cuda_runtime|__CUDA_ARCH__|__CUDACC__|\bcuda[A-Z]\w*\(", "a CUDA shim"),
    (r"__HIP_PLATFORM_(AMD|NVIDIA|HCC|NVCC)__", "a dual-platform path"),
    (r"hipify", "hipify output"),
]


@pytest.mark.parametrize("path", SOURCES, ids=os.path.basename)
def test_sources_have_no_atomics_triton_or_cuda_shims(path):
    code = _strip_comments(open(path).read())
    for pat, what in FORBIDDEN_SOURCE:
        m = re.search(pat, code, flags=re.I)
        assert m is None, f"{os.path.basename(path)} contains {what}: {m.group(0)!r}"


def test_device_assembly_has_no_atomic_instructions(tmp_path):
    hipcc = "/opt/rocm/bin/hipcc" if os.path.exists("/opt/rocm/bin/hipcc") else shutil.which("hipcc")
    if hipcc is None:
        pytest.skip("hipcc not available")
    asm = str(tmp_path / "bia.s")
    cmd = [hipcc, "-O3", "-std=c++17", "--offload-arch=gfx950", "--cuda-device-only", "-S",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-mllvm", "-amdgpu-mfma-vgpr-form=1",
           f"-I{INCLUDE}", f"-I{CSRC}", os.path.join(CSRC, "bia.hip"), "-o", asm]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    text = open(asm).read()
    code = "\n".join(l.split(";")[0] for l in text.splitlines()
                     if l.startswith("\t") and not l.lstrip().startswith("."))
    assert "v_mfma_f32_32x32x16_bf16" in code   # the assembly is the kernels'
    bad = re.findall(r"^\s*((?:global|flat|buffer)_atomic\w*|ds_(?:add|sub|rsub|inc|dec|"
                     r"min|max|and|or|xor|mskor|cmpst|cmpswap|wrxchg)\w*)", code, flags=re.M)
    assert not bad, f"atomic instructions in the device code: {sorted(set(bad))[:10]}"
