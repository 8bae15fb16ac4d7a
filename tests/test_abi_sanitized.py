"""The C-ABI layer under AddressSanitizer and UndefinedBehaviorSanitizer, on
the CPU: abi.cpp is built with g++ -fsanitize=address,undefined into a shared
library whose kernel launchers are recording stubs (tests/abi_stubs.cpp), and
the ABI test suite (tests/test_abi_cpu.py) plus valid-call dispatch cases
(tests/abi_stub_dispatch.py) run against it in a child process with the ASan
runtime preloaded. Any sanitizer report aborts the child and fails the test.
Host code only: no GPU code is built or run here."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "fp4_quantized_diffusion_amd", "csrc")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def runtime(name):
    p = subprocess.run(["g++", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


@pytest.mark.skipif(runtime("libasan.so") is None, reason="no ASan runtime for g++")
def test_abi_layer_is_clean_under_asan_and_ubsan(tmp_path):
    lib = str(tmp_path / "libfp4rollout_asan.so")
    build = ["g++", "-std=c++17", "-O1", "-g", "-fPIC", "-shared", "-fno-omit-frame-pointer",
             "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-D__HIP_PLATFORM_AMD__",
             f"-I{ROCM}/include", f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}",
             os.path.join(CSRC, "abi.cpp"), os.path.join(ROOT, "tests", "abi_stubs.cpp"), "-o", lib]
    subprocess.run(build, check=True)
    env = dict(os.environ)
    env.update(LD_PRELOAD=runtime("libasan.so"), FP4_ABI_TEST_LIB=lib,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1",
               PYTHONPATH=ROOT)
    cmd = [sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-k", "not rollout_lora",
           os.path.join(ROOT, "tests", "test_abi_cpu.py"), os.path.join(ROOT, "tests", "abi_stub_dispatch.py")]
    r = subprocess.run(cmd, env=env, cwd=ROOT, capture_output=True, text=True, timeout=600)
    tail = (r.stdout + r.stderr)[-4000:]
    assert r.returncode == 0, tail
    assert "passed" in r.stdout and "ERROR: AddressSanitizer" not in tail and "runtime error" not in tail, tail
