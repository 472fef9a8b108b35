"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer,
without a GPU: a sanitized build of the library (host code instrumented, device
code as usual) and tests/abi_driver.c, which drives every entry point through its
argument, dimension and workspace checks, the size queries over wide ranges and
the timing API. Any sanitizer report fails the run."""

import importlib.util
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CLANG = "/opt/rocm/llvm/bin/clang"


def _build_module():
    spec = importlib.util.spec_from_file_location("vdm_build", os.path.join(ROOT, "shape_vae_decoding_amd", "build.py"))
    b = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(b)
    return b


@pytest.mark.skipif(not os.path.exists(CLANG), reason="ROCm clang not installed")
def test_abi_driver_under_asan_and_ubsan(tmp_path):
    lib = _build_module().build_sanitized(str(tmp_path))
    exe = str(tmp_path / "abi_driver")
    san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined"]
    subprocess.run([CLANG, "-O1", "-g", *san, "-I" + os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "abi_driver.c"),
                    "-o", exe, "-L" + str(tmp_path), "-lvdm_asan", "-Wl,-rpath," + str(tmp_path), "-lm"], check=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:halt_on_error=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error" not in out and "LeakSanitizer" not in out, out
    assert r.returncode == 0 and "ok: 0 failed checks" in out, out
