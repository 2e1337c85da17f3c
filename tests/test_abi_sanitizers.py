"""AddressSanitizer and UndefinedBehaviorSanitizer over the library's host code (CPU, no GPU needed).

The ABI implementation (api.cpp) is rebuilt with host-side sanitizers (each -fsanitize= behind -Xarch_host,
so no GPU code is instrumented), linked with the kernels' ordinary objects into a separate library, and
driven by tests/abi_sanitize_driver.cpp through every entry point's argument validation. The driver is a
host-only program built with the same sanitizers; it exits with the number of failed checks, and any
sanitizer finding fails the run."""
import os
import subprocess

import pytest

from long_context_block_amd import build as B

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CLANG = os.path.join(os.path.dirname(os.path.realpath(B.HIPCC)), "..", "llvm", "bin", "clang++")
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined", "-Xarch_host",
       "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return r


@pytest.mark.skipif(not os.path.exists(CLANG), reason="the ROCm clang++ is not installed")
def test_host_abi_under_asan_and_ubsan(tmp_path):
    objs = [os.path.join(B.OBJDIR, s + ".o") for s in B.SOURCES if s != "api.cpp"]
    if not all(os.path.exists(o) for o in objs):
        B.build()
    api_o = str(tmp_path / "api_san.o")
    _run([B.HIPCC, *B.COMMON, *SAN, "-x", "hip", "-c", os.path.join(B.CSRC, "api.cpp"), "-o", api_o])
    lib = str(tmp_path / "libpisa_san.so")
    _run([B.HIPCC, f"--offload-arch={B.ARCH}", "-shared", "-fPIC", "-o", lib, api_o, *objs])
    exe = str(tmp_path / "abi_driver")
    # host-only driver (no GPU code on this line): the sanitizer runtimes come with it
    _run([CLANG, "-std=c++17", "-g", "-O1", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
          "-fno-omit-frame-pointer", "-I", os.path.join(ROOT, "include"), os.path.join(HERE, "abi_sanitize_driver.cpp"),
          lib, f"-Wl,-rpath,{tmp_path}", "-o", exe])
    env = dict(os.environ)
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1"  # the HIP runtime keeps allocations until exit
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    env["HIP_VISIBLE_DEVICES"] = ""
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error" not in out, out
    assert r.returncode == 0, out
    assert "0 failed checks" in r.stdout, out
