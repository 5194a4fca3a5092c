"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (no GPU):
the C ABI's argument validation (api.cpp, its kernel launchers replaced by
host stand-ins that record the call) and every entry point of the CPU
oracle (oracle/oracle.c), driven by tests/c/sanitize_main.cpp with ordinary,
degenerate and extreme arguments.  Built with the host compilers only (gcc
and g++); no device code is involved."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
       "-g", "-O1"]


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return r


@pytest.mark.skipif(shutil.which("gcc") is None or shutil.which("g++") is None,
                    reason="host compilers not found")
def test_abi_validation_and_oracle_under_asan_ubsan(tmp_path):
    inc = ["-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include",
           "-D__HIP_PLATFORM_AMD__"]
    objs = []
    _run(["gcc", "-std=gnu11", "-fopenmp", "-ffp-contract=off", *SAN, "-c",
          os.path.join(ROOT, "oracle", "oracle.c"), "-o", str(tmp_path / "oracle.o")])
    objs.append(str(tmp_path / "oracle.o"))
    for src in ("block_sparse_gemm_amd/csrc/api.cpp", "tests/c/sanitize_stubs.cpp",
                "tests/c/sanitize_main.cpp"):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        _run(["g++", "-std=c++17", *SAN, *inc, "-c", os.path.join(ROOT, src), "-o", obj])
        objs.append(obj)
    exe = str(tmp_path / "sanitize_driver")
    _run(["g++", *SAN, "-fopenmp", *objs, "-o", exe])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1", OMP_NUM_THREADS="2")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out
    assert "runtime error" not in out and "AddressSanitizer" not in out, out
    assert "sanitized checks passed" in out
