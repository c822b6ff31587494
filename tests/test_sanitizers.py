"""AddressSanitizer + UndefinedBehaviorSanitizer builds of the host code, on
the CPU (no GPU, no device code):

* the library's host side (crkv_api.hip compiled as plain C++ with g++:
  argument validation, the planner, budget and format sizes) linked into
  tests/sanitize/host_driver.cpp, which runs the ABI's argument cases and
  planner round trips on every workload shape, including forced kernel
  choices and edge shapes (empty and length-1 chunks, no documents, decode);
* the oracle (oracle/oracle.c) linked into tests/sanitize/oracle_driver.c,
  which runs every mode and input type on small problems, a row range, the
  unmasked flag, top-k with ties and signed zeros, and the budget.

Any sanitizer report (out-of-bounds access, use after free, leak, signed
overflow, misaligned or null access, ...) aborts the driver and fails the
test. Both drivers print a marker line when they finish cleanly."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
ROCM = "/opt/rocm"
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600, **kw)
    assert r.returncode == 0, "%s\n%s\n%s" % (" ".join(cmd), r.stdout[-4000:], r.stderr[-4000:])
    return r


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.exists(os.path.join(ROCM, "include", "hip")),
                    reason="needs g++ and the HIP headers")
def test_host_code_under_sanitizers(tmp_path):
    obj = tmp_path / "crkv_api.o"
    exe = tmp_path / "host_driver"
    inc = ["-I" + os.path.join(ROCM, "include"), "-I" + os.path.join(ROOT, "include"),
           "-I" + os.path.join(ROOT, "attention_precomputed_chunk_amd", "csrc")]
    # host-only C++: the HIP runtime API from the headers, no device code
    _run(["g++", "-std=c++17", "-x", "c++", "-D__HIP_PLATFORM_AMD__", "-DHIP_SYMBOL(X)=X", "-Wall"] + SAN + inc +
         ["-c", os.path.join(ROOT, "attention_precomputed_chunk_amd", "csrc", "crkv_api.hip"), "-o", str(obj)])
    _run(["g++", "-std=c++17", "-D__HIP_PLATFORM_AMD__", "-Wall"] + SAN + inc +
         [os.path.join(HERE, "host_driver.cpp"), str(obj), "-L" + os.path.join(ROCM, "lib"), "-lamdhip64",
          "-Wl,-rpath," + os.path.join(ROCM, "lib"), "-o", str(exe)])
    r = _run([str(exe)], env=ENV)
    assert "HOST_SANITIZE_OK" in r.stdout


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_under_sanitizers(tmp_path):
    exe = tmp_path / "oracle_driver"
    _run(["gcc", "-std=c11", "-fopenmp", "-Wall"] + SAN +
         [os.path.join(HERE, "oracle_driver.c"), os.path.join(ROOT, "oracle", "oracle.c"), "-lm", "-o", str(exe)])
    r = _run([str(exe)], env=ENV)
    assert "ORACLE_SANITIZE_OK" in r.stdout
