"""Host code under the address and undefined-behaviour sanitizers (no GPU).

- The C ABI layer (api.cpp) and the workspace sizes (sizes.cpp), built by the host compiler
  with stand-in launchers (tests/sanitize/stub_kernels.cpp), driven through every entry
  point: valid calls, each documented error, aliasing, launch failures, overflowing sizes.
- The CPU oracle's C code (token recurrence and its adjoint) on small seeded inputs, with
  several thread counts and checkpoint segments.

Any sanitizer report aborts the driver (-fno-sanitize-recover=all), failing the test."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "gated_delta_rule_06_amd", "csrc")
HERE = os.path.join(ROOT, "tests", "sanitize")
SAN = ["-g", "-O1", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
       "-fno-omit-frame-pointer", "-Wall", "-Wextra", "-Werror"]
HIP_INC = "/opt/rocm/include"


def run(cmd, **kw):
    out = subprocess.run(cmd, capture_output=True, text=True, timeout=600, **kw)
    assert out.returncode == 0, f"{' '.join(map(str, cmd))}\n{out.stdout[-4000:]}\n{out.stderr[-4000:]}"
    return out


def test_c_abi_host_logic_is_clean_under_sanitizers(tmp_path):
    cxx = shutil.which("g++")
    if cxx is None or not os.path.exists(os.path.join(HIP_INC, "hip", "hip_runtime.h")):
        pytest.skip("needs g++ and the HIP runtime headers")
    exe = tmp_path / "abi_driver"
    run([cxx, "-std=c++17", *SAN, "-D__HIP_PLATFORM_AMD__", f"-I{HIP_INC}",
         f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}",
         os.path.join(CSRC, "api.cpp"), os.path.join(CSRC, "sizes.cpp"),
         os.path.join(HERE, "stub_kernels.cpp"), os.path.join(HERE, "abi_driver.cpp"),
         "-o", str(exe)])
    out = run([str(exe)], env={**os.environ, "ASAN_OPTIONS": "detect_leaks=1"})
    assert out.stdout.strip().endswith("launches") and out.stdout.startswith("0 failures"), out.stdout


def test_oracle_c_code_is_clean_under_sanitizers(tmp_path):
    cc = shutil.which("gcc")
    if cc is None:
        pytest.skip("needs gcc")
    exe = tmp_path / "oracle_driver"
    run([cc, "-std=c11", *SAN, "-fopenmp", os.path.join(ROOT, "oracle", "recurrence.c"),
         os.path.join(HERE, "oracle_driver.c"), "-lm", "-o", str(exe)])
    out = run([str(exe)], env={**os.environ, "ASAN_OPTIONS": "detect_leaks=1"})
    assert "oracle driver: ok" in out.stdout, out.stdout
