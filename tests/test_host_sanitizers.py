"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Two separate host-only builds, each with its own driver under
tests/host_sanitize/:

* the library's argument contract and launch planner (csrc/fa_api.cpp and
  csrc/fa_plan.cpp, with stub launch functions that abort if reached): every
  check of the pages' chain and the added ones, the workspace sizes of the five
  workloads and of limit shapes, the forward's early returns and host-side
  device checks;
* the fp64 oracle (oracle/fa_oracle.c): packed and paged layouts, windows at
  the int32 limit, empty sequences, ALiBi, fp16, several threads, the append's
  skip rule and the widening of every 16-bit pattern.

The GPU kernels are not built here (sanitizers run on host code only).
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "host_sanitize")
CSRC = os.path.join(ROOT, "varlen_flash_attention_fa_amd", "csrc")
SAN = ["-g", "-O1", "-fno-omit-frame-pointer", "-fsanitize=address,undefined", "-fno-sanitize-recover=all"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")


def _run(cmd, **kw):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, **kw)
    return r.returncode, r.stdout


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir("/opt/rocm/include"),
                    reason="needs g++ and the ROCm headers")
def test_contract_and_planner_under_sanitizers(tmp_path):
    exe = str(tmp_path / "contract")
    rc, out = _run(["g++", "-std=c++17"] + SAN + ["-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
                   os.path.join(CSRC, "fa_api.cpp"), os.path.join(CSRC, "fa_plan.cpp"),
                   os.path.join(HERE, "stubs.cpp"), os.path.join(HERE, "contract_driver.cpp"),
                   "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-o", exe])
    assert rc == 0, out
    rc, out = _run([exe], env=ENV, timeout=120)
    assert rc == 0 and "0 mismatches" in out, out
    assert "runtime error" not in out and "AddressSanitizer" not in out, out


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle")
    rc, out = _run(["gcc", "-std=c11", "-pthread", "-fno-fast-math", "-ffp-contract=off"] + SAN +
                   [os.path.join(ROOT, "oracle", "fa_oracle.c"), os.path.join(HERE, "oracle_driver.c"),
                    "-lm", "-o", exe])
    assert rc == 0, out
    rc, out = _run([exe], env=ENV, timeout=120)
    assert rc == 0 and "0 mismatches" in out, out
    assert "runtime error" not in out and "AddressSanitizer" not in out, out
