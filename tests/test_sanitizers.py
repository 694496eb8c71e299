"""AddressSanitizer / UndefinedBehaviorSanitizer builds of the CPU-side code,
run on the host (no GPU):

* the fp64 oracle (``oracle/gdn_oracle.c``, gcc), driven through every entry
  point on small inputs by ``tests/sanitize/oracle_main.c``;
* the host side of ``libgdn`` (argument validation, workspace-size queries,
  the carving of the prefill workspace into regions), driven by
  ``tests/sanitize/abi_main.cpp``.  hipcc applies the sanitizers to the host
  code only (``-Xarch_host``); the kernels are compiled but never launched,
  since every call the driver makes is rejected before any HIP call.

Any out-of-bounds access or undefined operation aborts the driver.  Leak
checking stays on for the oracle; for the library driver it is off, since the
HIP runtime it links keeps allocations of its own until exit.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")


def _run(cmd, env=None, timeout=300):
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=timeout, env=env)
    assert r.returncode == 0, f"{' '.join(cmd[:3])}... failed ({r.returncode}):\n{r.stdout[-3000:]}\n{r.stderr[-3000:]}"
    return r.stdout


def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_san")
    _run(["gcc", "-std=c99", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
          "-fno-sanitize-recover=all", "-o", exe, os.path.join(HERE, "oracle_main.c"),
          os.path.join(ROOT, "oracle", "gdn_oracle.c"), "-lm"])
    assert "ok" in _run([exe])


@pytest.mark.skipif(not os.path.exists("/opt/rocm/bin/hipcc"), reason="hipcc not installed")
def test_library_host_code_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "abi_san")
    csrc = os.path.join(ROOT, "linear_attention_sequence_gdn_amd", "csrc")
    srcs = [os.path.join(csrc, f) for f in ("gdn_api.hip", "gdn_prefill.hip", "gdn_decode.hip", "gdn_backward.hip")]
    _run(["/opt/rocm/bin/hipcc", "--offload-arch=gfx950", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
          "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
          "-Xarch_host", "-fno-sanitize-recover=all",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-o", exe, os.path.join(HERE, "abi_main.cpp"), *srcs], timeout=600)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0")
    assert "ok" in _run([exe], env=env)
