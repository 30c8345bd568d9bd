"""Host code under AddressSanitizer and UndefinedBehaviourSanitizer (CPU only).

- The host dispatch (csrc/tree_attn.cpp: argument checks, split choice,
  workspace layout) is built with g++ and the sanitizers, with the kernel
  launchers replaced by recording stubs (tests/sanitize/host_checks.cpp), and
  every entry point is called with valid and invalid arguments.
- The oracle (oracle/tree_attn_oracle.c) is built with gcc and the sanitizers
  and driven through each of its functions (tests/sanitize/oracle_driver.c).

Any sanitizer report aborts the program (no recovery), and both drivers
check their own results, so a non-zero exit fails the test.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
       "-fno-sanitize-recover=all"]


def _run(cmd, cwd):
    res = subprocess.run(cmd, cwd=cwd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True,
                         timeout=300)
    return res.returncode, res.stdout


def _need(tool):
    if shutil.which(tool) is None:
        pytest.skip(f"{tool} not available")


def test_host_dispatch_under_sanitizers(tmp_path):
    _need("g++")
    exe = str(tmp_path / "host_checks")
    rc, out = _run(["g++", "-std=c++17", *SAN, "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
                    "-I", os.path.join(ROOT, "include"),
                    "-I", os.path.join(ROOT, "tree_masked_attention_plan_amd", "csrc"),
                    os.path.join(ROOT, "tests", "sanitize", "host_checks.cpp"),
                    os.path.join(ROOT, "tree_masked_attention_plan_amd", "csrc", "tree_attn.cpp"),
                    "-o", exe], str(tmp_path))
    assert rc == 0, out
    rc, out = _run([exe], str(tmp_path))
    assert rc == 0 and "host checks ok" in out, out


def test_oracle_under_sanitizers(tmp_path):
    _need("gcc")
    exe = str(tmp_path / "oracle_driver")
    rc, out = _run(["gcc", "-std=c11", *SAN,
                    os.path.join(ROOT, "tests", "sanitize", "oracle_driver.c"),
                    os.path.join(ROOT, "oracle", "tree_attn_oracle.c"), "-o", exe, "-lm", "-lpthread"],
                   str(tmp_path))
    assert rc == 0, out
    rc, out = _run([exe], str(tmp_path))
    assert rc == 0 and "oracle driver ok" in out, out
