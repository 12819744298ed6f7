"""The host side of the C ABI (plan and argument checks) under
AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU.

fsa_plan.cpp and fsa_api.cpp are plain C++; g++ builds them with
-fsanitize=address,undefined (no recovery) against stub launchers
(tests/host/stub_launchers.cpp) into a shared library. A child Python, with
the ASan runtime preloaded, then runs the plan tests (bit-exact against the
oracle, including the hypothesis sweep) and every ABI rejection test against
that library instead of libfsa.so. Any sanitizer report aborts the child.
"""
import os
import shutil
import subprocess
import sys

import pytest

from tests.conftest import ROOT

CSRC = os.path.join(ROOT, "frame_windowed_block_amd", "csrc")
STUBS = os.path.join(ROOT, "tests", "host", "stub_launchers.cpp")

CHILD = r"""
import sys
sys.path.insert(0, {root!r})
from frame_windowed_block_amd import _abi
_abi.LIB_PATH = {lib!r}
import pytest
sys.exit(pytest.main(["-q", "-p", "no:cacheprovider", "--noconftest",
                      "tests/test_plan.py", "tests/test_abi.py"]))
"""


@pytest.mark.slow
def test_plan_and_abi_checks_under_asan_ubsan(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not found")
    lib = str(tmp_path / "libfsa_host_sanitized.so")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fPIC", "-shared",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-I", os.path.join(ROOT, "include"),
           os.path.join(CSRC, "fsa_plan.cpp"), os.path.join(CSRC, "fsa_api.cpp"), STUBS, "-o", lib]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    asan = subprocess.run([gxx, "-print-file-name=libasan.so"], capture_output=True,
                          text=True).stdout.strip()
    assert os.path.isabs(asan) and os.path.exists(asan), asan
    env = dict(os.environ)
    env["LD_PRELOAD"] = asan
    # the interpreter itself is not instrumented: its allocations at exit are
    # not this library's leaks
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    env["PYTHONPATH"] = ROOT
    r = subprocess.run([sys.executable, "-c", CHILD.format(root=ROOT, lib=lib)], cwd=ROOT, env=env,
                       capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    assert "ERROR: AddressSanitizer" not in out, out[-4000:]
    assert "runtime error:" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in r.stdout, out[-2000:]
    print(r.stdout.strip().splitlines()[-1])
