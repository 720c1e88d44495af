"""The C-ABI layer (api.cpp) built for the host alone with AddressSanitizer
and UndefinedBehaviorSanitizer, no recovery, and driven through every entry
point with fixed cases and a seeded sweep of edge values
(tests/host_sanitize/abi_driver.cpp).  Stubs stand in for the kernel
launchers and check what the validated layer hands them; nothing touches a
GPU.  Catches out-of-bounds host accesses, signed overflow in the
validation arithmetic, and calls that launch although they fail."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "host_sanitize")
CSRC = os.path.join(ROOT, "yarn_rope_blockwise_amd", "csrc")


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_abi_layer_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "abi_driver")
    # host compiler only: the stand-in HIP header comes first on the path
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-I", HERE, "-I", CSRC,
           os.path.join(CSRC, "api.cpp"), os.path.join(HERE, "launch_stubs.cpp"),
           os.path.join(HERE, "abi_driver.cpp"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    env.pop("LD_PRELOAD", None)
    r = subprocess.run([exe, "200000"], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "0 failures" in r.stdout, r.stdout
