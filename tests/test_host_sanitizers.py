"""The C ABI layer (csrc/api.cpp, compiled unchanged) under AddressSanitizer
and UndefinedBehaviorSanitizer on the host: tests/hostcheck/driver.cpp calls
every entry point with valid and invalid arguments and checks the statuses
and what reaches the (recording, host-only) launchers of stubs.cpp.  The
sanitizers apply to host code only (each -fsanitize is passed through
-Xarch_host, and the objects are built host-only); no GPU is used."""

import os
import shutil
import subprocess
import tempfile

import pytest

from conftest import ROOT

HERE = os.path.join(ROOT, "tests", "hostcheck")
CSRC = os.path.join(ROOT, "draft_sampling_verification_bias_amd", "csrc")


def _hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    pytest.skip("hipcc not available")


def test_c_abi_under_address_and_undefined_behaviour_sanitizers():
    hipcc = _hipcc()
    san = []
    for flag in ("-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"):
        san += ["-Xarch_host", flag]
    inc = ["-I" + os.path.join(ROOT, "include"), "-I" + CSRC, "-I" + HERE]
    with tempfile.TemporaryDirectory() as tmp:
        objs = []
        for src in (os.path.join(CSRC, "api.cpp"), os.path.join(HERE, "stubs.cpp"), os.path.join(HERE, "driver.cpp")):
            obj = os.path.join(tmp, os.path.basename(src) + ".o")
            cmd = [hipcc, "-x", "hip", "--offload-host-only", "-std=c++17", "-O1", "-g"] + inc + san + ["-c", src, "-o", obj]
            res = subprocess.run(cmd, capture_output=True, text=True)
            assert res.returncode == 0, res.stderr
            objs.append(obj)
        exe = os.path.join(tmp, "hostcheck")
        res = subprocess.run([hipcc, "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                              "-o", exe] + objs, capture_output=True, text=True)
        assert res.returncode == 0, res.stderr
        env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
        run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
        assert run.returncode == 0, run.stdout + run.stderr
        assert "host checks passed" in run.stdout
        assert "runtime error" not in run.stderr and "AddressSanitizer" not in run.stderr
