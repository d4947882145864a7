"""Host code of the C ABI under AddressSanitizer and UndefinedBehaviorSanitizer.

Builds the library's host side (argument validation, workspace carving,
sequence tables) with -fsanitize=address,undefined (host code only; the
device code is built as usual and never runs), links tests/abi_check.c against it and runs it: every entry point
is called with valid and invalid arguments and must return its documented
status with no sanitizer report.  Runs only on a host without a GPU, where a
call that passes validation stops at the device check."""
import glob
import os
import shutil
import subprocess

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang"

pytestmark = pytest.mark.skipif(torch.cuda.device_count() > 0 or not os.path.exists(HIPCC)
                                or not os.path.exists(CLANG), reason="needs a host without a GPU and ROCm clang")


def test_abi_validation_under_asan_ubsan(tmp_path):
    srcs = sorted(glob.glob(os.path.join(ROOT, "sdpa_backward_fa2_amd", "csrc", "*.hip")))
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined"]
    objs = []
    procs = []
    for s in srcs:
        o = str(tmp_path / (os.path.basename(s) + ".o"))
        objs.append(o)
        procs.append(subprocess.Popen([HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-fPIC",
                                       "-std=c++17", "-fno-omit-frame-pointer", *san, "-c", s, "-o", o],
                                      stdout=subprocess.PIPE, stderr=subprocess.STDOUT))
    for p in procs:
        out, _ = p.communicate()
        assert p.returncode == 0, out.decode()[-3000:]
    lib = str(tmp_path / "libsdpa_bwd_san.so")
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC",
                    "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined", "-o", lib, *objs],
                   check=True, capture_output=True)
    exe = str(tmp_path / "abi_check")
    subprocess.run([CLANG, "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                    os.path.join(ROOT, "tests", "abi_check.c"), lib, "-o", exe,
                    "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-lstdc++"],
                   check=True, capture_output=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", HIP_VISIBLE_DEVICES="")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    report = r.stdout + r.stderr
    assert r.returncode == 0, report[-4000:]
    assert "runtime error" not in report and "AddressSanitizer" not in report, report[-4000:]
    assert "abi_check: 0 failure(s)" in report
