"""The C-ABI layer (cpattn.cpp) built for the host with AddressSanitizer and
UndefinedBehaviorSanitizer, its HIP runtime calls and kernel launchers
replaced by host stubs (tests/sanitize/): the C-ABI tests' rejection paths
and every call's success path with large sizes run under both sanitizers,
in a child process that preloads their runtimes.  Needs no GPU."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")


def _runtime(name):
    path = subprocess.run(["g++", f"-print-file-name={name}"], capture_output=True,
                          text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def test_host_layer_under_asan_and_ubsan(tmp_path):
    if shutil.which("g++") is None:
        pytest.skip("no host C++ compiler")
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if not asan or not ubsan:
        pytest.skip("sanitizer runtimes not installed")
    lib = str(tmp_path / "libcpattn_san.so")
    build = ["g++", "-std=c++17", "-g", "-O1", "-fPIC", "-shared", "-fno-omit-frame-pointer",
             "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
             "-I", SAN, "-I", os.path.join(ROOT, "include"),
             "-I", os.path.join(ROOT, "sequence_attention_cpa_amd", "csrc"),
             os.path.join(ROOT, "sequence_attention_cpa_amd", "csrc", "cpattn.cpp"),
             os.path.join(SAN, "stub_runtime.cpp"), "-o", lib]
    r = subprocess.run(build, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, LD_PRELOAD=f"{asan} {ubsan}",
               ASAN_OPTIONS="detect_leaks=0:verify_asan_link_order=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([sys.executable, os.path.join(SAN, "run_abi_tests.py"), lib], env=env,
                       capture_output=True, text=True, timeout=300)
    out = r.stdout[-3000:] + r.stderr[-3000:]
    assert r.returncode == 0, out
    assert "passed" in r.stdout and "success paths" in r.stdout, out
    assert "runtime error" not in out and "AddressSanitizer" not in out, out
