"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

api.cpp and plan.cpp are compiled for the host alone with both sanitizers, the kernel launches
replaced by stand-ins that report no device (tests/sanitize/launch_stubs.cpp), and
tests/test_abi.py runs against that library in a child process with the sanitizer runtime
preloaded. Any report (a heap or stack overflow, a use after free, undefined behaviour) fails the
test."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "delta_rule_linear_chunked_amd", "csrc")
HIPCC = "/opt/rocm/bin/hipcc"
# host-side sanitizers only (no device code is compiled)
SAN = "-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined -Xarch_host -fno-sanitize-recover=undefined".split()


def _runtime():
    r = subprocess.run([HIPCC, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = r.stdout.strip()
    return path if r.returncode == 0 and os.path.isabs(path) and os.path.exists(path) else None


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc is not installed")
def test_abi_under_sanitizers(tmp_path):
    rt = _runtime()
    if rt is None:
        pytest.skip("no AddressSanitizer runtime next to hipcc")
    objs = []
    for src in (os.path.join(CSRC, "api.cpp"), os.path.join(CSRC, "plan.cpp"),
                os.path.join(ROOT, "tests", "sanitize", "launch_stubs.cpp")):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        cmd = [HIPCC, "-x", "hip", "--offload-host-only", "-O1", "-g", "-fPIC", "-std=c++17",
               "-fno-omit-frame-pointer", *SAN, "-I", os.path.join(ROOT, "include"), "-c", src, "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-3000:]
        objs.append(obj)
    lib = str(tmp_path / "libdeltarule_sanitized.so")
    r = subprocess.run([HIPCC, "-shared", "-fPIC", *SAN, *objs, "-o", lib], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, DELTARULE_LIBRARY=lib, LD_PRELOAD=rt,
               ASAN_OPTIONS="detect_leaks=0:verify_asan_link_order=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
                        os.path.join(ROOT, "tests", "test_abi.py")], capture_output=True, text=True, env=env,
                       cwd=ROOT, timeout=600)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in out
