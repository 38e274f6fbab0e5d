"""The library's plain C++ parts under the address and undefined-behaviour
sanitizers, on the CPU: the arena allocator, the plane-paging residency
bookkeeping (shared with the pager through csrc/residency.hpp), the planners
and the exponent encoder, driven by a fuzz driver (tests/host/sanitize_driver.cpp)
built with g++ from the same sources the library is built from."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "any_precision_quantized_amd", "csrc")
SOURCES = [os.path.join(ROOT, "tests", "host", "sanitize_driver.cpp")] + \
    [os.path.join(CSRC, f) for f in ("planner.cpp", "exp_encode.cpp", "arena.cpp")]


@pytest.mark.timeout(300)
def test_host_code_clean_under_sanitizers(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not found")
    exe = str(tmp_path / "sanitize_driver")
    build = [gxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
             "-fno-sanitize-recover=all", f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}", *SOURCES, "-o", exe]
    r = subprocess.run(build, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=240)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "ERROR: AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert "clean" in r.stdout
