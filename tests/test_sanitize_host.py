"""The host-only parts of the library under AddressSanitizer and
UndefinedBehaviorSanitizer (CPU only). The scale-overlay reader parses files
from disk, so it gets a seeded mutation run (tests/sanitize/overlay_fuzz.cpp)
built with both sanitizers from the library's own source."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs a host C++ compiler")
def test_scale_overlay_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "overlay_fuzz")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-I" + os.path.join(ROOT, "include"),
           os.path.join(ROOT, "fp8_quantised_paged_amd", "csrc", "scale_overlay.cpp"),
           os.path.join(ROOT, "tests", "sanitize", "overlay_fuzz.cpp"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe, str(tmp_path), "3000"], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, (r.returncode, r.stdout[-2000:], r.stderr[-4000:])
    assert "overlay fuzz:" in r.stdout
