"""The host side of the C ABI under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

A host-only build of the library (no device code; linear_cross_entropy_vocab_amd.build.
build_host_sanitized) is loaded in a fresh Python process with the sanitizer runtime preloaded,
and the ABI and binding tests run against it: every argument check, workspace size and plan
computation, and the rejection of bad calls before any device work.  Any sanitizer report
fails the run."""

import glob
import os
import shutil
import subprocess
import sys

import pytest

from linear_cross_entropy_vocab_amd import build as lbuild

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


def test_abi_host_code_under_asan_and_ubsan(tmp_path):
    if shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"):
        pytest.skip("hipcc not available")
    try:
        rt = lbuild.sanitizer_runtime()
    except RuntimeError as e:
        pytest.skip(str(e))
    lib = lbuild.build_host_sanitized()
    logs = str(tmp_path / "san")
    env = dict(os.environ, LCE_LIBRARY=lib, LD_PRELOAD=rt,
               ASAN_OPTIONS=f"detect_leaks=0:halt_on_error=1:log_path={logs}",
               UBSAN_OPTIONS=f"halt_on_error=1:print_stacktrace=1:log_path={logs}")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(HERE, "test_abi.py"), os.path.join(HERE, "test_binding_checks.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    reports = "".join(open(f).read() for f in glob.glob(logs + "*"))
    assert r.returncode == 0 and not reports, (r.stdout[-3000:], r.stderr[-3000:], reports[:5000])
