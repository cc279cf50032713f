"""The CPU suite once more against host-sanitized builds: the library (planner,
C-ABI and launch code under AddressSanitizer + UndefinedBehaviorSanitizer;
device code as usual) and the oracle's C code, both loaded through their
path variables with the sanitizer runtime preloaded. Any report ends the run
(halt_on_error), so a clean pass means no out-of-bounds access, use after
free or undefined behaviour on any host path the suite reaches."""
import os
import shutil
import subprocess
import sys

import pytest

import oracle
from tiled_prefill_amd import _build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which(_build.hipcc()) is None and not os.path.exists(_build.hipcc()),
                    reason="hipcc not available")
@pytest.mark.skipif(bool(os.environ.get("ATTN_LIB")), reason="already inside a sanitized run")
def test_cpu_suite_under_host_sanitizers(tmp_path):
    lib = _build.build_sanitized(str(tmp_path))
    ref = oracle.build_sanitized(str(tmp_path))
    env = dict(os.environ, LD_PRELOAD=_build.asan_runtime(), ATTN_LIB=lib, ATTNREF_LIB=ref,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "tests", "-m", "not gpu", "-x", "-q", "-p", "no:cacheprovider",
                        "--ignore", os.path.join("tests", "test_host_sanitizers.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=1200)
    tail = (r.stdout[-4000:] + "\n" + r.stderr[-4000:])
    assert r.returncode == 0, tail
    assert " passed" in r.stdout and "ERROR: AddressSanitizer" not in r.stderr and "runtime error:" not in r.stderr, tail
