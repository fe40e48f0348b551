"""The host-side API tests (tests/test_api.py) again, against a copy of the library whose
host code is built with AddressSanitizer and UndefinedBehaviorSanitizer (device code
unchanged; no GPU needed). Any out-of-bounds access, use after free or undefined
behaviour in argument validation and dispatch aborts the run."""
import os
import subprocess
import sys
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parents[1]
sys.path.insert(0, str(ROOT / "linear_recurrent_sequence_rn_amd"))


def test_api_tests_pass_under_asan_and_ubsan(tmp_path):
    import build
    if not Path(build.HIPCC).exists():
        pytest.skip("hipcc not available")
    lib = build.build(sanitize=True, lib=tmp_path / "librn_retention.so")
    out = subprocess.run(["nm", "-D", str(lib)], capture_output=True, text=True).stdout
    assert "__asan_report" in out and "__ubsan_handle" in out, "sanitizers not compiled in"
    rt = build.sanitizer_runtime()
    assert Path(rt).exists(), rt
    env = dict(os.environ, RN_LIB_PATH=str(lib), LD_PRELOAD=rt,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        "-m", "not gpu", "tests/test_api.py"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    tail = (r.stdout[-3000:] + r.stderr[-3000:])
    assert r.returncode == 0, tail
    assert " passed" in r.stdout and "failed" not in r.stdout, tail
