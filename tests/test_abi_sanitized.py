"""The C-ABI checks of tests/test_abi.py, run on the CPU against a copy of the library
whose host-side argument checking (fwmem_api.cpp) is built with AddressSanitizer and
UndefinedBehaviorSanitizer (errors halt the run). No GPU call is made."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_checks_are_clean_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    from linear_attention_scan_amd import build as B
    if not os.path.exists(B.HIPCC):
        pytest.skip("hipcc not found")
    runtime = B.asan_runtime()
    if not runtime:
        pytest.skip("the ROCm clang AddressSanitizer runtime is not installed")
    lib = B.build_sanitized()
    log = tmp_path / "san"
    env = dict(os.environ, FWMEM_LIB=lib, LD_PRELOAD=runtime,
               ASAN_OPTIONS=f"detect_leaks=0:halt_on_error=1:log_path={log}",
               UBSAN_OPTIONS=f"halt_on_error=1:print_stacktrace=1:log_path={log}")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    reports = "".join(p.read_text() for p in tmp_path.glob("san*"))
    assert r.returncode == 0 and not reports, f"{r.stdout[-3000:]}\n{r.stderr[-2000:]}\n{reports[:4000]}"
    assert " passed" in r.stdout
