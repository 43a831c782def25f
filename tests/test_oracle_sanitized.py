"""The oracle under sanitizers (CPU): an AddressSanitizer + UBSan executable
that calls every oracle function on edge cases, and the whole pin suite run
against a UBSan build of the oracle library (every report fatal)."""

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

pytestmark = pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")


@pytest.fixture(scope="module")
def sanitized():
    from oracle import build
    build.build(sanitize=True)
    return build


def test_oracle_functions_under_address_and_ub_sanitizers(sanitized):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    p = subprocess.run([sanitized.CHECK_EXE], stdout=subprocess.PIPE, stderr=subprocess.STDOUT, env=env,
                       timeout=300)
    out = p.stdout.decode(errors="replace")
    assert p.returncode == 0 and "oracle sanitizer run: ok" in out, out[-3000:]


def test_oracle_pins_pass_on_the_ubsan_build(sanitized):
    env = dict(os.environ, PLE_ORACLE_LIB=sanitized.UBSAN_LIB, UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    check = subprocess.run([sys.executable, "-c", "import oracle, sys; sys.exit(0 if oracle.LIB.endswith("
                            "'libple_oracle_ubsan.so') and oracle.mix64(1) != 0 else 1)"], cwd=ROOT, env=env, timeout=120)
    assert check.returncode == 0
    p = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, timeout=900)
    out = p.stdout.decode(errors="replace")
    assert p.returncode == 0, out[-3000:]
    assert "runtime error" not in out, out[-3000:]
