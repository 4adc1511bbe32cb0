"""The CPU oracle built with AddressSanitizer and UndefinedBehaviorSanitizer (gcc,
host code only) and run through a C driver (tests/csrc/oracle_sanitize_main.c):
odd sizes, k = 3, 5, 7, up to five levels, empty tensors, skipped outputs.  The
sanitizers fail the run on any out-of-bounds access, leak or undefined
behaviour; the driver also checks the adjoint identity and the Haar round trip."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_under_address_and_undefined_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_sanitized")
    cmd = ["gcc", "-std=c99", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=undefined", "-ffp-contract=off", "-fopenmp",
           os.path.join(ROOT, "oracle", "wtconv_oracle.c"),
           os.path.join(ROOT, "tests", "csrc", "oracle_sanitize_main.c"), "-lm", "-o", exe]
    subprocess.run(cmd, check=True, capture_output=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1",
               OMP_NUM_THREADS="2")
    res = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "ok" in res.stdout
    assert "ERROR: AddressSanitizer" not in res.stderr and "runtime error" not in res.stderr
