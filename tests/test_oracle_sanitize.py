"""The oracle under AddressSanitizer and UndefinedBehaviorSanitizer (host code).

oracle/sanitize_driver.c calls every oracle function on small, ragged inputs
(all pooled modes, both visiting orders, per-head and shared masks, pyramid
levels, all token orders); built here with the sanitizers, it must exit
cleanly: no out-of-bounds access, use after free, leak or undefined
arithmetic anywhere in the fp64 reference.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ORACLE = os.path.join(ROOT, "oracle")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_clean_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_sanitized")
    cmd = ["gcc", "-O1", "-g", "-fno-omit-frame-pointer", "-fopenmp", "-ffp-contract=off",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           os.path.join(ORACLE, "bsa_oracle.c"), os.path.join(ORACLE, "sanitize_driver.c"),
           "-o", exe, "-lm"]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    env = dict(os.environ, OMP_NUM_THREADS="4",
               ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:exitcode=23:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1:exitcode=24")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    assert "sanitized oracle run ok" in r.stdout
