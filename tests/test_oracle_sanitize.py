"""The CPU oracle under AddressSanitizer and UndefinedBehaviorSanitizer.

tests/native/oracle_sanitize_driver.c calls every exported routine of
oracle/tsenor_oracle.c (Dykstra in fp64 and fp32, rounding with and without
the optional stages and their traces, the exact optimum) on small seeded
matrices of every M.  Built with gcc -fsanitize=address,undefined
-fno-sanitize-recover, any invalid access or undefined operation aborts the
run; the same driver without sanitizers must print the same checksum.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ORACLE_SRC = os.path.join(ROOT, "oracle", "tsenor_oracle.c")
DRIVER = os.path.join(ROOT, "tests", "native", "oracle_sanitize_driver.c")


def _build_and_run(tmp_path, name, flags):
    exe = str(tmp_path / name)
    subprocess.check_call(["gcc", "-O1", "-g", "-ffp-contract=off", *flags, "-o", exe, DRIVER,
                           ORACLE_SRC, "-lm"])
    # verify_asan_link_order=0: the environment may preload other libraries
    # ahead of the sanitizer runtime; that is harmless for this driver.
    env = dict(os.environ,
               ASAN_OPTIONS="detect_leaks=1:abort_on_error=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    return r.stdout.strip()


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_clean_under_asan_ubsan(tmp_path):
    plain = _build_and_run(tmp_path, "plain", [])
    san = _build_and_run(tmp_path, "san", ["-fsanitize=address,undefined",
                                           "-fno-sanitize-recover=all",
                                           "-fno-omit-frame-pointer"])
    assert plain.startswith("checksum") and "failures 0" in plain
    assert san == plain
