"""The CPU oracle built with AddressSanitizer and UndefinedBehaviorSanitizer
(host code, gcc) and driven over every entry point on small ragged shapes
with exactly sized buffers: any out-of-bounds access, use after free, leak,
signed overflow or bad shift fails the test."""
import os
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRCS = [os.path.join(ROOT, "oracle", "oracle.c"), os.path.join(ROOT, "oracle", "kvcache.c"),
        os.path.join(ROOT, "tests", "sanitize", "oracle_driver.c")]


def test_oracle_under_address_and_undefined_behaviour_sanitizers():
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    d = tempfile.mkdtemp()
    exe = os.path.join(d, "oracle_driver")
    flags = ["-O1", "-g", "-std=c11", "-ffp-contract=off", "-frounding-math", "-fno-omit-frame-pointer",
             "-fsanitize=address,undefined", "-fno-sanitize-recover=all"]
    subprocess.run([gcc, *flags, "-o", exe, *SRCS, "-lm"], check=True, capture_output=True, text=True)
    # verify_asan_link_order=0: a library the environment preloads may come
    # before the sanitizer runtime; that does not affect these checks
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0:exitcode=23",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    assert r.returncode == 0, r.stderr[-4000:]
    assert "ran clean" in r.stdout
    shutil.rmtree(d, ignore_errors=True)
