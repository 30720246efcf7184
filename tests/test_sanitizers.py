"""The C oracle and the C input generator built with AddressSanitizer and
UndefinedBehaviorSanitizer (host code only, gcc), driven through every entry
point on small shapes by tests/sanitize_driver.c. Any out-of-bounds access,
use after free, leak or undefined operation in either makes the run fail."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_and_generator_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "sanitize_driver")
    srcs = [os.path.join(ROOT, "tests", "sanitize_driver.c"),
            os.path.join(ROOT, "oracle", "oracle.c"),
            os.path.join(ROOT, "synth", "gen.c")]
    cmd = ["gcc", "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer", "-fopenmp",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", *srcs, "-o", exe, "-lm"]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    env = dict(os.environ)
    env["ASAN_OPTIONS"] = "detect_leaks=1:abort_on_error=0:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    env["OMP_NUM_THREADS"] = "2"
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    assert "ran clean" in r.stdout
