"""The CPU oracle and the seeded input generator under AddressSanitizer and UndefinedBehaviorSanitizer.

tests/sanitize/oracle_synth_check.c compiles oracle/oracle.c and synth/synth.c into one program with gcc
(-fsanitize=address,undefined, no recovery) and drives every entry point on tiny models (F32 tied; bf16
untied with the llama3 rope), ragged generator spans and the error paths; any out-of-bounds access, leak,
overflow or other undefined behaviour ends it with a report, as does a failed identity check.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "sanitize", "oracle_synth_check.c")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_and_generator_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_synth_check")
    cmd = ["gcc", "-O1", "-g", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-o", exe, SRC, "-lm"]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    # verify_asan_link_order=0: the environment may preload a library ahead of the sanitizer runtime
    env = dict(os.environ, ASAN_OPTIONS="halt_on_error=1:detect_leaks=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "checks passed" in r.stdout
