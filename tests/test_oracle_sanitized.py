"""The CPU oracle (oracle/dg_oracle.c) under AddressSanitizer and
UndefinedBehaviorSanitizer: tests/oracle_sanitized.c calls every entry point on
small edge-case shapes with exactly sized buffers (the cases are listed in its
header).  The oracle is test infrastructure; this checks its memory safety and
basic consistency, its values are pinned by the other test_oracle_* modules."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_oracle_under_sanitizers(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    exe = str(tmp_path / "oracle_sanitized")
    cmd = [gcc, "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer", "-fopenmp",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-Wall", "-Wextra",
           "-Werror", os.path.join(ROOT, "tests", "oracle_sanitized.c"),
           os.path.join(ROOT, "oracle", "dg_oracle.c"), "-lm", "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    env = dict(os.environ, OMP_NUM_THREADS="2", ASAN_OPTIONS="detect_leaks=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "oracle under sanitizers" in r.stdout
    assert "runtime error" not in r.stderr, r.stderr
    print(r.stdout.strip())
