"""Host-only property test of the split-key plan under AddressSanitizer and
UndefinedBehaviorSanitizer.

tests/plan_props.cpp links the library's own planners (canvas_attention_amd/csrc/
dg_plan.cpp) and the unit decode the kernels run (dg_plan.h) into a plain g++
program built with -fsanitize=address,undefined; no device and no HIP runtime are
involved.  Its properties (every key of every (sequence, kv head, row tile)
covered exactly once, unit decode injective and inverted by the merge's
addressing, exact reciprocal divisions over the kernels' numerator ranges, the
workspace within the published bound, the XCD dealing a bijection) are listed in
its header.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "canvas_attention_amd", "csrc")


@pytest.fixture(scope="module")
def plan_props(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    exe = str(tmp_path_factory.mktemp("plan_props") / "plan_props")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-Wall", "-Wextra",
           "-Werror", f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}",
           os.path.join(ROOT, "tests", "plan_props.cpp"), os.path.join(CSRC, "dg_plan.cpp"),
           "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    return exe


@pytest.mark.parametrize("seed", [20261203, 7])
def test_plan_properties_under_sanitizers(plan_props, seed):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([plan_props, "300", str(seed)], capture_output=True, text=True,
                       timeout=600, env=env)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "plan properties: 300 cases" in r.stdout
    assert "runtime error" not in r.stderr, r.stderr
    print(r.stdout.strip())
