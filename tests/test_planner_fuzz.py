"""The planner's C ABI under AddressSanitizer and UBSan (host only).

tests/native/planner_fuzz.cpp feeds fg_plan_pass random pass descriptions:
half of them valid (every one must be accepted and give a consistent plan),
half with invalid fields (sizes, head layouts, block ids, null pointers,
knobs), which must be rejected with a status.  The planner source is built
with g++ and the sanitizers, so any out-of-bounds access, leak or
undefined behaviour ends the run with an error.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "ragged_paged_attention_splitfuse_amd", "csrc")
DRIVER = os.path.join(ROOT, "tests", "native", "planner_fuzz.cpp")


@pytest.fixture(scope="module")
def fuzz_binary(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    exe = str(tmp_path_factory.mktemp("planner_fuzz") / "planner_fuzz")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-Wall", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=undefined", f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}",
           os.path.join(CSRC, "plan.cpp"), DRIVER, "-o", exe]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stdout + res.stderr
    return exe


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_planner_fuzz_under_sanitizers(fuzz_binary, seed):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    res = subprocess.run([fuzz_binary, str(seed), "1200"], capture_output=True, text=True,
                         timeout=240, env=env)
    assert res.returncode == 0, (res.stdout + res.stderr)[-4000:]
    assert "plans accepted" in res.stdout
    assert "runtime error" not in res.stderr and "AddressSanitizer" not in res.stderr
