"""The host split planner under the host compiler's address and
undefined-behaviour checks, on randomized inputs (CPU only).

tests/plan_fuzz.cpp drives mla::build_plan directly with random batches,
lengths (short, long, mixed, up to 2^24), query shapes, page sizes and CU
counts, and checks every schedule's invariants and its size against the room
a plan reserves for in-place updates; refused arguments must be refused with a
message.  Built with g++ (no GPU code involved)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "decode_attention_absorbed_amd", "csrc")


@pytest.fixture(scope="module")
def fuzz_bin(tmp_path_factory):
    gxx = shutil.which("g++")
    if not gxx:
        pytest.skip("g++ not available")
    out = str(tmp_path_factory.mktemp("plan_fuzz") / "plan_fuzz")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-I", CSRC, os.path.join(CSRC, "plan.cpp"), os.path.join(ROOT, "tests", "plan_fuzz.cpp"), "-o", out]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-3000:]
    return out


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_random_plans_hold_their_invariants(fuzz_bin, seed):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    res = subprocess.run([fuzz_bin, "400", str(seed)], capture_output=True, text=True, env=env, timeout=300)
    print(res.stdout, res.stderr[-2000:])
    assert res.returncode == 0, res.stderr[-3000:]
    assert res.stdout.startswith("ok:")
