"""The host prefix cache under AddressSanitizer and UndefinedBehaviorSanitizer.

tests/pcache_model_check.cpp drives csrc/prefix_cache.cpp (host code only,
built here with g++, no HIP) through random reserve / insert / insert_many /
lookup / release / commit / unreserve operations (and refused calls) against
a reference model, with pools small enough that reservations evict entries,
under both retention policies, and compares every return value and counter
after each operation.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = [os.path.join(ROOT, "tests", "pcache_model_check.cpp"),
       os.path.join(ROOT, "linear_attention_recurrence_decode_amd", "csrc", "prefix_cache.cpp")]

pytestmark = pytest.mark.skipif(shutil.which("g++") is None, reason="no g++")


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    exe = str(tmp_path_factory.mktemp("pcache") / "pcache_model_check")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-omit-frame-pointer",
           "-fno-sanitize-recover=all", "-I", os.path.join(ROOT, "include")] + SRC + ["-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    if r.returncode != 0 and "asan" in (r.stderr + r.stdout).lower():
        pytest.skip("sanitizer runtime not available: " + r.stderr[-300:])
    assert r.returncode == 0, r.stderr
    return exe


@pytest.mark.parametrize("policy", [(0, 0), (1, 0), (1, 5)], ids=["keep_all", "second_hit", "second_hit_ghosts5"])
@pytest.mark.parametrize("unit", [1, 4, 16, 64])
@pytest.mark.parametrize("slots", [8, 24, 64])
def test_model_check_under_sanitizers(checker, unit, slots, policy):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    for seed in (1, 2, 3):
        args = [checker, str(seed), "3000", str(unit), str(slots), str(policy[0]), str(policy[1])]
        r = subprocess.run(args, capture_output=True, text=True, timeout=300, env=env)
        assert r.returncode == 0 and r.stdout.strip() == "ok 3000", (args, r.stdout[-500:], r.stderr[-2000:])
