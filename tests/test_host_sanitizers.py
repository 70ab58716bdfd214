"""The library's host layer (argument validation with its size and extent
arithmetic, the varlen plan builder, the THD planner and its first-position
table) built for the host with AddressSanitizer and UndefinedBehaviorSanitizer
and fuzzed: seeded random calls of every entry point with sizes, strides,
dtype codes and fake device pointers at the edges of their ranges, and random
planner batches, a quarter of them malformed.  Any out-of-bounds access,
signed overflow, division by zero, invalid enum value or leak fails the run.
The launches the validation lets through go to counting stubs; no kernel is
built or run."""

import os
import shutil
import subprocess
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parents[1]
CSRC = ROOT / "context_attention_movement_amd" / "csrc"
HERE = Path(__file__).resolve().parent / "host_sanitize"


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    exe = tmp_path_factory.mktemp("host_sanitize") / "driver"
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-ffp-contract=off", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-I", str(ROOT / "include"), "-I", str(CSRC),
           str(CSRC / "cam_api.cpp"), str(CSRC / "thd_planner.cpp"), str(HERE / "stubs.cpp"), str(HERE / "driver.cpp"),
           "-o", str(exe)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0 and "sanitize" in res.stderr and "unrecognized" in res.stderr:
        pytest.skip("the host compiler has no sanitizers")
    assert res.returncode == 0, res.stderr[-3000:]
    return exe


@pytest.mark.parametrize("seed", [1, 2])
def test_host_layer_under_sanitizers(driver, seed):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1", UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    res = subprocess.run([str(driver), str(seed), "200000", "4000"], capture_output=True, text=True, env=env,
                         timeout=600)
    out = res.stdout + res.stderr
    assert res.returncode == 0 and "runtime error" not in out and "ERROR: " not in out, out[-4000:]
    assert "planned" in out
