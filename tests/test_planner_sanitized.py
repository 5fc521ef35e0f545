"""The planner (pure host code) under AddressSanitizer and
UndefinedBehaviorSanitizer: planner_fuzz.cpp draws random parameters and page
tables, valid and invalid, runs build_host_plan / block_table_csr on them and
checks every accepted plan's units against what the decode kernel relies on
(the units of each request and kv head tile its attended tokens in chunk
order, workspace slots are distinct, fields in range); every rejection must
leave a message. Built with g++ (host code only, no GPU)."""
import shutil
import subprocess
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parents[1]


@pytest.fixture(scope="module")
def fuzz_bin(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not found")
    out = tmp_path_factory.mktemp("planner_fuzz") / "planner_fuzz"
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-I", str(ROOT / "include"),
           "-I", str(ROOT / "paged_kv_decode_09_amd" / "csrc"),
           str(ROOT / "tests" / "planner_fuzz.cpp"),
           str(ROOT / "paged_kv_decode_09_amd" / "csrc" / "planner.cpp"), "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    if r.returncode != 0 and "sanitize" in r.stderr and "not supported" in r.stderr:
        pytest.skip("sanitizers not supported by this g++")
    assert r.returncode == 0, r.stderr[-2000:]
    return out


@pytest.mark.parametrize("seed", [1, 2])
def test_planner_fuzz_under_sanitizers(fuzz_bin, seed):
    r = subprocess.run([str(fuzz_bin), "1000", str(seed)], capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 0, (r.stdout + r.stderr)[-3000:]
    ok, plans, rejected = r.stdout.split()
    assert ok == "ok" and int(plans) > 300 and int(rejected) > 100
