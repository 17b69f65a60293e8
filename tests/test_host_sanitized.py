"""The host chooser and index math built with g++ under the address and
undefined-behaviour sanitizers (CPU only, no GPU code), driven over a fixed
pseudo-random sweep of valid and invalid inputs, and compared call by call
with the independent Python mirror in oracle.plan."""
import os
import shutil
import subprocess
import tempfile

import pytest

from oracle import plan as mirror

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "absorbed_mla_paged_amd", "csrc")


@pytest.fixture(scope="module")
def driver_output():
    gxx = shutil.which("g++")
    if gxx is None or not os.path.exists("/opt/rocm/include/hip/hip_runtime_api.h"):
        pytest.skip("g++ or the HIP runtime headers are missing")
    with tempfile.TemporaryDirectory() as tmp:
        exe = os.path.join(tmp, "plan_driver")
        cmd = [gxx, "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined",
               "-fno-sanitize-recover=all", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
               "-I", os.path.join(ROOT, "include"), "-I", CSRC,
               os.path.join(CSRC, "plan.cpp"), os.path.join(ROOT, "tests", "host", "plan_driver.cpp"),
               "-o", exe]
        res = subprocess.run(cmd, capture_output=True, text=True)
        assert res.returncode == 0, res.stderr[-4000:]
        env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
                   UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
        run = subprocess.run([exe, "3000"], capture_output=True, text=True, env=env, timeout=300)
        assert run.returncode == 0, run.stderr[-4000:]
        assert "runtime error" not in run.stderr, run.stderr[-4000:]
        return run.stdout.splitlines()


def _ints(s):
    return [int(x) for x in s.split()]


def test_chooser_under_sanitizers_matches_mirror(driver_output):
    plans = [l for l in driver_output if l.startswith("plan ")]
    assert len(plans) == 3000
    ok = 0
    for line in plans:
        parts = [x.strip() for x in line[len("plan "):].split("|")]
        batch, heads, q_len, bs = _ints(parts[0])
        ctx = _ints(parts[1])
        num_cus, hpw, tile, wpc, fp, fs, limit = _ints(parts[2])
        status = int(parts[3])
        prm = mirror.PlanParams(num_cus=num_cus or 256, heads_per_wg=hpw, min_tile_blocks=tile,
                                wgs_per_cu=wpc, force_partitions=fp, force_splits=fs,
                                workspace_limit_bytes=limit)
        try:
            ref = mirror.choose_partitions(batch, heads, q_len, ctx, prm, block_size=bs)
        except ValueError:
            ref = None
        assert (ref is None) == (status != 0), line
        if ref is None:
            continue
        ok += 1
        ps = [tuple(int(v) for v in x.split("/")) for x in parts[4].split()]
        assert [p for p, _ in ps] == ref["P"] and [s for _, s in ps] == ref["S"], line
        assert _ints(parts[5]) == ref["row_indptr"], line
        rows, maxr, hpw_o, groups, tile_o, needs, pob, plb = _ints(parts[6])
        assert (rows, maxr, hpw_o, groups, tile_o, needs) == (
            ref["total_rows"], ref["max_rows_per_req"], ref["heads_per_wg"], ref["groups"],
            ref["tile_blocks"], ref["needs_reduce"]), line
        assert pob + plb == ref["workspace_bytes"], line
    assert ok > 500   # most draws are valid plans


def test_index_math_under_sanitizers_matches_mirror(driver_output):
    ranges = [l for l in driver_output if l.startswith("range ")]
    assert len(ranges) == 3000
    for line in ranges:
        a, st, r = [x.strip() for x in line[len("range "):].split("|")]
        c, bs, P, S, p, s = _ints(a)
        valid = (c >= 0 and bs in (16, 32) and P >= 1 and S >= 1 and 0 <= p < P and 0 <= s < S)
        assert (int(st) == 0) == valid, line
        if valid:
            assert tuple(_ints(r)) == mirror.partition_range(c, P, S, p, s, bs), line
