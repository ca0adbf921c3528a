"""Host-side checks of device helpers that decide which data a block works
on, compiled from the library's own header with hipcc and run on the CPU
(no GPU call is made)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"

PROG = r"""
#include <cstdio>
#include <vector>
#include "ldv_device.hpp"
// Every hardware block maps to exactly one logical block, also when the
// grid is not a whole number of units (the kernels pass units = grid / per),
// and below the tail the blocks of one unit share the XCD (hardware block i
// runs on XCD i % 8).
int main() {
    long bad = 0, cases = 0;
    for (unsigned units = 1; units <= 400; ++units)
        for (unsigned per = 1; per <= 8; ++per)
        for (unsigned rest = 0; rest < per; ++rest) {
            const unsigned n = units * per + rest, full = (units / 8) * 8 * per;
            std::vector<int> seen(n, 0);
            std::vector<int> xcd(units, -1);
            for (unsigned b = 0; b < n; ++b) {
                const unsigned l = ldv::xcd_spread(b, units, per);
                if (l >= n) { ++bad; continue; }
                ++seen[l];
                if (b < full) {
                    const unsigned u = l / per;
                    if (xcd[u] < 0) xcd[u] = (int)(b % 8);
                    else if (xcd[u] != (int)(b % 8)) ++bad;
                }
            }
            for (unsigned l = 0; l < n; ++l) bad += seen[l] != 1;
            ++cases;
        }
    std::printf("%ld cases, %ld bad\n", cases, bad);
    return bad != 0;
}
"""


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
def test_xcd_spread_is_a_bijection(tmp_path):
    src = tmp_path / "spread.hip"
    src.write_text(PROG)
    exe = tmp_path / "spread"
    inc = os.path.join(ROOT, "speculative_decoding_verify_amd", "csrc")
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-O1", "-std=c++17", "-I", inc, "-I",
                    os.path.join(ROOT, "include"), str(src), "-o", str(exe)], check=True, capture_output=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.strip().endswith(" 0 bad"), r.stdout


def test_bench_algorithmic_bytes():
    """bench.py's algorithmic verify bytes: per head the state (64 KiB at
    d = 128) and, per node, bf16 q/k/v (768) and the gates (8) read, fp32 o
    and u (1024) and log P (4) written: 79,968 bytes per head for a chain of
    8.  A chain longer than 64 nodes reads one base state per chunk and
    writes one per chunk but the last.  Commit reads and writes the state of
    each committing head and reads the path's u, k and log P."""
    import numpy as np

    import bench
    from workloads import LONG_WORKLOADS, WORKLOADS, make_inputs
    wl = WORKLOADS["gdn1.3b-chain"].replace(B=2, H=3)
    x = make_inputs(wl, with_gather=False)
    alg, _ = bench.algorithmic(wl, x)
    rd, wr = alg["verify"]
    assert (rd, wr) == (2 * 3 * (65536 + 8 * 776), 2 * 3 * 8 * 1028) and rd + wr == 2 * 3 * 79968
    x["accepted"] = np.array([3, -1], np.int32)  # one sequence commits node 3 (a path of 4 nodes)
    alg, _ = bench.algorithmic(wl, x)
    assert alg["commit"] == (3 * (65536 + 4 * (512 + 256 + 4)) + 2 * 4, 3 * 65536)
    wl = LONG_WORKLOADS["gdn1.3b-chain1024"].replace(B=1, H=2, T=130)  # three chunks
    rd, wr = bench.algorithmic(wl, make_inputs(wl, with_gather=False))[0]["verify"]
    assert rd + wr == 2 * (5 * 65536 + 130 * 1804) and rd == 2 * (3 * 65536 + 130 * 776)


def test_bench_ceiling_choice():
    """Each kernel is graded against the best stream probe at its read:write
    ratio or a more write-heavy one; an in-place commit against the in-place
    probe."""
    import bench
    peaks = {"read_GB_s": 7.0, "copy_GB_s": 6.0, "rmw_GB_s": 6.2, "read2write1_GB_s": 6.1,
             "read4write1_GB_s": 6.5, "read8write1_GB_s": 6.3}
    assert bench.ceiling_for(10, 10, True, peaks) == ("rmw_GB_s", 6.2)
    assert bench.ceiling_for(10, 10, False, peaks) == ("rmw_GB_s", 6.2)
    assert bench.ceiling_for(15, 10, False, peaks) == ("rmw_GB_s", 6.2)          # 1.5:1: the 1:1 probes only
    assert bench.ceiling_for(77952, 16448, False, peaks) == ("read4write1_GB_s", 6.5)   # 27B-hybrid verify, 4.7:1
    assert bench.ceiling_for(69632, 8192, False, peaks) == ("read4write1_GB_s", 6.5)    # gather, 8.5:1
    assert bench.ceiling_for(1000, 1, False, peaks) == ("read_GB_s", 7.0)               # 1000:1: reads only
    assert bench.ceiling_for(1000, 0, False, peaks) == ("read_GB_s", 7.0)
    assert bench.ceiling_for(1, 2, False, peaks) == ("copy_GB_s", 6.0)                  # more writes than reads
    assert bench.ceiling_for(1, 1, False, None) == (None, None)
