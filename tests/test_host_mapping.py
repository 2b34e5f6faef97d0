"""Host-side checks of the workgroup -> work-item map that the grouped prefill and rotation
launches use (csrc/m3_mapping.h, compiled here with the host compiler, no GPU).

The map must be a permutation of the grid's items: every (b, h, segment) item runs exactly once.
It also reorders the items, so the segments of one sequence are not dispatched in order: no
segment of a split prefill's pass may rely on segment 0 starting before the last segment ends
(why no segment of a pass writes h_out or phi_out while segment 0 of the same pass may still
read h_in or phi_in from the same buffer: h_out comes from the chaining kernel between the
passes, and every segment takes its start angle from the angle pass)."""
from __future__ import annotations

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "state_space_sequence_m3_amd", "csrc")

PROGRAM = r"""
#include <cstdio>
#include <vector>
#include "m3_mapping.h"
int main() {
    // permutation check for every grid size up to 4096
    for (long n = 1; n <= 4096; ++n) {
        std::vector<int> seen(n, 0);
        for (long i = 0; i < n; ++i) {
            const long it = (long)m3::xcd_item(i, n);
            if (it < 0 || it >= n || seen[it]++) { std::printf("BAD %ld %ld\n", n, i); return 1; }
        }
    }
    // 100 (b, h) pairs in 6 segments (pass 1 of a split sequence): the blocks that run segment 0
    // and the last segment of pair 12
    const long n = 600, segs = 6, bh = 12;
    long first = -1, last = -1;
    for (long i = 0; i < n; ++i) {
        const long it = (long)m3::xcd_item(i, n);
        if (it == bh * segs) first = i;
        if (it == bh * segs + segs - 1) last = i;
    }
    std::printf("%ld %ld\n", first, last);
    // head groups: the slot of each head
    std::printf("%d %d %d %d\n", m3::bc_slot(0, 8, 2), m3::bc_slot(3, 8, 2), m3::bc_slot(4, 8, 2),
                m3::bc_slot(7, 8, 0));
    return 0;
}
"""


@pytest.fixture(scope="module")
def mapping_output(tmp_path_factory):
    cxx = shutil.which("g++")
    if cxx is None:
        pytest.skip("no host C++ compiler")
    d = tmp_path_factory.mktemp("mapping")
    src = d / "mapping.cpp"
    src.write_text(PROGRAM)
    exe = d / "mapping"
    subprocess.run([cxx, "-std=c++17", "-O1", "-I", CSRC, str(src), "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True)
    assert out.returncode == 0, out.stdout + out.stderr
    return out.stdout.split("\n")


def test_xcd_item_is_a_permutation(mapping_output):
    assert not any(line.startswith("BAD") for line in mapping_output)


def test_xcd_item_reorders_segments(mapping_output):
    first, last = map(int, mapping_output[0].split())
    # pair 12's last segment runs in block 17, its segment 0 in block 576: past the 512
    # workgroups the GPU holds at once, so it may start after the last segment has finished
    assert (first, last) == (576, 17)


def test_bc_slot(mapping_output):
    assert mapping_output[1].split() == ["0", "0", "1", "7"]
