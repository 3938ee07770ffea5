"""CPU checks of the attention kernel's chip schedule, on the same source the
kernels compile: `sched_check.cpp` includes `attn_sched.h` in a host build
and sweeps the tile orders, the frame-window key ranges and the split of the
last partial round of tiles (see its header). The split's partial records
must also fit in the workspace the library asks for, which this test checks
against the library's own h3attn_forward_ex_workspace_bytes."""
import os
import shutil
import subprocess

import pytest

from video_dit_dense_amd import h3attn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "video_dit_dense_amd", "csrc")
SRC = os.path.join(ROOT, "tests", "sched_check.cpp")


def record_floats(D):
    """Floats per partial record, over the 512 threads of a workgroup, sized
    for the largest tiling of the head dim: per thread the accumulators of
    its share of the workgroup's query rows x D channels, then one row
    offset and one partial sum per 16-row query tile it holds (four at head
    dim 64, whose waves hold 64 rows; three at 128, 48 rows; two at 256,
    where the two waves of a pair share 32 rows and split the channels)."""
    tiles = {64: 4, 128: 3, 256: 2}[D]
    return (max(query_rows(D)) * D // 512 + 2 * tiles) * 512


def query_rows(D):
    """Query rows per workgroup of each tiling a launch may take."""
    return {64: (512,), 128: (256, 384), 256: (128,)}[D]


@pytest.fixture(scope="module")
def sched_output(tmp_path_factory):
    cxx = shutil.which("g++") or shutil.which("c++")
    if cxx is None:
        pytest.skip("no host C++ compiler")
    exe = str(tmp_path_factory.mktemp("sched") / "sched_check")
    subprocess.run([cxx, "-O2", "-std=c++17", "-Wall", "-Werror", "-I", CSRC, SRC, "-o", exe], check=True)
    res = subprocess.run([exe], capture_output=True, text=True, timeout=300)
    assert res.returncode == 0, res.stdout[-2000:] + res.stderr[-2000:]
    return res.stdout


def test_schedule_sweeps_pass(sched_output):
    last = sched_output.strip().splitlines()[-1]
    assert last.startswith("OK "), last


def test_split_records_fit_the_workspace(sched_output):
    rows = [l.split()[1:] for l in sched_output.splitlines() if l.startswith("WS ")]
    assert len(rows) >= 10
    for B, Sq, Sk, H, D, slots, max_rec in ((int(x) for x in r) for r in rows):
        assert max_rec < slots, (B, Sq, Sk, H, D)
        pad = lambda s, m=256: (s + m - 1) // m * m   # noqa: E731
        kn = (B * H * ((pad(Sk) + 4095) // 4096) * 4 + 255) // 256 * 256   # key-norm maxima
        sq_pad = max([pad(Sq)] + [pad(Sq, r) for r in query_rows(D)])
        needed = (B * H * sq_pad + 2 * B * H * pad(Sk)) * 2 * D + \
            slots * record_floats(D) * 4 + kn
        got = h3attn.forward_ex_workspace_bytes(B, Sq, Sk, H, H, head_dim=D)
        assert got == needed, (B, Sq, Sk, H, D, got, needed)


def test_query_tile_choice_on_the_workload_shapes(sched_output):
    """At head dim 128 the launcher takes three query tiles per wave where
    their 384-row blocks give the shorter schedule on 256 compute units
    (the full sequence, padded), and two where 256-row blocks fill whole
    rounds (mid: exactly one round of 256 tiles) or the launch is tiny."""
    got = {tuple(int(x) for x in l.split()[1:8]): int(l.split()[8])
           for l in sched_output.splitlines() if l.startswith("QT ")}
    assert got[(1, 104448, 104448, 6, 128, 104448, 104448)] == 3
    assert got[(1, 32768, 32768, 8, 128, 30720, 30720)] == 3
    assert got[(1, 8192, 8192, 8, 128, 8192, 8192)] == 2
    assert got[(1, 512, 512, 2, 128, 512, 512)] == 2
    assert got[(1, 104448, 104448, 12, 64, 104448, 104448)] == 4
    assert got[(1, 104448, 104448, 3, 256, 104448, 104448)] == 2
