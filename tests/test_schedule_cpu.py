"""CPU checks of the two forward kernels' static schedules.

tests/schedule_check.cpp includes the resident kernel's schedule header
(vision_transformer_token_amd/csrc/lisa_resident.hpp) and checks exact
coverage of every token, staging of every window cell a tile token needs,
LDS bounds of every region, DMA run and slot-table row, and the combine
partition.  tests/flow_schedule_check.cpp does the same for the streaming
kernel (lisa_flow_schedule.hpp): tiles, token ranges, chunks, combine
elements, groups and slices, staging bounds, the float quotients of the
staging DMA, and that the stage order its producer waves walk is the one its
consumer waves run.  Both use the library's own planners.  They are built
with hipcc for the host only and run on every workload shape, the test
suites' ragged and edge shapes, and the same shapes planned for devices with
other compute-unit counts.
"""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "schedule_check.cpp")
FLOW_SRC = os.path.join(ROOT, "tests", "flow_schedule_check.cpp")
INC = os.path.join(ROOT, "vision_transformer_token_amd", "csrc")

# (B * heads, H, W, T): the workloads and the GPU tests' shapes.
SHAPES = [
    (1, 14, 14, 3), (192, 14, 14, 3), (192, 24, 24, 3), (192, 24, 24, 5), (32, 56, 56, 3), (1, 200, 320, 5),
    (1, 64, 64, 5), (1, 128, 128, 5), (1, 256, 256, 5),
    (1, 1, 1, 3), (2, 1, 7, 3), (2, 7, 1, 4), (6, 5, 7, 2), (1, 13, 17, 5), (3, 13, 17, 8), (1, 3, 100, 3),
    (2, 2, 65, 6), (2, 9, 33, 3), (1, 70, 70, 3), (1, 41, 45, 7), (1, 260, 260, 3), (288, 14, 14, 3),
    (260, 9, 11, 4), (1, 24, 24, 3), (2, 13, 17, 8), (1, 56, 56, 8), (4, 56, 56, 3), (6, 10, 13, 3),
    (2, 17, 9, 5), (6, 20, 15, 5), (1, 12, 12, 8), (3, 1, 1, 3), (2, 1, 40, 4), (1, 16, 17, 3), (4, 13, 21, 3),
    (2, 9, 11, 6), (2, 12, 10, 3), (4, 8, 9, 4), (2, 10, 13, 6), (2, 19, 23, 4), (1, 9, 11, 3), (1, 33, 29, 3),
    (1, 1, 320, 5), (1, 320, 1, 5), (1, 2, 2, 1), (1, 100, 3, 2), (1, 30, 30, 1),
]


def gmax(n):
    """Ranks the workspace's partials are sized for: a power of two, at most
    one per 128 tokens and 256 (lisa_api.hip plan_ranks)."""
    per = min(256, -(-n // 128))
    g = 1
    while 2 * g <= per:
        g *= 2
    return g


def gcap(cus, bh, n):
    return min(max(1, cus // bh), gmax(n))


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    exe = str(tmp_path_factory.mktemp("sched") / "schedule_check")
    res = subprocess.run([hipcc, "-O1", "-std=c++17", "-I", INC, SRC, "-o", exe], capture_output=True, text=True)
    assert res.returncode == 0, res.stdout + res.stderr
    return exe


@pytest.mark.parametrize("cus", [256, 304, 80, 32])
def test_resident_schedule_covers_exactly_once(checker, cus):
    args = []
    for bh, H, W, T in SHAPES:
        args += [str(H), str(W), str(T), str(gcap(cus, bh, H * W))]
    res = subprocess.run([checker, *args], capture_output=True, text=True)
    print(res.stdout)
    assert res.returncode == 0, res.stdout + res.stderr
    assert res.stdout.count("ok ") + res.stdout.count("none ") == len(SHAPES)


def test_projection_schedules_cover_exactly_once(checker):
    """The layer's projections (lisa_layer.hpp): for row counts from 1 to
    PVT-T stage 1's 100,352 and 64 to 576 outputs, the blocked kernel's
    workgroups and the streaming kernel's units each take every output block
    once, and a streaming workgroup's units share its column block."""
    res = subprocess.run([checker], capture_output=True, text=True)
    assert res.returncode == 0, res.stdout + res.stderr
    assert res.stdout.count(" covered: ") == 36, res.stdout
    assert "proj 100352 192 covered: 1176 workgroups, 4704 units on 1008" in res.stdout, res.stdout


def test_headline_tiling(checker):
    """PVT-T stage 1 (32 slices of 56 x 56) on 256 compute units: eight ranks
    per slice on 28 x 14 tiles, everything on chip."""
    res = subprocess.run([checker, "56", "56", "3", str(gcap(256, 32, 3136))], capture_output=True, text=True)
    assert res.returncode == 0, res.stdout
    assert "G=8 tiles 2x4 of 28x14" in res.stdout, res.stdout


@pytest.fixture(scope="module")
def flow_checker(tmp_path_factory):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    exe = str(tmp_path_factory.mktemp("flow") / "flow_schedule_check")
    res = subprocess.run([hipcc, "-O1", "-std=c++17", "-I", INC, FLOW_SRC, "-o", exe], capture_output=True, text=True)
    assert res.returncode == 0, res.stdout + res.stderr
    return exe


@pytest.mark.parametrize("cus,xccs", [(256, 8), (304, 8), (80, 1), (32, 1)])
def test_streaming_schedule_covers_exactly_once(flow_checker, cus, xccs):
    args, count = [], 0
    for bh, H, W, T in SHAPES + [(1, 56, 56, 16), (2, 13, 17, 12), (1, 20, 23, 16), (128, 9, 11, 9)]:
        for es in (2, 4):
            for per_token in (0, 1):
                args += [str(v) for v in (H, W, T, bh, es, per_token, cus, xccs, gmax(H * W))]
                count += 1
    res = subprocess.run([flow_checker, *args], capture_output=True, text=True)
    print(res.stdout[-3000:])
    assert res.returncode == 0, res.stdout[-3000:] + res.stderr
    assert res.stdout.count("ok ") == count, res.stdout[-3000:]


def test_streaming_headline_plan(flow_checker):
    """PVT-T stage 1 (32 slices of 56 x 56, bf16, per-token weights) on 256
    compute units: eight ranks per slice, one slice per group."""
    res = subprocess.run([flow_checker, "56", "56", "3", "32", "2", "1", "256", "8", str(gmax(3136))],
                         capture_output=True, text=True)
    assert res.returncode == 0, res.stdout
    assert "G=8 S=32 Z=1 xcd=0" in res.stdout, res.stdout
