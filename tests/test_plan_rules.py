"""Host-side checks of the heavy-tile plan rules (launch.h), compiled from
tests/plan_rules_check.cpp: each expert's rows are covered by its tiles with
no tile to spare, the split is the cheapest of the candidates the rule
considers, and the XCD slices are monotone, cover every tile and are of
about equal cost."""
import os
import shutil
import subprocess

import pytest

from expert_ffn_layer_amd import build as B

HERE = os.path.dirname(os.path.abspath(__file__))
COST = {256: 1000, 224: 1020, 192: 1060, 160: 1130, 128: 1250}
HEIGHTS = (256, 224, 192, 160, 128)
UNITS = {tm: (tm * COST[tm] + 8000) // 16000 for tm in HEIGHTS}


@pytest.fixture(scope="module")
def output(tmp_path_factory):
    if not shutil.which(B.HIPCC) and not os.path.exists(B.HIPCC):
        pytest.skip("hipcc not available")
    exe = str(tmp_path_factory.mktemp("plan") / "plan_rules_check")
    subprocess.run([B.HIPCC, "-O1", "-std=c++17", "-I", B.CSRC, os.path.join(HERE, "plan_rules_check.cpp"),
                    "-o", exe], check=True, capture_output=True)
    return subprocess.run([exe], check=True, capture_output=True, text=True).stdout.splitlines()


def candidates(n, heights=HEIGHTS):
    """(cost, ntiles, height) of cutting n rows into equal tiles of each height."""
    return [(-(-n // tm) * tm * COST[tm], -(-n // tm), tm) for tm in heights]


def test_tile_split(output):
    """One height per expert (the tiles that share its weights stay in step),
    the cheapest of the five, no tile to spare."""
    rows = [l.split() for l in output if l[0].isdigit()]
    assert len(rows) == 3000
    for n, nt, mt, lt, cost in (map(int, r) for r in rows):
        assert mt == lt and mt in HEIGHTS
        assert nt * mt >= n > (nt - 1) * mt, (n, nt, mt)  # no tile to spare
        assert nt * mt * COST[mt] == min(c[0] for c in candidates(n)), n
        assert cost == nt * UNITS[mt]
    # the rows of an expert of 640 rows (long prefill) and of 160 (prefill)
    # go in equal tiles with little padding
    by_n = {int(r[0]): (int(r[1]), int(r[2])) for r in rows}
    assert by_n[640] == (3, 224) and by_n[160] == (1, 160)


def test_tile_split_max_192(output):
    """With heights limited to 192 (MXFP8 weights): one height per expert,
    the cheapest of 192, 160 and 128, no taller tile, no tile to spare."""
    rows = [list(map(int, l.split()[1:])) for l in output if l.startswith("mx ")]
    assert len(rows) == 1500
    for n, nt, mt, lt in rows:
        assert mt == lt and mt in (128, 160, 192)
        assert nt * mt >= n > (nt - 1) * mt
        best = min(c[0] for c in candidates(n, (192, 160, 128)))
        assert nt * mt * COST[mt] == best, n


def test_xcd_bounds(output):
    line = [l for l in output if l.startswith("xcd ")][0].split()
    C, T = int(line[1]), int(line[2])
    b = list(map(int, line[3:]))
    assert len(b) == 9 and b[0] == 0 and b[-1] == T and b == sorted(b)
    # each slice ends at the first tile where the running cost reaches its
    # share, so every slice is within one tile (at most 16 units) of C/8
    sl = list(map(int, [l for l in output if l.startswith("slices ")][0].split()[1:]))
    assert sum(sl) == C
    assert all(abs(c - C / 8) <= 16 for c in sl), sl


def test_xcd_bounds_rounded(output):
    """Bounds rounded to whole rounds of 4 tiles: monotone, multiples of 4
    (but the last), each within 2 tiles of the unrounded one, so every slice
    stays within 5 tiles (80 units) of C/8."""
    un = list(map(int, [l for l in output if l.startswith("xcd ")][0].split()[3:]))
    line = [l for l in output if l.startswith("xcdr ")][0].split()
    C, T = int(line[1]), int(line[2])
    b = list(map(int, line[3:]))
    assert len(b) == 9 and b[0] == 0 and b[-1] == T and b == sorted(b)
    assert all(x % 4 == 0 for x in b[:-1])
    assert all(abs(x - y) <= 2 for x, y in zip(b, un))
    sl = list(map(int, [l for l in output if l.startswith("slicesr ")][0].split()[1:]))
    assert sum(sl) == C and all(abs(c - C / 8) <= 80 for c in sl), sl
    # tiles per round: 256 CUs / 8 XCDs = 32 blocks per slice over the N blocks
    # of the narrower GEMM (8 -> 4 tiles, 16 -> 2), 1 where it does not divide
    assert [l for l in output if l.startswith("round ")][0].split()[1:] == ["4", "2", "1", "1"]


def test_light_rule(output):
    line = [l for l in output if l.startswith("light ")][0].split()
    assert int(line[1]) == int(line[3])  # 4000 rows over 500 experts: mean 8 -> light
    assert int(line[2]) == int(line[4])  # one row more: only the cold tail stays light
    assert 0 <= int(line[4]) <= 16
