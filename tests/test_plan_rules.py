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
COST = {256: 1000, 192: 1060, 128: 1250}
UNITS = {256: 16, 192: 13, 128: 10}


@pytest.fixture(scope="module")
def output(tmp_path_factory):
    if not shutil.which(B.HIPCC) and not os.path.exists(B.HIPCC):
        pytest.skip("hipcc not available")
    exe = str(tmp_path_factory.mktemp("plan") / "plan_rules_check")
    subprocess.run([B.HIPCC, "-O1", "-std=c++17", "-I", B.CSRC, os.path.join(HERE, "plan_rules_check.cpp"),
                    "-o", exe], check=True, capture_output=True)
    return subprocess.run([exe], check=True, capture_output=True, text=True).stdout.splitlines()


def candidates(n):
    out = []
    for tm in (256, 192, 128):
        k = -(-n // tm)
        out.append((k * tm * COST[tm], k, tm, tm))
    q, rem = divmod(n, 256)
    if q and rem:
        r = 128 if rem <= 128 else (192 if rem <= 192 else 256)
        out.append((q * 256 * COST[256] + r * COST[r], q + 1, 256, r))
    return out


def test_tile_split(output):
    rows = [l.split() for l in output if l[0].isdigit()]
    assert len(rows) == 3000
    for n, nt, mt, lt, cost in (map(int, r) for r in rows):
        covered = (nt - 1) * mt + lt
        assert covered >= n > covered - lt, (n, nt, mt, lt)  # no tile to spare
        best = min(c[0] for c in candidates(n))
        assert (nt - 1) * mt * COST[mt] + lt * COST[lt] == best, n
        assert cost == (nt - 1) * UNITS[mt] + UNITS[lt]


def test_tile_split_max_192(output):
    """With heights limited to 192 (MXFP8 weights): one height per expert,
    the cheaper of all-192 and all-128, no 256-row tile, no tile to spare."""
    rows = [list(map(int, l.split()[1:])) for l in output if l.startswith("mx ")]
    assert len(rows) == 1500
    for n, nt, mt, lt in rows:
        assert mt == lt and mt in (128, 192)
        assert nt * mt >= n > (nt - 1) * mt
        best = min(-(-n // tm) * tm * COST[tm] for tm in (192, 128))
        assert nt * mt * COST[mt] == best, n


def test_xcd_bounds(output):
    line = [l for l in output if l.startswith("xcd ")][0].split()
    C, T = int(line[1]), int(line[2])
    b = list(map(int, line[3:]))
    assert len(b) == 9 and b[0] == 0 and b[-1] == T and b == sorted(b)
    # each slice ends at the first tile where the running cost reaches its
    # share, so every slice is within one tile (at most 16 units) of C/8
    sl = list(map(int, [l for l in output if l.startswith("slices")][0].split()[1:]))
    assert sum(sl) == C
    assert all(abs(c - C / 8) <= 16 for c in sl), sl


def test_light_rule(output):
    line = [l for l in output if l.startswith("light ")][0].split()
    assert int(line[1]) == int(line[3])  # 4000 rows over 500 experts: mean 8 -> light
    assert int(line[2]) == int(line[4])  # one row more: only the cold tail stays light
    assert 0 <= int(line[4]) <= 16
