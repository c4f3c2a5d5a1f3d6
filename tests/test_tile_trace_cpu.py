"""The per-tile trace tool on the CPU: the traced library's exports, and the
summary arithmetic on a hand-made trace whose answer is known."""
import ctypes
import os
import re

import numpy as np
import pytest

from sparse_mixture_experts_22_amd import build, tile_trace

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_tile_trace.h")


def _declared():
    with open(HEADER) as fh:
        text = re.sub(r"/\*.*?\*/", "", fh.read(), flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", text)))


def test_header_layout_matches_tool():
    with open(HEADER) as fh:
        text = fh.read()
    dims = {k: int(v) for k, v in re.findall(r"#define MOE_TILE_TRACE_(\w+) (\d+)", text)}
    assert (dims["PROJS"], dims["WGS"], dims["TILES"], dims["FIELDS"]) == (
        tile_trace.PROJS, tile_trace.WGS, tile_trace.TILES, tile_trace.FIELDS)


def test_traced_library_exports_the_trace_calls():
    if not os.path.exists(build.TRACE_LIB):
        pytest.skip("libmoe_tiletrace.so not built")
    L = ctypes.CDLL(build.TRACE_LIB)
    for sym in _declared():
        assert hasattr(L, sym), sym
    assert _declared() == ["moe_tile_trace_clear", "moe_tile_trace_read"]


def test_regular_library_has_no_trace_calls():
    if not os.path.exists(build.LIB):
        pytest.skip("libmoe.so not built")
    L = ctypes.CDLL(build.LIB)
    for sym in _declared():
        assert not hasattr(L, sym), sym


def test_summary_of_a_known_trace():
    """Two workgroups, up projection only: workgroup 0 runs two tiles, workgroup 1
    one.  Each k-loop: 8 live blocks x 4 k-steps = 128 MFMAs per wave, given
    6400 cycles (50 per MFMA) in 4 us (1.6 GHz)."""
    tr = np.zeros((tile_trace.PROJS, tile_trace.WGS, tile_trace.TILES, tile_trace.FIELDS), dtype=np.int64)

    def tile(wg, j, t0_us, clk0):
        # moments (us): loop start, loop end (+4), barrier (+0.05), transition (+0.2), epilogue (+0.15)
        rt = np.array([0.0, 4.0, 4.05, 4.25, 4.4]) + t0_us
        ck = np.array([0, 6400, 6480, 6800, 7040]) + clk0
        tr[0, wg, j, 0:5] = np.round(rt * 100).astype(np.int64) + 1000
        tr[0, wg, j, 5:10] = ck
        tr[0, wg, j, 10] = 8 + 16 * 4
        tr[0, wg, j, 11] = 8

    tile(0, 0, 0.0, 10_000)
    tile(0, 1, 4.42, 20_000)
    tile(1, 0, 0.0, 30_000)
    s = tile_trace.summarize(tr, "known")
    assert "3 tiles on 2 workgroups" in s
    assert "50.0 cycles per MFMA" in s and "64.0% of it" in s and "clock 1.60 GHz" in s
    assert "no tiles recorded" in s  # the down projection
    # workgroup 1 ends at 4.4 us, workgroup 0 at 8.82 us: idle tail 4.42 of 2 x 8.82 = 25.1%;
    # k-loops 3 x 4 us of 2 x 8.82 = 68.0%
    assert "idle tail 25.1%" in s and "k-loops 68.0%" in s
    m = re.search(r"k-loop\s+([\d.]+)\s+([\d.]+)", s)
    assert m and float(m.group(1)) == pytest.approx(4.0)
    assert re.search(r"transition \(next tile's loads issued\)\s+0\.20\s+0\.20\s+0\.20\s+320\s+1\.60", s)
