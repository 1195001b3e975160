"""Host logic of the per-wave timeline summary (paged_kv_cache_69_amd.timeline.summarize) on hand-made
records: [start, first tile, loop end, end, XCC << 32 | HW_ID, tiles, 0, 0], times in 100 MHz ticks."""

from __future__ import annotations

import numpy as np

from paged_kv_cache_69_amd.timeline import WORDS, summarize


def _hw(se, cu, simd):
    return (se << 13) | (cu << 8) | (simd << 4)


def _rec(start, first, end, xcc, se, cu, simd, tiles):
    r = np.zeros(WORDS, dtype=np.uint64)
    r[:6] = [start, first, end, end, (xcc << 32) | _hw(se, cu, simd), tiles]
    return r


def test_summary_of_hand_made_records():
    t0 = 1_000_000
    rows = [
        # two waves on one SIMD with equal work: the earlier one ends first
        _rec(t0, t0 + 400, t0 + 9000, 0, 1, 2, 3, 10),
        _rec(t0 + 10, t0 + 500, t0 + 12000, 0, 1, 2, 3, 10),
        # a wave on another XCD, and a wave with no tile
        _rec(t0 + 20, t0 + 300, t0 + 15000, 5, 0, 0, 0, 4),
        _rec(t0 + 30, 0, t0 + 700, 5, 0, 0, 1, 0),
    ]
    rec = np.stack(rows + [np.zeros(WORDS, dtype=np.uint64)] * 3)  # unused slots stay zero
    out = "\n".join(summarize(rec, 4))
    assert "waves_recorded = 4" in out
    assert "waves_with_tiles = 3" in out
    assert "tiles = 24" in out
    assert "span_us = 150.00" in out  # latest end, 15000 ticks of 10 ns after the first start
    assert "xcd 0: waves 2 tiles 20 end p50 105.00 max 120.00" in out
    assert "xcd 5: waves 1 tiles 4 end p50 150.00 max 150.00" in out
    assert ("simd_pairs_equal_tiles = 1: the earlier-started wave ends first in 1, the later one in 0; "
            "duration p50 90.00 us vs 119.90 us") in out
