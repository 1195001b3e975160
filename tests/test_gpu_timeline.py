"""The per-wave timeline build on the GPU: one cold batch64 call records every wave of its launch, and the
tiles the waves report add up to the call's tiles (16-position tiles of every sequence, for every kv head)."""

from __future__ import annotations

import os

import numpy as np
import pytest

pytestmark = pytest.mark.gpu


def test_timeline_records_every_wave_and_tile():
    import paged_kv_cache_69_amd as pa
    from paged_kv_cache_69_amd import timeline
    from paged_kv_cache_69_amd._build import TIMELINE_LIB_PATH
    from workloads import make_case

    if not os.path.exists(TIMELINE_LIB_PATH):
        pytest.skip("timeline build not present")
    saved = pa._lib
    try:
        print("[case] timeline batch64", flush=True)
        recs = timeline.record("batch64", replicas=2)
    finally:
        pa._lib = saved  # later tests run on libpa.so again
    assert set(recs) == {"mfma"}
    rec = recs["mfma"]
    live = rec[rec[:, 0] > 0]
    case = make_case("batch64")
    lens = case.seq_lens.numpy()
    hkv = case.k_pool.shape[1]
    assert len(live) == len(lens) * hkv * 4  # one workgroup of four waves per (sequence, kv head)
    assert int(live[:, 5].sum()) == int(((lens + 15) // 16).sum()) * hkv
    assert (live[:, 3] >= live[:, 0]).all()  # every wave ends after it starts
    lines = timeline.summarize(rec, 4)
    assert any(line.startswith("span_us = ") for line in lines)
    assert np.isfinite(float(lines[3].split("=")[1]))
