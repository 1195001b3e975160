"""Host-side pieces of bench.py: byte accounting, the counter summary and the one-GPU guard."""

from __future__ import annotations

import csv
import json
import os

import pytest

import bench
from workloads import make_case


def test_algorithmic_bytes_tiny_by_hand():
    """tiny: 4 seqs of L = {1, 17, 33, 64}, 4 q / 2 kv heads, head_dim 64, fp32, b = 16."""
    case = make_case("tiny")
    kv = (1 + 17 + 33 + 64) * 2 * 2 * 64 * 4          # K and V rows, every kv head
    q = 4 * 1 * 4 * 64 * 4
    out = 4 * 1 * 4 * 64 * 4
    tables = 4 * (1 + 2 + 3 + 4) + 4 * 4               # used table entries + lengths
    assert bench.algorithmic_bytes(case) == kv + q + out + tables


def test_kv_bytes_per_position_matches_pages_figure():
    """8 kv heads x head_dim 128 x bf16: 4 KiB of K and V per position in one layer."""
    assert bench.kv_bytes_per_position(8, 128, 2) == 4096


def test_unique_bytes_counts_shared_prefix_once():
    case = make_case("prefix", num_seqs=3)
    per_pos = bench.kv_bytes_per_position(8, 128, 2)
    lens = [int(x) for x in case.seq_lens]
    shared = 2048
    kv_unique = (shared + sum(L - shared for L in lens)) * per_pos
    kv_logical = sum(lens) * per_pos
    assert bench.unique_bytes(case) - kv_unique == bench.algorithmic_bytes(case) - kv_logical


def test_more_than_one_gpu_is_refused(capsys):
    assert bench.main(["--gpus", "2"]) == 2
    assert "one GPU" in capsys.readouterr().err


def _write_pmc(dirpath, counter, rows):
    os.makedirs(dirpath, exist_ok=True)
    with open(os.path.join(dirpath, "run_counter_collection.csv"), "w", newline="") as fh:
        w = csv.writer(fh)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        for i, (name, value) in enumerate(rows):
            w.writerow([i, name, counter, value])


def test_summarize_pmc_scales_by_copy_kernel(tmp_path):
    """The copy kernel reads and writes CALIBRATION_BYTES; counters that read half of that give a
    factor of 2, which then scales the decode kernels' readings."""
    copy_kib = bench.CALIBRATION_BYTES / 1024 / 2
    neg = "void at::native::vectorized_elementwise_kernel<4, at::native::neg_kernel_cuda>"
    dec = "void pa::(anonymous namespace)::decode_mfma_kernel<1, 16, 4, 1, false>(pa::DecodeParams)"
    _write_pmc(tmp_path / "f", "FETCH_SIZE", [(neg, copy_kib)] * 3 + [(dec, 1000.0), (dec, 1000.0), (dec, 5000.0)])
    _write_pmc(tmp_path / "w", "WRITE_SIZE", [(neg, copy_kib)] * 3 + [(dec, 10.0)] * 3)
    log = tmp_path / "bench.log"
    log.write_text("noise\n" + json.dumps({"roofline": {"bytes_per_launch": 4096000}}) + "\n")
    text = bench.summarize_pmc(str(tmp_path / "f"), str(tmp_path / "w"), str(log), "batch64")
    s = {}
    for line in text.splitlines():
        if " = " in line and not line.startswith("#"):
            k, v = line.split(" = ", 1)
            s[k] = v
    assert float(s["fetch_factor"]) == pytest.approx(2.0)
    assert float(s["write_factor"]) == pytest.approx(2.0)
    assert int(s["traffic_bytes_per_call"]) == (1000 + 10) * 1024 * 2   # medians, scaled
    assert float(s["traffic_over_algorithmic"]) == pytest.approx((1010 * 2048) / 4096000, rel=1e-3)
    assert s["library_sha256"] == bench.library_sha256()


def test_summarize_l2_hit_rate(tmp_path):
    """TCC_HIT_sum / TCC_MISS_sum medians per kernel give hits / (hits + misses); other kernels are left out."""
    cas = "void pa::(anonymous namespace)::cascade_kernel<1, 16, true>(pa::DecodeParams, int, int)"
    other = "void at::native::vectorized_elementwise_kernel<4, at::native::neg_kernel_cuda>"
    d = tmp_path / "l2"
    os.makedirs(d)
    with open(d / "run_counter_collection.csv", "w", newline="") as fh:
        w = csv.writer(fh)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        rows = [(cas, "TCC_HIT_sum", v) for v in (300, 100, 300)] + [(cas, "TCC_MISS_sum", v) for v in (100, 900, 100)]
        rows += [(other, "TCC_HIT_sum", 5), (other, "TCC_MISS_sum", 5)]
        for i, (name, counter, value) in enumerate(rows):
            w.writerow([i, name, counter, value])
    text = bench.summarize_l2(str(d), "prefix", "rocprofv3 ...")
    s = dict(line.split(" = ", 1) for line in text.splitlines() if " = " in line and not line.startswith("#"))
    assert s["kernel_0_tcc_hit"] == "300" and s["kernel_0_tcc_miss"] == "100"
    assert float(s["kernel_0_l2_hit_rate"]) == pytest.approx(0.75)
    assert "kernel_1" not in s and "neg_kernel" not in text


def test_traffic_ignored_when_sources_changed(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    (tmp_path / "traffic_decode_batch64.txt").write_text(
        "library_sha256 = 0000\ntraffic_bytes_per_call = 123\n")
    assert bench.traffic_from_profiles("batch64") is None
    (tmp_path / "traffic_decode_batch64.txt").write_text(
        f"library_sha256 = {bench.library_sha256()}\ntraffic_bytes_per_call = 123\n")
    assert bench.traffic_from_profiles("batch64") == 123
