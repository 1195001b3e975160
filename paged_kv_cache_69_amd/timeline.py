"""Per-wave timeline of one decode call on the GPU, from libpa_timeline.so (include/pa_timeline.h).

    python -m paged_kv_cache_69_amd._build --timeline        # once, on the build host
    python -m paged_kv_cache_69_amd.timeline --workload long [--split-schedule S] [--replicas N]

The call is the benchmark's step for that workload (the fused append + decode for the bf16 workloads;
the decode call for the 8-bit ones), made on cold pools: the pools are replicated until the copies
exceed the GPU's 256 MiB last-level cache and the recorded call reads the copy used longest ago. It
prints, from the records of every wave of the launch: the spread of wave starts, first tiles and ends;
the waves in flight over time; the ends per XCD; and, for waves that share a SIMD, how long the one
that started first ran against the other.
"""

from __future__ import annotations

import argparse
import ctypes
import sys

import numpy as np

WORDS = 8


def _load(pa):
    from paged_kv_cache_69_amd._build import TIMELINE_LIB_PATH

    lib = pa.load_library(TIMELINE_LIB_PATH)
    lib.pa_timeline_read.argtypes = [ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t]
    lib.pa_timeline_read.restype = ctypes.c_int
    lib.pa_timeline_clear.argtypes = []
    lib.pa_timeline_clear.restype = ctypes.c_int
    pa._lib = lib  # the package's wrappers call into this build from here on
    return lib


def _call(pa, name, case, g, split_schedule):
    """The workload's step on the pools in g (the benchmark's call shapes)."""
    pt = {"batch64": None, "long": 512, "spec": None, "prefix": 256}[name.split("_")[0]]
    if name.endswith(("_int8", "_fp8")):
        dec = pa.decode_int8 if name.endswith("_int8") else pa.decode_fp8
        if pt is None:
            return dec(g["q"], g["k_pool"], g["v_pool"], g["scales"], g["block_tables"], g["seq_lens"], case.scale)
        decp = pa.decode_partitioned_int8 if name.endswith("_int8") else pa.decode_partitioned_fp8
        return decp(g["q"], g["k_pool"], g["v_pool"], g["scales"], g["block_tables"], g["seq_lens"], case.scale,
                    case.max_seq_len, pt, split_schedule=split_schedule)
    if name == "prefix":
        return pa.write_kv_decode_cascade(g["q"], g["k_new"], g["v_new"], g["k_pool"], g["v_pool"], g["block_tables"],
                                          g["seq_lens"], case.scale, 2048, case.max_seq_len, pt)  # the shared prefix
    kw = dict(max_seq_len=case.max_seq_len, partition_tokens=pt, split_schedule=split_schedule) if pt else {}
    return pa.write_kv_decode(g["q"], g["k_new"], g["v_new"], g["k_pool"], g["v_pool"], g["block_tables"],
                              g["seq_lens"], case.scale, **kw)


def record(name: str, split_schedule: int = 0, replicas: int = 0):
    """Run the workload's call on cold pools and return {family: records [waves, 8] uint64}."""
    import torch

    import paged_kv_cache_69_amd as pa
    from workloads import fp8_pools, int8_pools, make_case

    lib = _load(pa)
    base = name.replace("_int8", "").replace("_fp8", "")
    case = make_case(base, pool_device="cuda:0")
    g = {k: getattr(case, k).to("cuda:0") for k in ("q", "k_new", "v_new", "k_pool", "v_pool", "block_tables",
                                                    "seq_lens")}
    if name.endswith(("_int8", "_fp8")):
        kc, vc, sc = (int8_pools if name.endswith("_int8") else fp8_pools)(case)
        g.update(k_pool=kc.to("cuda:0"), v_pool=vc.to("cuda:0"), scales=sc.to("cuda:0"))
    pool_bytes = 2 * g["k_pool"].numel() * g["k_pool"].element_size()
    n = replicas or max(2, -(-(512 << 20) // pool_bytes))
    reps = [dict(g)] + [dict(g, k_pool=g["k_pool"].clone(), v_pool=g["v_pool"].clone()) for _ in range(n - 1)]
    for _ in range(2):
        for r in reps:
            _call(pa, name, case, r, split_schedule)
    for r in reps[:-1]:
        _call(pa, name, case, r, split_schedule)
    torch.cuda.synchronize()
    if lib.pa_timeline_clear() != 0:
        raise RuntimeError("pa_timeline_clear failed")
    _call(pa, name, case, reps[-1], split_schedule)
    torch.cuda.synchronize()
    out = {}
    for fam, label in ((0, "mfma"), (1, "balanced")):
        buf = np.zeros(16384 * WORDS, dtype=np.uint64)
        if lib.pa_timeline_read(fam, buf.ctypes.data, buf.nbytes) != 0:
            raise RuntimeError("pa_timeline_read failed")
        rec = buf.reshape(-1, WORDS)
        if (rec[:, 0] > 0).any():
            out[label] = rec
    return out


def summarize(rec: np.ndarray, waves_per_group: int) -> list[str]:
    """Text summary of one family's records (times in microseconds from the first wave's start)."""
    idx = np.nonzero(rec[:, 0] > 0)[0]
    r = rec[idx]
    t0 = r[:, 0].astype(np.int64).min()
    us = lambda x: (x.astype(np.int64) - t0) / 100.0  # noqa: E731  (100 MHz clock)
    st, en = us(r[:, 0]), us(r[:, 3])
    first = np.where(r[:, 1] > 0, us(r[:, 1]), np.nan)
    tiles = r[:, 5].astype(np.int64)
    hw = (r[:, 4] & 0xFFFFFFFF).astype(np.int64)
    xcc = (r[:, 4] >> 32).astype(np.int64)
    simd, cu, se = (hw >> 4) & 3, (hw >> 8) & 15, (hw >> 13) & 7
    work = tiles > 0
    pct = lambda a, q: np.percentile(a, q) if len(a) else float("nan")  # noqa: E731
    lines = [f"waves_recorded = {len(r)}", f"waves_with_tiles = {int(work.sum())}", f"tiles = {int(tiles.sum())}",
             f"span_us = {en.max():.2f}",
             "start_us p50/p90/max = %.2f / %.2f / %.2f" % (pct(st, 50), pct(st, 90), st.max()),
             "first_tile_us p10/p50/p90 = %.2f / %.2f / %.2f" % tuple(pct(first[work], q) for q in (10, 50, 90)),
             "end_us (waves with tiles) p10/p50/p90/max = %.2f / %.2f / %.2f / %.2f" % (
                 *(pct(en[work], q) for q in (10, 50, 90)), en[work].max() if work.any() else float("nan"))]
    for t in np.linspace(0.0, en.max(), 11):
        lines.append(f"waves_in_flight t={t:7.2f} us: {int(((st <= t) & (en > t) & work).sum())}")
    for x in range(8):
        m = work & (xcc == x)
        if m.any():
            lines.append(f"xcd {x}: waves {int(m.sum())} tiles {int(tiles[m].sum())} end p50 {np.median(en[m]):.2f} "
                         f"max {en[m].max():.2f}")
    # waves that share a SIMD and overlap in time: the one that started first against the other
    key = ((xcc * 8 + se) * 16 + cu) * 4 + simd
    older_first = younger_first = 0
    d_old, d_young = [], []
    for k in np.unique(key[work]):
        w = np.nonzero(work & (key == k))[0]
        if len(w) != 2:
            continue
        a, b = w[np.argsort(st[w])]
        if st[b] >= en[a] or tiles[a] != tiles[b]:
            continue  # not side by side, or unequal work
        d_old.append(en[a] - st[a])
        d_young.append(en[b] - st[b])
        older_first += en[a] < en[b]
        younger_first += en[b] < en[a]
    if d_old:
        lines.append(f"simd_pairs_equal_tiles = {len(d_old)}: the earlier-started wave ends first in {older_first}, "
                     f"the later one in {younger_first}; duration p50 {np.median(d_old):.2f} us vs "
                     f"{np.median(d_young):.2f} us")
    return lines


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--workload", default="long",
                    choices=["batch64", "long", "spec", "prefix", "batch64_int8", "long_int8", "batch64_fp8",
                             "long_fp8"])
    ap.add_argument("--split-schedule", type=int, default=0)
    ap.add_argument("--replicas", type=int, default=0)
    args = ap.parse_args(argv)
    recs = record(args.workload, args.split_schedule, args.replicas)
    print(f"# per-wave timeline of one {args.workload} call (split schedule {args.split_schedule}), cold pools")
    print(f"# command (from the repository root): python -m paged_kv_cache_69_amd.timeline --workload {args.workload}"
          f" --split-schedule {args.split_schedule}")
    for fam, rec in recs.items():
        print(f"family = {fam}")
        for line in summarize(rec, 8 if fam == "balanced" else 4):
            print(line)
    return 0


if __name__ == "__main__":
    sys.exit(main())
