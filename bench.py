#!/usr/bin/env python3
"""Benchmark of the paged-KV decode step on one MI355X.

A step is one pass of the whole hot path over one batch: the KV append and
decode attention over every sequence. On the workloads whose launch
configuration says so (batch64, long) the step is one pa_write_kv_decode call
(or its split-context form); otherwise it is pa_write_kv then pa_decode /
pa_decode_partitioned (the _int8 entry points for int8 pools); --no-fused
always times the separate calls. Inputs are synthetic, seeded and resident in HBM before the timed
region starts. R independent replicas of (pools, tables, q, new rows) are
rotated step by step, so the 256 MB Infinity Cache cannot serve the KV of one
step from the previous one; R * (bytes one step touches) >= 1 GB. The K timed
steps run as HIP graph replays (one captured step per replica), so host launch
cost is not timed; that gives `value`. Then K of the step's attention calls
(the fused call, or the decode call) run back to back as one graph between a
pair of HIP events on their stream, which gives that call's average duration
for `roofline`.

Prints one JSON line. `value` is decode tokens per second of the whole step.
`roofline` relates the decode call's algorithmic bytes to its measured
duration and to the 8 TB/s HBM peak; its `traffic` is the HBM bytes one call
moved as rocprofv3's FETCH_SIZE + WRITE_SIZE counters read them (scaled by
what the same counters read for a copy kernel of known size), taken from the
summary under profiles/ when that summary was made with the libpa.so now
built, else null. `roofline` also relates the call to two figures measured in
the same run with libpa_probe.so: `stream_gbps`, the best rate a plain
streaming-read kernel reaches over 2 GiB (`frac_of_stream` = achieved /
stream_gbps), and `floor_us`, the duration of a launch that makes only the
dependent loads in front of each decode workgroup's first K/V tile (length and
table entry together, then the tile) over the same cold replicas;
`model_us` = floor_us + bytes / stream_gbps. The prefill line's roofline (the
bf16 matrix peak) carries `measured_mfma_tflops`, the rate a register-only MFMA
loop of the same instruction reaches on this GPU in the same run, and
`frac_of_measured_mfma`. `cpu_baseline` is the float64
oracle on this host's cores (sequences spread over a thread pool, BLAS on
one BLAS thread per worker), over a bounded sample of the same workload, with a
one-thread figure beside it.

Two helper modes turn rocprofv3 output into those profiles/ summaries:
``--summarize-pmc FETCH_DIR WRITE_DIR BENCH_LOG`` and ``--summarize-stats DIR``.
"""

from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import math
import os
import re
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "paged decode attention: tokens/s and achieved HBM GB/s (% of peak), 1 MI355X"
HBM_PEAK_GBPS = 8000.0
COLD_BYTES = 1 << 30  # replicas rotate over at least this much memory
REPLICAS = 0  # --replicas N: that many input copies instead of enough for a cold cache (a warm-cache run)
PAGED_PROBE = True  # --no-paged-probe: skip the paged-read probe sweep
MFMA_PROBE = True  # --no-mfma-probe: skip the matrix-rate probe of the prefill line
SPLIT_SCHEDULE = 0  # --split-schedule N: pa_dims.split_schedule of split calls (0: the library's choice)
CALIBRATION_BYTES = 512 << 20  # the copy kernel that calibrates the traffic counters reads and writes this much
STREAM_BYTES = 2 << 30  # the streaming-read probe reads this much per launch (far past every cache)
PROFILES = os.path.join(ROOT, "profiles")

# Launch configuration per workload: partition_tokens None = single-pass decode; fused = the step is
# one fused append + decode call (pa_write_kv_decode[_partitioned|_cascade]), measured faster than the
# two calls on batch64, long and prefix; the speculative workload keeps the two calls.
WORKLOADS = {
    "batch64": dict(partition_tokens=None, fused=True, desc="64 seqs, L~U[20,500], 32 q / 8 kv heads, head_dim 128, b=16, "
                                               "bf16 (Llama-3-8B-shaped layer)"),
    "long": dict(partition_tokens=512, fused=True, desc="16 seqs, L log-uniform [4096,32768], 32 q / 8 kv heads, head_dim 128, "
                                            "b=16, bf16, 512-token partitions + merge"),
    "prefix": dict(partition_tokens=256, cascade=2048, fused=True,
                   desc="128 seqs sharing a 2048-token (128-block) prefix + U[64,1024] private suffix, 32 q / 8 kv "
                        "heads, head_dim 128, b=16, bf16; cascade: the prefix read once for all sequences, "
                        "256-token suffix partitions + merge"),
    "spec": dict(partition_tokens=None, desc="256 seqs, L~U[1024,8192], 4 causal query tokens, 64 q / 8 kv heads, "
                                             "head_dim 128, b=16, bf16"),
    "tiny": dict(partition_tokens=None, desc="4 seqs L={1,17,33,64}, 4 q / 2 kv heads, head_dim 64, b=16, fp32"),
    # int8 KV pools (one fp32 scale per block and kv head) on the same shapes and lengths
    "batch64_int8": dict(partition_tokens=None, base="batch64", int8=True,
                         desc="batch64 with int8 K/V pools + per-(block, kv head) scales, bf16 q"),
    "long_int8": dict(partition_tokens=512, base="long", int8=True,
                      desc="long with int8 K/V pools + per-(block, kv head) scales, bf16 q, 512-token partitions"),
    # FP8 (E4M3) KV pools, same shapes and lengths
    "batch64_fp8": dict(partition_tokens=None, base="batch64", fp8=True,
                        desc="batch64 with FP8 E4M3 K/V pools + per-(block, kv head) scales, bf16 q"),
    "long_fp8": dict(partition_tokens=512, base="long", fp8=True,
                     desc="long with FP8 E4M3 K/V pools + per-(block, kv head) scales, bf16 q, 512-token partitions"),
    # paged (chunked) prefill: a step is one pa_write_kv_varlen + one pa_prefill call
    "prefill": dict(partition_tokens=None, kind="prefill",
                    desc="16 seqs, chunks of U[512,2048] new tokens after paged histories of U[0,4096], 32 q / 8 kv "
                         "heads, head_dim 128, b=16, bf16 (causal attention over history + chunk)"),
    # copy-on-write block copies: one pa_copy_blocks call over many (source, destination) pairs
    "cow_copy": dict(partition_tokens=None, kind="copy",
                     desc="pa_copy_blocks of 4096 block pairs, 8 kv heads x 16 positions x 128 bf16 per block "
                          "(32 KiB of K and 32 KiB of V each), pools of 8192 blocks"),
}
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak


def kv_bytes_per_position(num_kv_heads: int, head_dim: int, itemsize: int) -> int:
    """K and V bytes one position holds in one layer: 2 * Hkv * D * sizeof(kv)
    (4096 B for 8 kv heads x 128 x bf16; the per-layer figure of [P2] section 1)."""
    return 2 * num_kv_heads * head_dim * itemsize


def _scale_bytes_per_block(case) -> int:
    """8-bit pools: the K and V fp32 scales of one block (all kv heads); 0 for float pools."""
    return 2 * 4 * case.k_pool.shape[1] if hasattr(case, "scales") else 0


def algorithmic_bytes(case) -> int:
    """Bytes one decode call must move: every visible K/V row once, q once, the fp32 output
    once, the used block-table entries and the lengths (4 bytes each), and for int8 pools the
    scales of every used block. Partials of a split run are overhead, not part of this figure."""
    b, t, hq, d = case.q.shape
    hkv = case.k_pool.shape[1]
    isz = case.k_pool.element_size()
    lens = [int(x) for x in case.seq_lens]
    blocks = sum(-(-L // case.block_size) for L in lens)
    kv = sum(lens) * kv_bytes_per_position(hkv, d, isz) + blocks * _scale_bytes_per_block(case)
    q = b * t * hq * d * case.q.element_size()
    out = b * t * hq * d * 4
    tables = 4 * blocks + 4 * b
    return kv + q + out + tables


def unique_bytes(case) -> int:
    """Like algorithmic_bytes, but a physical block shared by several tables counts once."""
    b, t, hq, d = case.q.shape
    hkv = case.k_pool.shape[1]
    isz = case.k_pool.element_size()
    bs = case.block_size
    seen = {}
    for i, row in enumerate(case.table_rows):
        L = int(case.seq_lens[i])
        for j, phys in enumerate(row):
            seen[phys] = max(seen.get(phys, 0), min(bs, L - j * bs))
    kv = sum(seen.values()) * kv_bytes_per_position(hkv, d, isz) + len(seen) * _scale_bytes_per_block(case)
    return kv + b * t * hq * d * (case.q.element_size() + 4) + 4 * sum(len(r) for r in case.table_rows) + 4 * b


def library_sha256() -> str:
    """Hash of the built libpa.so, the code whose traffic a summary records (the build is
    byte-reproducible, so a change of comments leaves it alone and any code change does not)."""
    from paged_kv_cache_69_amd import LIB_PATH

    h = hashlib.sha256()
    with open(LIB_PATH, "rb") as fh:
        h.update(fh.read())
    return h.hexdigest()


def read_summary(path: str) -> dict:
    """``key = value`` lines of a profiles/ summary (other lines ignored)."""
    out = {}
    with open(path) as fh:
        for line in fh:
            m = re.match(r"^([a-z_0-9]+) = (.*)$", line.strip())
            if m:
                out[m.group(1)] = m.group(2)
    return out


def traffic_from_profiles(workload: str):
    """HBM bytes per attention call from profiles/traffic_decode_<workload>.txt (traffic_prefill.txt for
    the prefill workload), or None when the summary
    is missing or was taken from another build of the library."""
    kind = WORKLOADS.get(workload, {}).get("kind", "decode")
    path = os.path.join(PROFILES, f"traffic_decode_{workload}.txt" if kind == "decode" else f"traffic_{workload}.txt")
    if not os.path.exists(path):
        return None
    s = read_summary(path)
    if s.get("library_sha256") != library_sha256():
        return None
    return int(float(s["traffic_bytes_per_call"]))


class Replica:
    """One independent copy of a step's device inputs, with ctypes arguments prepacked."""

    def __init__(self, pa, case, src, partition_tokens, variant=0, fused=False, cascade=0):
        import ctypes

        import torch

        self.t = {k: v.clone() for k, v in src.items()}
        self.out = torch.empty(case.q.shape, dtype=torch.float32, device=src["q"].device)
        self.lib = pa.load_library()
        self.dims = pa.make_dims(self.t["q"], self.t["k_pool"], self.t["block_tables"], out_dtype=torch.float32,
                                 variant=variant, split_schedule=SPLIT_SCHEDULE)
        kd = case.k_pool.shape
        self.int8 = "scales" in src
        code = pa.dtype_code(case.k_new.dtype)
        self.wdims = pa.PaDims(case.q.shape[0], case.q.shape[1], kd[1], kd[1], kd[3], kd[2], kd[0],
                               case.block_tables.shape[1], code, pa.dtype_code(case.k_pool.dtype), code, 0)
        self.scale = ctypes.c_float(case.scale)
        self.pt = partition_tokens
        self.max_len = case.max_seq_len
        self.ws = None
        self.cascade = cascade
        if partition_tokens:
            if cascade:
                n = pa.cascade_workspace_bytes(self.t["q"], self.t["k_pool"], self.t["block_tables"], cascade,
                                               self.max_len, partition_tokens)
            else:
                n = pa.workspace_bytes(self.t["q"], self.t["k_pool"].view(torch.int8) if self.int8 else
                                       self.t["k_pool"], self.t["block_tables"], self.max_len, partition_tokens,
                                       split_schedule=SPLIT_SCHEDULE)
            self.ws = torch.empty(n, dtype=torch.uint8, device=src["q"].device)
        p = {k: v.data_ptr() for k, v in self.t.items()}
        scales = (p["scales"],) if self.int8 else ()
        self.write_args = (ctypes.byref(self.wdims), p["k_new"], p["v_new"], p["k_pool"], p["v_pool"], *scales,
                           p["block_tables"], p["positions"])
        self.dec_args = (ctypes.byref(self.dims), p["q"], p["k_pool"], p["v_pool"], *scales, p["block_tables"],
                         p["seq_lens"], self.scale)
        sfx = ("_fp8" if case.k_pool.dtype == torch.float8_e4m3fn else "_int8") if self.int8 else ""
        self.f_write = getattr(self.lib, "pa_write_kv" + sfx)
        self.f_decode = getattr(self.lib, "pa_decode" + sfx)
        self.f_split = getattr(self.lib, "pa_decode_partitioned" + sfx)
        # 8-bit pools append with their own append call
        self.fused = fused and not self.int8
        self.fused_args = (ctypes.byref(self.dims), p["q"], p["k_new"], p["v_new"], p["k_pool"], p["v_pool"],
                           p["block_tables"], p["seq_lens"], self.scale)

    def step(self, stream):
        """One whole decode step: the fused append + decode call where there is one, else the two calls."""
        if self.fused:
            self.call(stream)
        else:
            self.write(stream)
            self.decode(stream)

    def call(self, stream):
        """The step's attention call, the one the roofline times: the fused call, or the decode call."""
        if not self.fused:
            self.decode(stream)
            return
        if self.cascade:
            st = self.lib.pa_write_kv_decode_cascade(*self.fused_args, self.out.data_ptr(), self.cascade, self.max_len,
                                                     self.pt, self.ws.data_ptr(), self.ws.numel(), stream)
        elif self.ws is None:
            st = self.lib.pa_write_kv_decode(*self.fused_args, self.out.data_ptr(), stream)
        else:
            st = self.lib.pa_write_kv_decode_partitioned(*self.fused_args, self.out.data_ptr(), self.max_len, self.pt,
                                                         self.ws.data_ptr(), self.ws.numel(), stream)
        if st:
            raise RuntimeError(f"write_kv_decode: {st}")

    def write(self, stream):
        st = self.f_write(*self.write_args, stream)
        if st:
            raise RuntimeError(f"pa_write_kv: {st}")

    def decode(self, stream):
        if self.cascade:
            st = self.lib.pa_decode_cascade(*self.dec_args, self.out.data_ptr(), self.cascade, self.max_len, self.pt,
                                            self.ws.data_ptr(), self.ws.numel(), stream)
        elif self.ws is None:
            st = self.f_decode(*self.dec_args, self.out.data_ptr(), stream)
        else:
            st = self.f_split(*self.dec_args, self.out.data_ptr(), self.max_len, self.pt,
                                                self.ws.data_ptr(), self.ws.numel(), stream)
        if st:
            raise RuntimeError(f"decode: {st}")


def measure_gpu(pa, case, partition_tokens, steps, warmup, variant=0, graphs=True, fused=False, cascade=0):
    """Returns (seconds per step, ms per decode call, replica count). Without ``graphs`` both come
    from eagerly launched steps (counter-collection runs only; the call time then includes the
    KV writes)."""
    import ctypes

    import torch

    dev = torch.device("cuda:0")
    keys = ["q", "k_new", "v_new", "k_pool", "v_pool", "block_tables", "seq_lens", "positions"]
    if hasattr(case, "scales"):
        keys += ["scales"]
    src = {k: getattr(case, k).to(dev) for k in keys}
    touched = unique_bytes(case)  # a block shared by several tables is cached once
    n_rep = REPLICAS or max(1, min(64, math.ceil(COLD_BYTES / touched)))
    reps = [Replica(pa, case, src, partition_tokens, variant, fused, cascade) for _ in range(n_rep)]
    del src
    torch.cuda.synchronize()

    def sh():
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    # untimed warmup, eager
    for s in range(warmup):
        reps[s % n_rep].step(sh())
    torch.cuda.synchronize()

    # Timed region A: the K steps as HIP graph replays (one graph per chunk of consecutive steps).
    def capture(count):
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            with torch.cuda.graph(g, stream=side):
                for c in range(count):
                    reps[c % n_rep].step(sh())
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        return g

    t0 = t1 = 0.0
    if graphs:
        chunk = n_rep
        full = capture(chunk)
        rem = steps % chunk
        tail = capture(rem) if rem else None
        full.replay()  # instantiate/upload once, outside the timed region
        if tail is not None:
            tail.replay()
        torch.cuda.synchronize()

        t0 = time.perf_counter()
        for _ in range(steps // chunk):
            full.replay()
        if tail is not None:
            tail.replay()
        torch.cuda.synchronize()
        t1 = time.perf_counter()

    # Timed region B: the decode calls alone, K of them back to back (replicas rotating), between
    # one pair of HIP events on the stream they run on. With graphs the calls are one captured
    # graph, so the figure is the kernels' own time plus the small gaps between graph nodes; a
    # partitioned call counts both of its kernels.
    stream = torch.cuda.current_stream()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    if graphs:
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            with torch.cuda.graph(g, stream=side):
                for s in range(steps):
                    reps[s % n_rep].call(sh())
        stream.wait_stream(side)
        g.replay()  # upload, untimed
        torch.cuda.synchronize()
        ev0.record(stream)
        g.replay()
        ev1.record(stream)
        torch.cuda.synchronize()
        del g
    else:
        handle = ctypes.c_void_p(stream.cuda_stream)
        torch.cuda.synchronize()
        e0 = time.perf_counter()
        ev0.record(stream)
        for s in range(steps):
            reps[s % n_rep].step(handle)
        ev1.record(stream)
        torch.cuda.synchronize()
        t0, t1 = e0, time.perf_counter()
    call_ms = ev0.elapsed_time(ev1) / steps
    floor = time_first_tile(reps, case, steps) if graphs and case.block_size * case.k_pool.shape[3] * \
        case.k_pool.element_size() <= 16384 else None
    if floor is not None and PAGED_PROBE:
        floor.update(time_paged_read(reps, case, steps))
    del reps
    torch.cuda.empty_cache()
    return (t1 - t0) / steps, call_ms, n_rep, floor


def probe_library():
    """libpa_probe.so (the measurement probes), loaded once with its signatures declared."""
    import ctypes

    global _PROBE
    if _PROBE is None:
        from paged_kv_cache_69_amd._build import PROBE_LIB_PATH

        if not os.path.exists(PROBE_LIB_PATH):
            raise RuntimeError(f"{PROBE_LIB_PATH} is missing: run __graft_entry__.build() first")
        lib = ctypes.CDLL(PROBE_LIB_PATH)
        P, I32 = ctypes.c_void_p, ctypes.c_int32
        lib.pa_probe_stream_read.argtypes = [P, ctypes.c_size_t, I32, I32, P, P]
        lib.pa_probe_stream_read.restype = ctypes.c_int
        lib.pa_probe_first_tile.argtypes = [P, P, P, P, I32, I32, I32, I32, I32, I32, I32, P, P]
        lib.pa_probe_first_tile.restype = ctypes.c_int
        lib.pa_probe_paged_read.argtypes = [P, P, P, P, I32, I32, I32, I32, I32, I32, I32, I32, I32, P, P]
        lib.pa_probe_paged_read.restype = ctypes.c_int
        lib.pa_probe_mfma.argtypes = [I32, I32, I32, P, P]
        lib.pa_probe_mfma.restype = ctypes.c_int
        _PROBE = lib
    return _PROBE


_PROBE = None
_STREAM = None
_MFMA = None


def calibrate_stream(runs: int = 5):
    """The best rate (GB/s) the streaming-read probe reaches over STREAM_BYTES, over launch shapes of 2048
    to 8192 workgroups and 4 or 8 loads in flight per thread; each shape's figure is the average of
    ``runs`` launches between HIP events on the stream they run on. Measured once per process."""
    import ctypes

    import torch

    global _STREAM
    if _STREAM is not None:
        return _STREAM
    lib = probe_library()
    buf = torch.empty(STREAM_BYTES // 4, dtype=torch.int32, device="cuda:0").random_(generator=torch.Generator(
        device="cuda:0").manual_seed(5))
    best = (0.0, None)
    stream = torch.cuda.current_stream()
    h = ctypes.c_void_p(stream.cuda_stream)
    for wg in (2048, 4096, 8192):
        out = torch.empty(wg, dtype=torch.int32, device="cuda:0")
        for unroll in (4, 8):
            if lib.pa_probe_stream_read(buf.data_ptr(), STREAM_BYTES, wg, unroll, out.data_ptr(), h):
                raise RuntimeError("pa_probe_stream_read failed")
            ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            ev0.record(stream)
            for _ in range(runs):
                lib.pa_probe_stream_read(buf.data_ptr(), STREAM_BYTES, wg, unroll, out.data_ptr(), h)
            ev1.record(stream)
            torch.cuda.synchronize()
            gbps = STREAM_BYTES / (ev0.elapsed_time(ev1) / runs * 1e-3) / 1e9
            if gbps > best[0]:
                best = (gbps, {"workgroups": wg, "loads_in_flight_per_thread": unroll})
    del buf
    torch.cuda.empty_cache()
    _STREAM = {"stream_gbps": round(best[0], 1), "stream_launch": best[1], "stream_bytes": STREAM_BYTES}
    return _STREAM


def calibrate_mfma(runs: int = 3, iters: int = 4000):
    """The bf16 matrix rate (TFLOP/s) this GPU sustains: pa_probe_mfma with 2 and 4 waves per SIMD
    (512 and 1024 workgroups), best of the two, alone and with 2 fp32 FMAs after each MFMA (about the
    prefill kernel's ratio of other vector instructions to MFMAs); each figure the average of ``runs``
    launches between HIP events on the stream they run on. Measured once per process."""
    import ctypes

    import torch

    global _MFMA
    if _MFMA is not None:
        return _MFMA
    lib = probe_library()
    stream = torch.cuda.current_stream()
    h = ctypes.c_void_p(stream.cuda_stream)
    res = {}
    for nv in (0, 2):
        best = (0.0, None)
        for wg in (512, 1024):
            out = torch.empty(wg * 256, dtype=torch.float32, device="cuda:0")
            if lib.pa_probe_mfma(wg, 100, nv, out.data_ptr(), h):
                raise RuntimeError("pa_probe_mfma failed")
            ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            ev0.record(stream)
            for _ in range(runs):
                lib.pa_probe_mfma(wg, iters, nv, out.data_ptr(), h)
            ev1.record(stream)
            torch.cuda.synchronize()
            flops = wg * 4 * iters * 8 * 16384
            tflops = flops / (ev0.elapsed_time(ev1) / runs * 1e-3) / 1e12
            if tflops > best[0]:
                best = (tflops, wg // 256)
        res["mfma_tflops" if nv == 0 else "mfma_tflops_2fma"] = round(best[0], 1)
        res["waves_per_simd" if nv == 0 else "waves_per_simd_2fma"] = best[1]
    _MFMA = res
    return _MFMA


def _graph_us(launch, reps, steps):
    """Average duration (us) of ``launch(replica, stream_handle)`` over one graph of ``steps`` launches with
    the replicas rotating, between HIP events on the stream the graph runs on (after one warm replay)."""
    import ctypes

    import torch

    stream = torch.cuda.current_stream()
    for s in range(len(reps)):
        launch(reps[s], ctypes.c_void_p(stream.cuda_stream))
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            for s in range(steps):
                launch(reps[s % len(reps)], ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    stream.wait_stream(side)
    g.replay()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    g.replay()
    ev1.record(stream)
    torch.cuda.synchronize()
    us = ev0.elapsed_time(ev1) / steps * 1e3
    del g
    return us


def time_first_tile(reps, case, steps):
    """Average duration (us) of the first-tile probe over the decode call's own replicas, launched and
    timed like the decode calls (one graph of ``steps`` launches, replicas rotating, HIP events around
    it): the loads a decode workgroup waits for before its first tile, with nothing else. Both forms:
    length and table entry issued together (as the kernels do), and length -> table -> tile."""
    import torch

    lib = probe_library()
    b, hkv = case.q.shape[0], case.k_pool.shape[1]
    n, _, bs, d = case.k_pool.shape
    row_bytes = d * case.k_pool.element_size()
    out = torch.empty(b * hkv, dtype=torch.int32, device="cuda:0")
    res = {}
    for dependent in (0, 1):
        def launch(r, h):
            t = r.t
            st = lib.pa_probe_first_tile(t["k_pool"].data_ptr(), t["v_pool"].data_ptr(), t["block_tables"].data_ptr(),
                                         t["seq_lens"].data_ptr(), b, hkv, case.block_tables.shape[1], n, bs,
                                         row_bytes, dependent, out.data_ptr(), h)
            if st:
                raise RuntimeError(f"pa_probe_first_tile: {st}")
        res["floor_dependent_us" if dependent else "floor_us"] = round(_graph_us(launch, reps, steps), 3)
    return res


def time_paged_read(reps, case, steps):
    """The paged-read probe over the decode call's own replicas and tables (every K/V block the call
    reads, no arithmetic), timed like the decode calls, at its best over launch shapes: 1, 4, 16 or 64
    blocks per wave, 1, 2 or 4 blocks in flight per wave, plain or nontemporal loads. Returns the rate (GB/s)
    of the best shape and that shape, or {} when the block is not 1, 2, 4 or 8 KiB per kv head."""
    import torch

    lib = probe_library()
    b, hkv = case.q.shape[0], case.k_pool.shape[1]
    n, _, bs, d = case.k_pool.shape
    mb = case.block_tables.shape[1]
    row_bytes = d * case.k_pool.element_size()
    if bs * row_bytes not in (1024, 2048, 4096, 8192):
        return {}
    blocks = int(((case.seq_lens.cpu().long() + bs - 1) // bs).clamp(max=mb).sum())
    nbytes = blocks * hkv * 2 * bs * row_bytes
    best = (0.0, None)
    for bpw in (1, 4, 16, 64):
        groups = (mb + 4 * bpw - 1) // (4 * bpw)
        out = torch.empty(b * groups * hkv, dtype=torch.int32, device="cuda:0")
        for unroll in (1, 2, 4):
            for nt in (0, 1):
                def launch(r, h):
                    t = r.t
                    st = lib.pa_probe_paged_read(t["k_pool"].data_ptr(), t["v_pool"].data_ptr(),
                                                 t["block_tables"].data_ptr(), t["seq_lens"].data_ptr(), b, hkv, mb,
                                                 n, bs, row_bytes, bpw, unroll, nt, out.data_ptr(), h)
                    if st:
                        raise RuntimeError(f"pa_probe_paged_read: {st}")
                gbps = nbytes / (_graph_us(launch, reps, steps) * 1e-6) / 1e9
                if gbps > best[0]:
                    best = (gbps, {"blocks_per_wave": bpw, "blocks_in_flight_per_wave": unroll, "nontemporal": nt})
    return {"paged_read_gbps": round(best[0], 1), "paged_read_launch": best[1], "paged_read_bytes": nbytes}


def host_cores() -> int:
    """Cores this process may use: the affinity mask, capped by OMP_NUM_THREADS when the host sets it."""
    n = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    env = os.environ.get("OMP_NUM_THREADS", "")
    return max(1, min(n, int(env))) if env.isdigit() and int(env) > 0 else max(1, n)


def cpu_baseline(case, budget_s: float):
    """The float64 oracle (KV write + decode) on this host, over a bounded sample of the workload: the
    first n sequences, n grown until one pass takes about ``budget_s`` or covers the whole batch, and a
    pass shorter than the budget repeated until the budget is spent. Measured twice: on every core (the
    KV write, then one oracle decode per sequence spread over a thread pool of that many workers, one
    BLAS thread each; numpy drops the GIL in its gathers and products), and on one thread."""
    import concurrent.futures as cf

    import numpy as np
    import torch
    from threadpoolctl import threadpool_limits

    import oracle

    def npbits(t):
        t = t.detach().cpu().contiguous()
        return t.view(torch.int16).numpy().view(np.uint16) if t.element_size() == 2 else \
            t.view(torch.int32).numpy().view(np.uint32)

    b = case.q.shape[0]
    kp_all, vp_all = npbits(case.k_pool), npbits(case.v_pool)
    q_all = case.q.float().numpy()
    tables_all, lens_all = case.block_tables.numpy(), case.seq_lens.numpy()

    def one_pass(n, pool):
        sl = slice(0, n)
        kp, vp = oracle.write_kv(kp_all, vp_all, npbits(case.k_new[sl]), npbits(case.v_new[sl]),
                                 tables_all[sl], case.positions[sl].numpy(), case.block_size)
        as_f = (lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).float().numpy()) \
            if kp.dtype == np.uint16 else (lambda a: a.view(np.float32))
        kf, vf = as_f(kp), as_f(vp)

        def seq(i):
            return oracle.decode(q_all[i:i + 1], kf, vf, tables_all[i:i + 1], lens_all[i:i + 1], case.scale,
                                 case.block_size)

        if pool is None:
            for i in range(n):
                seq(i)
        else:
            list(pool.map(seq, range(n)))

    def timed(cores):
        pool = cf.ThreadPoolExecutor(max_workers=cores) if cores > 1 else None
        try:
            # one BLAS thread per worker: the workers already use every core (BLAS threads on top of
            # them oversubscribe the host; the products are small)
            with threadpool_limits(limits=1):
                n = 1
                while True:
                    t0 = time.perf_counter()
                    one_pass(n, pool)
                    dt = time.perf_counter() - t0
                    if dt >= budget_s or n >= b:
                        break
                    n = min(b, max(n + 1, int(n * min(8.0, 1.2 * budget_s / max(dt, 1e-3)))))
                passes, total = 1, dt
                while total < budget_s:
                    t0 = time.perf_counter()
                    one_pass(n, pool)
                    total += time.perf_counter() - t0
                    passes += 1
        finally:
            if pool is not None:
                pool.shutdown()
        tokens = n * case.q.shape[1] * passes
        return round(tokens / total, 2), (f"KV write + float64 decode of the first {n} of {b} sequences "
                                          f"({int(case.seq_lens[:n].sum())} positions) x {passes} pass(es), "
                                          f"{cores} thread(s), {total:.1f} s")

    cores = host_cores()
    multi, multi_sample = timed(cores)
    single, single_sample = timed(1)
    return {"value": multi, "unit": "tokens/s", "cores": cores, "kind": "oracle", "sample": multi_sample,
            "single_thread": {"value": single, "cores": 1, "sample": single_sample}}


def calibrate_copy(n_runs: int = 3):
    """A plain elementwise kernel of known traffic (reads and writes CALIBRATION_BYTES), launched so a
    rocprofv3 counter run of this process can scale its FETCH_SIZE / WRITE_SIZE readings."""
    import torch

    src = torch.ones(CALIBRATION_BYTES // 4, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(n_runs):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    del src, dst
    torch.cuda.empty_cache()


def prefill_flops(case) -> int:
    """Matrix flops of one pa_prefill call: for every chunk token, query head and visible position,
    a 128-long dot product for the score and a 128-long update of the output, 2 flops per multiply-add:
    4 * D * Hq * sum_i sum_j (h_i + j + 1)."""
    return 4 * case.q.shape[2] * case.q.shape[1] * case.attended_pairs()


def prefill_algorithmic_bytes(case) -> int:
    """Bytes a prefill call must move at least: each sequence's K/V rows once (history + chunk, every kv
    head), q once, the fp32 output once, the used table entries, the lengths and q_start."""
    hkv, d = case.k_pool.shape[1], case.k_pool.shape[3]
    lens = [h + n for h, n in zip(case.histories, case.chunks)]
    blocks = sum(-(-L // case.block_size) for L in lens)
    total_q, hq, _ = case.q.shape
    return (sum(lens) * kv_bytes_per_position(hkv, d, case.k_pool.element_size())
            + total_q * hq * d * (case.q.element_size() + 4) + 4 * blocks + 4 * len(lens) + 4 * (len(lens) + 1))


def run_prefill_workload(pa, name, steps, warmup, graphs=True):
    """The prefill workload: a step is one pa_write_kv_varlen (the chunks' K/V into the pools) and one
    pa_prefill call, timed like the decode steps (graphs of whole steps; HIP events around a graph of
    the prefill calls alone)."""
    import ctypes

    import torch

    from workloads import make_prefill_case

    spec = WORKLOADS[name]
    case = make_prefill_case(name, pool_device="cuda:0")
    dev = torch.device("cuda:0")
    keys = ("q", "k_new", "v_new", "k_pool", "v_pool", "block_tables", "seq_lens", "q_start")
    touched = sum(getattr(case, k).numel() * getattr(case, k).element_size() for k in keys) + case.q.numel() * 4
    n_rep = max(1, min(8, math.ceil(COLD_BYTES / touched)))
    reps = []
    for _ in range(n_rep):
        t = {k: getattr(case, k).to(dev, copy=True) for k in keys}
        t["out"] = torch.empty(case.q.shape, dtype=torch.float32, device=dev)
        reps.append(t)
    lib = pa.load_library()
    hq, hkv, d = case.q.shape[1], case.k_pool.shape[1], case.q.shape[2]
    dims = pa.PaDims(len(case.chunks), case.max_chunk, hq, hkv, d, case.block_size, case.k_pool.shape[0],
                     case.block_tables.shape[1], pa.PA_BF16, pa.PA_BF16, pa.PA_F32, 0)
    wdims = pa.PaDims(len(case.chunks), case.max_chunk, hkv, hkv, d, case.block_size, case.k_pool.shape[0],
                      case.block_tables.shape[1], pa.PA_BF16, pa.PA_BF16, pa.PA_BF16, 0)
    scale = ctypes.c_float(case.scale)

    def write(t, h):
        st = lib.pa_write_kv_varlen(ctypes.byref(wdims), t["k_new"].data_ptr(), t["v_new"].data_ptr(),
                                    t["k_pool"].data_ptr(), t["v_pool"].data_ptr(), t["block_tables"].data_ptr(),
                                    t["seq_lens"].data_ptr(), t["q_start"].data_ptr(), h)
        if st:
            raise RuntimeError(f"pa_write_kv_varlen: {st}")

    def attend(t, h):
        st = lib.pa_prefill(ctypes.byref(dims), t["q"].data_ptr(), t["k_pool"].data_ptr(), t["v_pool"].data_ptr(),
                            t["block_tables"].data_ptr(), t["seq_lens"].data_ptr(), t["q_start"].data_ptr(), scale,
                            t["out"].data_ptr(), h)
        if st:
            raise RuntimeError(f"pa_prefill: {st}")

    def sh():
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    for s_ in range(warmup):
        write(reps[s_ % n_rep], sh())
        attend(reps[s_ % n_rep], sh())
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    if graphs:
        def capture(fn_list):
            g = torch.cuda.CUDAGraph()
            side = torch.cuda.Stream()
            side.wait_stream(stream)
            with torch.cuda.stream(side):
                with torch.cuda.graph(g, stream=side):
                    for s_ in range(steps):
                        for fn in fn_list:
                            fn(reps[s_ % n_rep], sh())
            stream.wait_stream(side)
            g.replay()  # upload, untimed
            torch.cuda.synchronize()
            return g

        g_step = capture([write, attend])
        t0 = time.perf_counter()
        g_step.replay()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        del g_step
        g_call = capture([attend])
        ev0.record(stream)
        g_call.replay()
        ev1.record(stream)
        torch.cuda.synchronize()
        del g_call
    else:
        h = ctypes.c_void_p(stream.cuda_stream)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        ev0.record(stream)
        for s_ in range(steps):
            write(reps[s_ % n_rep], h)
            attend(reps[s_ % n_rep], h)
        ev1.record(stream)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
    call_ms = ev0.elapsed_time(ev1) / steps
    sec_per_step = (t1 - t0) / steps
    flops = prefill_flops(case)
    tflops = flops / (call_ms * 1e-3) / 1e12
    tokens = sum(case.chunks)
    mfma = calibrate_mfma() if MFMA_PROBE else None
    res = {
        "tokens_per_s": tokens / sec_per_step,
        "ms_per_step": sec_per_step * 1e3,
        "achieved_gbps": prefill_algorithmic_bytes(case) / sec_per_step / 1e9,
        "roofline": {"bound": "mfma", "achieved": round(tflops, 1), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                     "traffic": traffic_from_profiles(name),
                     "kernel": "prefill_mfma_kernel (one pa_prefill call)", "flops_per_launch": flops,
                     "algorithmic_bytes_per_launch": prefill_algorithmic_bytes(case),
                     "avg_launch_us": round(call_ms * 1e3, 3), "launches_timed": steps,
                     **({"measured_mfma_tflops": mfma["mfma_tflops"],
                         "frac_of_measured_mfma": round(tflops / mfma["mfma_tflops"], 4),
                         "measured_mfma_tflops_2fma": mfma["mfma_tflops_2fma"]} if mfma else {})},
        "config": {"workload": f"{name}: {spec['desc']}", "num_seqs": len(case.chunks), "chunk_tokens": tokens,
                   "histories": sum(case.histories), "replicas": n_rep,
                   "step": "pa_write_kv_varlen call + pa_prefill call"},
        "dtype": "bf16",
    }
    del reps
    torch.cuda.empty_cache()
    return res


def run_copy_workload(pa, name, steps, warmup, graphs=True):
    """Copy-on-write block copies: one pa_copy_blocks call moves 4096 blocks of K and of V to fresh
    blocks; algorithmic bytes = 2 (read + write) x 2 (K, V) x 4096 x 32 KiB."""
    import ctypes

    import torch

    spec = WORKLOADS[name]
    n_blocks, hkv, b, d, n_pairs = 8192, 8, 16, 128, 4096
    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev).manual_seed(1008)
    k_pool = torch.randn((n_blocks, hkv, b, d), generator=gen, device=dev).to(torch.bfloat16)
    v_pool = torch.randn((n_blocks, hkv, b, d), generator=gen, device=dev).to(torch.bfloat16)
    perm = torch.randperm(n_blocks, generator=torch.Generator().manual_seed(1009))
    pairs = torch.stack([perm[:n_pairs], perm[n_pairs:2 * n_pairs]], dim=1).to(torch.int32).to(dev).contiguous()
    lib = pa.load_library()
    from paged_kv_cache_69_amd import blocks as _blocks

    _blocks._bind(lib)
    dims = pa.PaDims(0, 1, hkv, hkv, d, b, n_blocks, 1, pa.PA_BF16, pa.PA_BF16, pa.PA_BF16, 0)
    block_bytes = hkv * b * d * 2
    algo = 2 * 2 * n_pairs * block_bytes

    def call(h):
        st = lib.pa_copy_blocks(ctypes.byref(dims), k_pool.data_ptr(), v_pool.data_ptr(), None, pairs.data_ptr(), n_pairs,
                                h)
        if st:
            raise RuntimeError(f"pa_copy_blocks: {st}")

    def sh():
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    for _ in range(warmup):
        call(sh())
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    if graphs:
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            with torch.cuda.graph(g, stream=side):
                for _ in range(steps):
                    call(sh())
        stream.wait_stream(side)
        g.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        ev0.record(stream)
        g.replay()
        ev1.record(stream)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        del g
    else:
        h = ctypes.c_void_p(stream.cuda_stream)
        t0 = time.perf_counter()
        ev0.record(stream)
        for _ in range(steps):
            call(h)
        ev1.record(stream)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
    call_ms = ev0.elapsed_time(ev1) / steps
    achieved = algo / (call_ms * 1e-3) / 1e9
    res = {
        "tokens_per_s": n_pairs * b / ((t1 - t0) / steps),  # positions moved per second
        "ms_per_step": (t1 - t0) / steps * 1e3,
        "achieved_gbps": algo / ((t1 - t0) / steps) / 1e9,
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic_from_profiles(name),
                     "kernel": "copy_blocks_kernel (one pa_copy_blocks call)", "bytes_per_launch": algo,
                     "avg_launch_us": round(call_ms * 1e3, 3), "launches_timed": steps},
        "config": {"workload": f"{name}: {spec['desc']}", "block_pairs": n_pairs, "block_bytes": block_bytes},
        "dtype": "bf16",
    }
    del k_pool, v_pool
    torch.cuda.empty_cache()
    return res


def stream_terms(achieved_gbps, bytes_per_launch, launch_us, floor):
    """The call against the measured bounds: the streaming-read rate, the paged-read rate of its own
    tables, and the first-tile floor. model_us = floor + bytes / stream rate; paged_model_us = floor +
    bytes / paged-read rate."""
    out = {}
    if _STREAM is not None:
        out.update(stream_gbps=_STREAM["stream_gbps"], frac_of_stream=round(achieved_gbps / _STREAM["stream_gbps"], 4))
    if floor:
        out.update(floor)
        if _STREAM is not None:
            model = floor["floor_us"] + bytes_per_launch / (_STREAM["stream_gbps"] * 1e3)
            out.update(model_us=round(model, 3), over_model=round(launch_us / model, 4))
        if floor.get("paged_read_gbps"):
            pm = floor["floor_us"] + bytes_per_launch / (floor["paged_read_gbps"] * 1e3)
            out.update(frac_of_paged_read=round(achieved_gbps / floor["paged_read_gbps"], 4),
                       paged_model_us=round(pm, 3), over_paged_model=round(launch_us / pm, 4))
    return out


def run_workload(pa, name, steps, warmup, with_cpu, cpu_budget, variant=0, graphs=True, fused=True):
    import torch

    from workloads import fp8_pools, int8_pools, make_case

    spec = WORKLOADS[name]
    if spec.get("kind") == "prefill":
        return run_prefill_workload(pa, name, steps, warmup, graphs)
    if spec.get("kind") == "copy":
        return run_copy_workload(pa, name, steps, warmup, graphs)
    case = make_case(spec.get("base", name), pool_device="cuda:0")
    if spec.get("int8"):
        case.k_pool, case.v_pool, case.scales = int8_pools(case)
    if spec.get("fp8"):
        case.k_pool, case.v_pool, case.scales = fp8_pools(case)
    b, t = case.q.shape[0], case.q.shape[1]
    rows = case.q.shape[2] // case.k_pool.shape[1] * t
    mfma_ok = (case.k_pool.dtype in (torch.bfloat16, torch.int8, torch.float8_e4m3fn) and case.q.shape[3] == 128
               and rows <= 32)
    fused = fused and spec.get("fused", False) and variant != 1 and mfma_ok
    cascade = spec.get("cascade", 0) if variant != 1 else 0
    sec_per_step, dur_ms, n_rep, floor = measure_gpu(pa, case, spec["partition_tokens"], steps, warmup, variant,
                                                     graphs, fused, cascade)
    # a cascade reads each shared block once: count every physical block once
    algo = unique_bytes(case) if cascade else algorithmic_bytes(case)
    if fused:  # the call also reads the new rows and stores them into the pools
        algo += 2 * case.k_new.numel() * (case.k_new.element_size() + case.k_pool.element_size())
    achieved = algo / (dur_ms * 1e-3) / 1e9
    kernel = "decode_mfma_kernel" if (variant == 2 or (variant == 0 and mfma_ok)) else "decode_valu_kernel"
    if fused:
        kernel += " with the KV append fused in"
    call = ("pa_write_kv_decode" if fused else "pa_decode") + ("_partitioned" if spec["partition_tokens"] else "")
    if spec.get("int8") or spec.get("fp8"):
        call = ("pa_write_kv_decode" if fused else "pa_decode" + ("_partitioned" if spec["partition_tokens"] else "")) + (
            "_fp8" if spec.get("fp8") else "_int8")
    if cascade:
        call = "pa_write_kv_decode_cascade" if fused else "pa_decode_cascade"
        kernel = "cascade_kernel (shared-prefix items and per-sequence items in one launch" + (
            ", the KV append fused in)" if fused else ")")
    kernel += (" + merge_partials_kernel" if spec["partition_tokens"] else "") + f" (one {call} call)"
    traffic = traffic_from_profiles(name) if variant == 0 else None
    res = {
        "tokens_per_s": b * t / sec_per_step,
        "ms_per_step": sec_per_step * 1e3,
        "achieved_gbps": algo / sec_per_step / 1e9,
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic,
                     "kernel": kernel, "bytes_per_launch": algo, "avg_launch_us": round(dur_ms * 1e3, 3),
                     "launches_timed": steps, **stream_terms(achieved, algo, dur_ms * 1e3, floor)},
        "config": {"workload": f"{name}: {spec['desc']}", "num_seqs": b, "q_tokens": t,
                   "kv_positions": case.kv_tokens(), "max_seq_len": case.max_seq_len,
                   "partition_tokens": spec["partition_tokens"], "replicas": n_rep,
                   **({"shared_prefix_tokens": cascade} if cascade else {}),
                   "step": "one fused append + decode call" if fused else "append call + decode call"},
        "dtype": {torch.bfloat16: "bf16", torch.int8: "int8 KV (bf16 q, fp32 scales)",
                  torch.float8_e4m3fn: "fp8 e4m3 KV (bf16 q, fp32 scales)"}.get(case.k_pool.dtype, "f32"),
    }
    if cascade:
        # the roofline counts every shared block once; every sequence reading its whole context is the
        # logical figure (what a decode without the cascade would ask of memory)
        logical = algorithmic_bytes(case)
        res["unique_bytes"] = unique_bytes(case)
        res["logical_bytes"] = logical
        res["achieved_gbps_logical"] = round(logical / (dur_ms * 1e-3) / 1e9, 1)
    if with_cpu:
        res["cpu_baseline"] = cpu_baseline(case, cpu_budget)
    del case
    torch.cuda.empty_cache()
    return res


# ----------------------------------------------------------------------------- profiles/ summaries

def _pmc_rows(directory: str):
    paths = glob.glob(os.path.join(directory, "**", "*counter_collection.csv"), recursive=True)
    if not paths:
        raise FileNotFoundError(f"no *counter_collection.csv under {directory}")
    with open(paths[0], newline="") as fh:
        return list(csv.DictReader(fh))


def _short(name: str) -> str:
    name = re.sub(r"pa::\(anonymous namespace\)::", "", name)
    return re.sub(r"\(pa::DecodeParams\)", "", name).strip()


def summarize_pmc(fetch_dir: str, write_dir: str, bench_log: str, workload: str) -> str:
    """Text summary of one workload's decode-call traffic from a FETCH_SIZE run and a WRITE_SIZE run
    (rocprofv3 --pmc ... --output-format csv) of ``bench.py --workload W --calibrate-copy``."""
    with open(bench_log) as fh:
        line = [ln for ln in fh if ln.startswith("{")][-1]
    rec = json.loads(line)
    algo = int(rec["roofline"].get("bytes_per_launch") or rec["roofline"]["algorithmic_bytes_per_launch"])
    per = {}
    for counter, directory in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        for r in _pmc_rows(directory):
            if r["Counter_Name"] != counter:
                continue
            per.setdefault((counter, _short(r["Kernel_Name"])), []).append(float(r["Counter_Value"]))
    med = {k: statistics.median(v) for k, v in per.items()}
    copy = [k for k in med if "neg" in k[1].lower()]
    cf = [med[k] for k in copy if k[0] == "FETCH_SIZE"]
    cw = [med[k] for k in copy if k[0] == "WRITE_SIZE"]
    if not cf or not cw:
        raise RuntimeError("calibration copy kernel not found in the counter runs")
    f_fac = CALIBRATION_BYTES / (cf[0] * 1024.0)
    w_fac = CALIBRATION_BYTES / (cw[0] * 1024.0)
    kernels = sorted({k[1] for k in med
                      if k[1].startswith("void decode_") or "merge_partials" in k[1] or "prefill_mfma" in k[1]
                      or "copy_blocks" in k[1] or "cascade_kernel" in k[1] or "balanced_kernel" in k[1]})
    lines = [f"# HBM traffic of one decode call, workload {workload}",
             "# FETCH_SIZE and WRITE_SIZE (KiB per dispatch, median over dispatches), each scaled by",
             f"# what it reads for a copy kernel that reads and writes {CALIBRATION_BYTES} bytes.",
             "# commands (from the repository root; the summary itself comes from",
             "#   python bench.py --summarize-pmc /tmp/pa_prof/pmc_fetch_W /tmp/pa_prof/pmc_write_W <bench log> --workload W):",
             f"#   rocprofv3 --pmc FETCH_SIZE --output-format csv -d /tmp/pa_prof/pmc_fetch_{workload} -o run -- "
             f"python3 bench.py --workload {workload} --secondary '' --no-cpu --no-graph --no-stream --no-paged-probe --steps 20 --warmup 5 --calibrate-copy",
             f"#   rocprofv3 --pmc WRITE_SIZE --output-format csv -d /tmp/pa_prof/pmc_write_{workload} -o run -- "
             f"python3 bench.py --workload {workload} --secondary '' --no-cpu --no-graph --no-stream --no-paged-probe --steps 20 --warmup 5 --calibrate-copy",
             f"workload = {workload}",
             f"library_sha256 = {library_sha256()}",
             f"copy_fetch_kib = {cf[0]:.1f}",
             f"copy_write_kib = {cw[0]:.1f}",
             f"fetch_factor = {f_fac:.4f}",
             f"write_factor = {w_fac:.4f}"]
    total = 0.0
    for i, k in enumerate(kernels):
        fk = med.get(("FETCH_SIZE", k), 0.0)
        wk = med.get(("WRITE_SIZE", k), 0.0)
        bytes_k = fk * 1024.0 * f_fac + wk * 1024.0 * w_fac
        total += bytes_k
        lines += [f"kernel_{i} = {k}", f"kernel_{i}_fetch_kib = {fk:.1f}", f"kernel_{i}_write_kib = {wk:.1f}",
                  f"kernel_{i}_bytes = {bytes_k:.0f}"]
    lines += [f"traffic_bytes_per_call = {total:.0f}",
              f"algorithmic_bytes_per_call = {algo}",
              f"traffic_over_algorithmic = {total / algo:.4f}"]
    return "\n".join(lines) + "\n"


def summarize_l2(directory: str, workload: str, command: str) -> str:
    """L2 (TCC) hits and misses per kernel, median over dispatches, from a
    ``rocprofv3 --pmc TCC_HIT_sum TCC_MISS_sum`` run of ``bench.py --workload W``."""
    per = {}
    for r in _pmc_rows(directory):
        if r["Counter_Name"] in ("TCC_HIT_sum", "TCC_MISS_sum"):
            per.setdefault((r["Counter_Name"], _short(r["Kernel_Name"])), []).append(float(r["Counter_Value"]))
    med = {k: statistics.median(v) for k, v in per.items()}
    kernels = sorted({k[1] for k in med
                      if k[1].startswith("void decode_") or "merge_partials" in k[1] or "cascade_kernel" in k[1]
                      or "prefill_mfma" in k[1] or "balanced_kernel" in k[1]})
    lines = [f"# L2 (TCC) hits and misses of one decode call, workload {workload} (median over dispatches)",
             f"# command (from the repository root): {command}",
             f"workload = {workload}", f"library_sha256 = {library_sha256()}"]
    for i, k in enumerate(kernels):
        hit, miss = med.get(("TCC_HIT_sum", k), 0.0), med.get(("TCC_MISS_sum", k), 0.0)
        rate = hit / (hit + miss) if hit + miss else 0.0
        lines += [f"kernel_{i} = {k}", f"kernel_{i}_tcc_hit = {hit:.0f}", f"kernel_{i}_tcc_miss = {miss:.0f}",
                  f"kernel_{i}_l2_hit_rate = {rate:.4f}"]
    return "\n".join(lines) + "\n"


SIMDS = 1024  # 256 compute units x 4 SIMDs
XCDS = 8      # GRBM_GUI_ACTIVE comes back summed over the 8 XCDs' instances


def summarize_counters(directories: list, workload: str, commands: list) -> str:
    """Per-kernel medians (over dispatches) of the SQ / GRBM counters of one or more ``rocprofv3 --pmc``
    runs of ``bench.py --workload W``, with the derived shares: matrix-core busy = SQ_VALU_MFMA_BUSY_CYCLES
    / (GRBM_GUI_ACTIVE / 8 XCDs x 1024 SIMDs); vector-ALU busy = 4 x SQ_ACTIVE_INST_VALU (quad-cycles,
    summed over waves) over the same SIMD-cycles; matrix/vector co-execution =
    SQ_VALU_MFMA_COEXEC_CYCLES over them; a wave's time issuing, waiting to issue, and waiting on its
    counters or a barrier (SQ_ACTIVE_INST_ANY, SQ_WAIT_INST_ANY, SQ_WAIT_ANY over SQ_WAVE_CYCLES); LDS
    bank conflicts per LDS instruction; instructions per wave (SQ_INSTS_VALU counts the MFMAs too). GRBM_GUI_ACTIVE counts GPU-busy cycles once per XCD and rocprofv3 sums the instances, so one
    XCD's share is the kernel's elapsed cycles."""
    per = {}
    for directory in directories:
        for r in _pmc_rows(directory):
            per.setdefault((_short(r["Kernel_Name"]), r["Counter_Name"]), []).append(float(r["Counter_Value"]))
    med = {k: statistics.median(v) for k, v in per.items()}
    kernels = sorted({k[0] for k in med if k[0].startswith("void decode_") or "merge_partials" in k[0]
                      or "prefill_mfma" in k[0] or "balanced_kernel" in k[0] or "cascade_kernel" in k[0]
                      or "copy_blocks" in k[0]})
    lines = [f"# SQ / GRBM counters of one call, workload {workload} (median over dispatches)"]
    lines += [f"# command (from the repository root): {c}" for c in commands]
    lines += [f"workload = {workload}", f"library_sha256 = {library_sha256()}"]
    for i, k in enumerate(kernels):
        lines.append(f"kernel_{i} = {k}")
        names = sorted({c for (kk, c) in med if kk == k})
        for c in names:
            lines.append(f"kernel_{i}_{c} = {med[(k, c)]:.0f}")
        get = lambda c: med.get((k, c))  # noqa: E731
        if get("SQ_VALU_MFMA_BUSY_CYCLES") is not None and get("GRBM_GUI_ACTIVE"):
            lines.append(f"kernel_{i}_elapsed_cycles = {get('GRBM_GUI_ACTIVE') / XCDS:.0f}")
            lines.append(f"kernel_{i}_mfma_busy_frac = "
                         f"{get('SQ_VALU_MFMA_BUSY_CYCLES') / (get('GRBM_GUI_ACTIVE') / XCDS * SIMDS):.4f}")
        el = get("GRBM_GUI_ACTIVE") / XCDS if get("GRBM_GUI_ACTIVE") else None
        if el and get("SQ_ACTIVE_INST_VALU") is not None:
            # quad-cycles summed over waves; one SIMD issues one VALU instruction at a time
            lines.append(f"kernel_{i}_valu_busy_frac = {4 * get('SQ_ACTIVE_INST_VALU') / (el * SIMDS):.4f}")
        if el and get("SQ_VALU_MFMA_COEXEC_CYCLES") is not None:
            lines.append(f"kernel_{i}_valu_mfma_coexec_frac = "
                         f"{get('SQ_VALU_MFMA_COEXEC_CYCLES') / (el * SIMDS):.4f}")
        if get("SQ_WAVE_CYCLES"):
            for c, n in (("SQ_ACTIVE_INST_ANY", "issuing"), ("SQ_WAIT_INST_ANY", "waiting_to_issue"),
                         ("SQ_WAIT_ANY", "waiting_on_counters_or_barrier")):
                if get(c) is not None:
                    lines.append(f"kernel_{i}_wave_time_{n} = {get(c) / get('SQ_WAVE_CYCLES'):.4f}")
        if get("SQ_LDS_BANK_CONFLICT") is not None and get("SQ_INSTS_LDS"):
            lines.append(f"kernel_{i}_lds_bank_conflict_cycles_per_lds_inst = "
                         f"{get('SQ_LDS_BANK_CONFLICT') / get('SQ_INSTS_LDS'):.3f}")
        if get("SQ_WAVES"):
            for c in ("SQ_INSTS_MFMA", "SQ_INSTS_VALU", "SQ_INSTS_LDS", "SQ_INSTS_SALU", "SQ_INSTS_VMEM_RD"):
                if get(c) is not None:
                    lines.append(f"kernel_{i}_{c}_per_wave = {get(c) / get('SQ_WAVES'):.1f}")
    return "\n".join(lines) + "\n"


def summarize_stats(directory: str, command: str, bench_log: str | None = None) -> str:
    """Text summary of a rocprofv3 --kernel-trace --stats run (its *kernel_stats.csv, or the kernels
    of its results database): calls and durations per kernel, plus the bench line's own figure."""
    stats = []
    paths = glob.glob(os.path.join(directory, "**", "*kernel_stats.csv"), recursive=True)
    if paths:
        with open(paths[0], newline="") as fh:
            for r in csv.DictReader(fh):
                stats.append((_short(r["Name"]), int(r["Calls"]), float(r["AverageNs"]), float(r["MinNs"]),
                              float(r["MaxNs"]), float(r["Percentage"])))
    else:
        import sqlite3

        dbs = glob.glob(os.path.join(directory, "**", "*results.db"), recursive=True)
        if not dbs:
            raise FileNotFoundError(f"no kernel stats or results database under {directory}")
        con = sqlite3.connect(dbs[0])
        per = {}
        for name, dur in con.execute("select name, duration from kernels"):
            per.setdefault(_short(name), []).append(float(dur))
        con.close()
        total = sum(sum(v) for v in per.values())
        for name, v in per.items():
            stats.append((name, len(v), sum(v) / len(v), min(v), max(v), 100.0 * sum(v) / total))
    stats.sort(key=lambda r: -r[5])
    out = ["# rocprofv3 --kernel-trace --stats summary", f"# command: {command}", f"# library_sha256 = {library_sha256()}",
           f"{'kernel':80s} {'calls':>7s} {'avg_us':>10s} {'min_us':>10s} {'max_us':>10s} {'pct':>6s}"]
    for name, calls, avg, mn, mx, pct in stats:
        out.append(f"{name[:80]:80s} {calls:7d} {avg / 1e3:10.2f} {mn / 1e3:10.2f} {mx / 1e3:10.2f} {pct:6.2f}")
    if bench_log:
        with open(bench_log) as fh:
            rec = json.loads([ln for ln in fh if ln.startswith("{")][-1])
        out.append(f"# the same run's bench line: attention call avg {rec['roofline']['avg_launch_us']} us over "
                   f"{rec['roofline']['launches_timed']} calls (HIP events around one graph of the calls)")
    return "\n".join(out) + "\n"


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="batch64", choices=sorted(WORKLOADS))
    ap.add_argument("--secondary", default="long,prefix,spec,batch64_int8,long_int8,batch64_fp8,long_fp8,prefill,"
                                           "cow_copy",
                    help="comma-separated workloads also measured and reported under 'secondary' ('' for none)")
    ap.add_argument("--cpu-budget", type=float, default=10.0,
                    help="seconds of oracle work for each cpu_baseline leg (every core, then one thread)")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--variant", type=int, default=0, help="0 auto, 1 vector-ALU kernel, 2 MFMA kernel")
    ap.add_argument("--no-fused", action="store_true",
                    help="time the step as separate pa_write_kv and decode calls on every workload")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="first run a copy kernel of known size (for counter calibration)")
    ap.add_argument("--no-stream", action="store_true", help="skip the streaming-read calibration")
    ap.add_argument("--no-paged-probe", action="store_true", help="skip the paged-read probe sweep")
    ap.add_argument("--no-mfma-probe", action="store_true", help="skip the matrix-rate probe of the prefill line")
    ap.add_argument("--cpu-secondary", default="long",
                    help="comma-separated secondary workloads that also get a cpu_baseline ('' for none)")
    ap.add_argument("--no-graph", action="store_true",
                    help="time eagerly launched steps only (for counter-collection runs; not a headline number)")
    ap.add_argument("--summarize-pmc", nargs=3, metavar=("FETCH_DIR", "WRITE_DIR", "BENCH_LOG"))
    ap.add_argument("--summarize-l2", nargs=2, metavar=("L2_DIR", "COMMAND"))
    ap.add_argument("--replicas", type=int, default=0,
                    help="input copies to rotate over (default: enough to miss every cache; 1: warm)")
    ap.add_argument("--summarize-stats", nargs="+", metavar="DIR COMMAND [BENCH_LOG]")
    ap.add_argument("--summarize-counters", nargs="+", metavar="DIR:COMMAND",
                    help="counter runs of --workload W, each given as its output folder and command joined by '::'")
    ap.add_argument("--split-schedule", type=int, default=0,
                    help="pa_dims.split_schedule of the split calls: 0 the library's choice, 1 one partition per "
                         "wave, 2 two per wave, 3 balanced ranges")
    args = ap.parse_args(argv)
    if args.summarize_pmc:
        print(summarize_pmc(*args.summarize_pmc, args.workload), end="")
        return 0
    if args.summarize_l2:
        print(summarize_l2(args.summarize_l2[0], args.workload, args.summarize_l2[1]), end="")
        return 0
    if args.summarize_stats:
        print(summarize_stats(*args.summarize_stats), end="")
        return
    if args.summarize_counters:
        pairs = [x.split("::", 1) for x in args.summarize_counters]
        print(summarize_counters([d for d, _ in pairs], args.workload, [c for _, c in pairs]), end="")
        return 0
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported: the decode step runs on one "
              "GPU and needs no collectives: its (sequence, kv head) units split across GPUs with no exchange.",
              file=sys.stderr)
        return 2
    global REPLICAS, SPLIT_SCHEDULE, PAGED_PROBE, MFMA_PROBE
    REPLICAS = max(0, args.replicas)
    SPLIT_SCHEDULE = args.split_schedule
    PAGED_PROBE = not args.no_paged_probe
    MFMA_PROBE = not args.no_mfma_probe

    import torch

    import paged_kv_cache_69_amd as pa

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    pa.load_library()
    if args.calibrate_copy:
        calibrate_copy()
    if not args.no_stream:
        calibrate_stream()
    main_res = run_workload(pa, args.workload, args.steps, args.warmup, not args.no_cpu, args.cpu_budget,
                            args.variant, not args.no_graph, not args.no_fused)
    line = {
        "metric": METRIC,
        "value": round(main_res["tokens_per_s"], 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(main_res["ms_per_step"], 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": main_res["dtype"],
        "data": "synthetic" + (" (eager launches, no graphs)" if args.no_graph else ""),
        "config": main_res["config"],
        "achieved_gbps": round(main_res["achieved_gbps"], 1),
        "hbm_frac": round(main_res["achieved_gbps"] / HBM_PEAK_GBPS, 4),
        "roofline": main_res["roofline"],
    }
    if "cpu_baseline" in main_res:
        line["cpu_baseline"] = main_res["cpu_baseline"]
    if _STREAM is not None:
        line["stream_calibration"] = _STREAM
    secondary = {}
    cpu_secondary = {c for c in args.cpu_secondary.split(",") if c} if not args.no_cpu else set()
    for name in [s for s in args.secondary.split(",") if s and s != args.workload]:
        r = run_workload(pa, name, args.steps, args.warmup, name in cpu_secondary, args.cpu_budget, args.variant,
                         not args.no_graph, not args.no_fused)
        secondary[name] = {"tokens_per_s": round(r["tokens_per_s"], 1), "ms_per_step": round(r["ms_per_step"], 6),
                           "achieved_gbps": round(r["achieved_gbps"], 1), "roofline": r["roofline"],
                           "config": r["config"], **{k: r[k] for k in ("unique_bytes", "logical_bytes",
                                                                     "achieved_gbps_logical", "cpu_baseline") if k in r}}
    if secondary:
        line["secondary"] = secondary
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
