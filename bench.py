#!/usr/bin/env python3
"""Benchmark of the paged-KV decode step on one MI355X.

A step is one pass of the whole hot path over one batch: the KV-append
scatter (pa_write_kv), then decode attention over every sequence
(pa_decode, or pa_decode_partitioned plus its merge pass). Inputs are
synthetic, seeded and resident in HBM before the timed region starts.
R independent replicas of (pools, tables, q, new rows) are rotated step by
step, so the 256 MB Infinity Cache cannot serve the KV of one step from the
previous one; R * (bytes one step touches) >= 1 GB. The K timed steps run as
HIP graph replays (one captured step per replica), so host launch cost is not
timed; that gives `value`. The same K steps are then launched directly with a
pair of HIP events on the launch stream around every decode call, which gives
the dominant kernel's average duration for `roofline`.

Prints one JSON line. `value` is decode tokens per second of the whole step.
`roofline` relates the dominant kernel's algorithmic bytes to its measured
duration and to the 8 TB/s HBM peak. `cpu_baseline` is the float64 oracle on
this host's cores, over a bounded sample of the same workload.
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "paged decode attention: tokens/s and achieved HBM GB/s (% of peak), 1 MI355X"
HBM_PEAK_GBPS = 8000.0
COLD_BYTES = 1 << 30  # replicas rotate over at least this much memory

WORKLOADS = {
    "batch64": dict(partition_tokens=None, desc="64 seqs, L~U[20,500], 32 q / 8 kv heads, head_dim 128, b=16, "
                                               "bf16 (Llama-3-8B-shaped layer)"),
    "long": dict(partition_tokens=512, desc="16 seqs, L log-uniform [4096,32768], 32 q / 8 kv heads, head_dim 128, "
                                            "b=16, bf16, 512-token partitions + merge"),
    "prefix": dict(partition_tokens=512, desc="128 seqs sharing a 2048-token (128-block) prefix + U[64,1024] private "
                                              "suffix, 32 q / 8 kv heads, head_dim 128, b=16, bf16"),
    "spec": dict(partition_tokens=512, desc="256 seqs, L~U[1024,8192], 4 causal query tokens, 64 q / 8 kv heads, "
                                            "head_dim 128, b=16, bf16"),
    "tiny": dict(partition_tokens=None, desc="4 seqs L={1,17,33,64}, 4 q / 2 kv heads, head_dim 64, b=16, fp32"),
}


def kv_bytes_per_position(num_kv_heads: int, head_dim: int, itemsize: int) -> int:
    """K and V bytes one position holds in one layer: 2 * Hkv * D * sizeof(kv)
    (4096 B for 8 kv heads x 128 x bf16; the per-layer figure of [P2] section 1)."""
    return 2 * num_kv_heads * head_dim * itemsize


def algorithmic_bytes(case, *, include_out: bool = True) -> int:
    """Bytes the decode step must move: every visible K/V row once, q once, the output once,
    the used block-table entries and the lengths (4 bytes each)."""
    b, t, hq, d = case.q.shape
    hkv = case.k_pool.shape[1]
    isz = case.k_pool.element_size()
    lens = [int(x) for x in case.seq_lens]
    kv = sum(lens) * kv_bytes_per_position(hkv, d, isz)
    q = b * t * hq * d * case.q.element_size()
    out = b * t * hq * d * 4 if include_out else 0
    tables = 4 * sum(-(-L // case.block_size) for L in lens) + 4 * b
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
    kv = sum(seen.values()) * kv_bytes_per_position(hkv, d, isz)
    return kv + b * t * hq * d * (case.q.element_size() + 4) + 4 * sum(len(r) for r in case.table_rows) + 4 * b


class Replica:
    """One independent copy of a step's device inputs, with ctypes arguments prepacked."""

    def __init__(self, pa, case, src, partition_tokens, variant=0):
        import ctypes

        import torch

        self.t = {k: v.clone() for k, v in src.items()}
        self.out = torch.empty(case.q.shape, dtype=torch.float32, device=src["q"].device)
        self.lib = pa.load_library()
        self.dims = pa.make_dims(self.t["q"], self.t["k_pool"], self.t["block_tables"], out_dtype=torch.float32,
                                 variant=variant)
        kd = case.k_pool.shape
        code = pa.dtype_code(case.k_pool.dtype)
        self.wdims = pa.PaDims(case.q.shape[0], case.q.shape[1], kd[1], kd[1], kd[3], kd[2], kd[0],
                               case.block_tables.shape[1], code, code, code, 0)
        self.scale = ctypes.c_float(case.scale)
        self.pt = partition_tokens
        self.max_len = case.max_seq_len
        self.ws = None
        if partition_tokens:
            n = pa.workspace_bytes(self.t["q"], self.t["k_pool"], self.t["block_tables"], self.max_len,
                                   partition_tokens)
            self.ws = torch.empty(n, dtype=torch.uint8, device=src["q"].device)
        p = {k: v.data_ptr() for k, v in self.t.items()}
        self.write_args = (ctypes.byref(self.wdims), p["k_new"], p["v_new"], p["k_pool"], p["v_pool"],
                           p["block_tables"], p["positions"])
        self.dec_args = (ctypes.byref(self.dims), p["q"], p["k_pool"], p["v_pool"], p["block_tables"],
                         p["seq_lens"], self.scale)

    def write(self, stream):
        st = self.lib.pa_write_kv(*self.write_args, stream)
        if st:
            raise RuntimeError(f"pa_write_kv: {st}")

    def decode(self, stream):
        if self.ws is None:
            st = self.lib.pa_decode(*self.dec_args, self.out.data_ptr(), stream)
        else:
            st = self.lib.pa_decode_partitioned(*self.dec_args, self.out.data_ptr(), self.max_len, self.pt,
                                                self.ws.data_ptr(), self.ws.numel(), stream)
        if st:
            raise RuntimeError(f"decode: {st}")


def measure_gpu(pa, case, partition_tokens, steps, warmup, variant=0):
    """Returns (seconds per step, per-launch decode-kernel ms list, replicas)."""
    import ctypes

    import torch

    dev = torch.device("cuda:0")
    src = {k: getattr(case, k).to(dev) for k in ("q", "k_new", "v_new", "k_pool", "v_pool", "block_tables",
                                                   "seq_lens", "positions")}
    touched = algorithmic_bytes(case)
    n_rep = max(1, min(64, math.ceil(COLD_BYTES / touched)))
    reps = [Replica(pa, case, src, partition_tokens, variant) for _ in range(n_rep)]
    del src
    torch.cuda.synchronize()

    def sh():
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    # untimed warmup, eager
    for s in range(warmup):
        r = reps[s % n_rep]
        r.write(sh())
        r.decode(sh())
    torch.cuda.synchronize()

    # Timed region A: the K steps as HIP graph replays (one graph per chunk of consecutive steps).
    def capture(first_step, count):
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            with torch.cuda.graph(g, stream=side):
                for c in range(count):
                    r = reps[(first_step + c) % n_rep]
                    r.write(sh())
                    r.decode(sh())
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        return g

    chunk = n_rep
    full = capture(0, chunk)
    rem = steps % chunk
    tail = capture(0, rem) if rem else None
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

    # Timed region B: the same K steps launched directly, with HIP events on the launch stream
    # bracketing every decode call (for a partitioned decode: both of its kernels).
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    handle = ctypes.c_void_p(stream.cuda_stream)
    for s in range(steps):
        r = reps[s % n_rep]
        r.write(handle)
        evs[s][0].record(stream)
        r.decode(handle)
        evs[s][1].record(stream)
    torch.cuda.synchronize()
    kernel_ms = [a.elapsed_time(b) for a, b in evs]
    return (t1 - t0) / steps, kernel_ms, reps


def cpu_baseline(case, budget_s: float):
    """The float64 oracle (KV write + decode) on this host, on a bounded sample of the
    workload's sequences (grown until the sample takes about ``budget_s``)."""
    import numpy as np
    import torch
    from threadpoolctl import threadpool_limits

    import oracle

    def npbits(t):
        t = t.detach().cpu().contiguous()
        return t.view(torch.int16).numpy().view(np.uint16) if t.element_size() == 2 else \
            t.view(torch.int32).numpy().view(np.uint32)

    b = case.q.shape[0]
    with threadpool_limits(limits=1):
        kp_all, vp_all = npbits(case.k_pool), npbits(case.v_pool)
        n = 1
        while True:
            sl = slice(0, n)
            t0 = time.perf_counter()
            kp, vp = oracle.write_kv(kp_all, vp_all, npbits(case.k_new[sl]), npbits(case.v_new[sl]),
                                     case.block_tables[sl].numpy(), case.positions[sl].numpy(), case.block_size)
            as_f = (lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).float().numpy()) \
                if kp.dtype == np.uint16 else (lambda a: a.view(np.float32))
            oracle.decode(case.q[sl].float().numpy(), as_f(kp), as_f(vp), case.block_tables[sl].numpy(),
                          case.seq_lens[sl].numpy(), case.scale, case.block_size)
            dt = time.perf_counter() - t0
            if dt >= budget_s or n >= b:
                break
            n = min(b, max(n + 1, int(n * min(8.0, 1.5 * budget_s / max(dt, 1e-3)))))
    tokens = n * case.q.shape[1]
    return {"value": tokens / dt, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"KV write + float64 decode of the first {n} of {b} sequences "
                      f"({int(case.seq_lens[:n].sum())} positions), one thread, {dt:.1f} s"}


def run_workload(pa, name, steps, warmup, with_cpu, cpu_budget, variant=0):
    import torch

    from workloads import make_case

    spec = WORKLOADS[name]
    case = make_case(name, pool_device="cuda:0")
    sec_per_step, kernel_ms, reps = measure_gpu(pa, case, spec["partition_tokens"], steps, warmup, variant)
    b, t = case.q.shape[0], case.q.shape[1]
    algo = algorithmic_bytes(case, include_out=spec["partition_tokens"] is None)
    dur_ms = sum(kernel_ms) / max(1, len(kernel_ms))
    achieved = algo / (dur_ms * 1e-3) / 1e9
    rows = case.q.shape[2] // case.k_pool.shape[1] * t
    mfma_ok = case.k_pool.dtype == torch.bfloat16 and case.q.shape[3] == 128 and rows <= 32
    kernel = "decode_mfma_kernel" if (variant == 2 or (variant == 0 and mfma_ok)) else "decode_valu_kernel"
    res = {
        "tokens_per_s": b * t / sec_per_step,
        "ms_per_step": sec_per_step * 1e3,
        "achieved_gbps": algo / sec_per_step / 1e9,
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": None,
                     "kernel": kernel + (" (partial pass; merge pass excluded)" if spec["partition_tokens"] else ""),
                     "bytes_per_launch": algo, "avg_launch_us": round(dur_ms * 1e3, 3),
                     "launches_timed": len(kernel_ms)},
        "config": {"workload": f"{name}: {spec['desc']}", "num_seqs": b, "q_tokens": t,
                   "kv_positions": case.kv_tokens(), "max_seq_len": case.max_seq_len,
                   "partition_tokens": spec["partition_tokens"], "replicas": len(reps)},
        "dtype": "bf16" if case.k_pool.dtype == torch.bfloat16 else "f32",
    }
    if name == "prefix":
        res["unique_bytes"] = unique_bytes(case)
    if with_cpu:
        res["cpu_baseline"] = cpu_baseline(case, cpu_budget)
    del reps
    torch.cuda.empty_cache()
    return res


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="batch64", choices=sorted(WORKLOADS))
    ap.add_argument("--secondary", default="long",
                    help="comma-separated workloads also measured and reported under 'secondary' ('' for none)")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle work for cpu_baseline")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--variant", type=int, default=0, help="0 auto, 1 vector-ALU kernel, 2 MFMA kernel")
    args = ap.parse_args(argv)
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (the decode step needs no "
              "collectives; see DESIGN.md for how it would shard).", file=sys.stderr)
        return 2

    import torch

    import paged_kv_cache_69_amd as pa

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    pa.load_library()
    main_res = run_workload(pa, args.workload, args.steps, args.warmup, not args.no_cpu, args.cpu_budget,
                            args.variant)
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
        "data": "synthetic",
        "config": main_res["config"],
        "achieved_gbps": round(main_res["achieved_gbps"], 1),
        "hbm_frac": round(main_res["achieved_gbps"] / HBM_PEAK_GBPS, 4),
        "roofline": main_res["roofline"],
    }
    if "cpu_baseline" in main_res:
        line["cpu_baseline"] = main_res["cpu_baseline"]
    secondary = {}
    for name in [s for s in args.secondary.split(",") if s and s != args.workload]:
        r = run_workload(pa, name, args.steps, args.warmup, False, 0, args.variant)
        secondary[name] = {"tokens_per_s": round(r["tokens_per_s"], 1), "ms_per_step": round(r["ms_per_step"], 6),
                           "achieved_gbps": round(r["achieved_gbps"], 1), "roofline": r["roofline"],
                           "config": r["config"], **({"unique_bytes": r["unique_bytes"]} if "unique_bytes" in r else {})}
    if secondary:
        line["secondary"] = secondary
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
