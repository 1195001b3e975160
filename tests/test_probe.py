"""libpa_probe.so, the benchmark's measurement probes: on the CPU, the library loads and exports what
include/pa_probe.h declares, and rejects bad arguments before any launch; on the GPU, each probe reads
exactly the bytes it states (the XOR it writes equals torch's XOR of the same words), the MFMA probe
computes what its header states, and the stream figures bench.py derives from the probes are
consistent."""

from __future__ import annotations

import ctypes
import os
import re

import numpy as np
import pytest
import torch

import bench

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "pa_probe.h")


def _declared():
    text = re.sub(r"/\*.*?\*/", "", open(HEADER, encoding="utf-8").read(), flags=re.S)
    return sorted(set(re.findall(r"\b(pa_probe_[a-z_0-9]+)\s*\(", text)))


def test_probe_library_exports_every_declared_function():
    lib = bench.probe_library()
    assert _declared() == ["pa_probe_first_tile", "pa_probe_mfma", "pa_probe_paged_read", "pa_probe_stream_read"]
    for name in _declared():
        assert hasattr(lib, name), name


def test_probe_arguments_rejected_without_a_launch():
    lib = bench.probe_library()
    fake, out = ctypes.c_void_p(0x1000), ctypes.c_void_p(0x2000)
    assert lib.pa_probe_stream_read(fake, 100, 64, 4, out, None) == -1  # not a multiple of 16
    assert lib.pa_probe_stream_read(fake, 1024, 64, 3, out, None) == -1  # no such unroll
    assert lib.pa_probe_stream_read(fake, 1024, 0, 4, out, None) == -1
    assert lib.pa_probe_first_tile(fake, fake, fake, fake, 4, 8, 4, 10, 16, 100, 0, out, None) == -1  # row bytes
    assert lib.pa_probe_first_tile(fake, fake, fake, fake, 4, 8, 4, 10, 64, 512, 0, out, None) == -1  # tile > 16 KiB
    # paged read: a block of 16 rows of 100 bytes is not 1, 2, 4 or 8 KiB; no such unroll; no blocks per wave
    assert lib.pa_probe_paged_read(fake, fake, fake, fake, 4, 8, 4, 10, 16, 100, 16, 2, 0, out, None) == -1
    assert lib.pa_probe_paged_read(fake, fake, fake, fake, 4, 8, 4, 10, 16, 256, 16, 3, 0, out, None) == -1
    assert lib.pa_probe_paged_read(fake, fake, fake, fake, 4, 8, 4, 10, 16, 256, 0, 2, 0, out, None) == -1
    assert lib.pa_probe_paged_read(fake, fake, fake, fake, 4, 8, 4, 10, 64, 256, 16, 2, 0, out, None) == -1  # 16 KiB
    # MFMA rate: no workgroups, no rounds, no such number of FMAs per MFMA, no output
    assert lib.pa_probe_mfma(0, 10, 0, out, None) == -1
    assert lib.pa_probe_mfma(4, 0, 0, out, None) == -1
    assert lib.pa_probe_mfma(4, 10, 3, out, None) == -1
    assert lib.pa_probe_mfma(4, 10, 0, None, None) == -1


def test_stream_terms_model():
    bench._STREAM = {"stream_gbps": 5000.0}
    try:
        t = bench.stream_terms(2500.0, 50_000_000, 15.0, {"floor_us": 5.0, "floor_dependent_us": 7.0})
    finally:
        bench._STREAM = None
    assert t["frac_of_stream"] == 0.5 and t["floor_us"] == 5.0
    assert t["model_us"] == pytest.approx(5.0 + 10.0) and t["over_model"] == pytest.approx(1.0)
    assert "frac_of_paged_read" not in t
    # with the paged-read rate: 50 MB at 4000 GB/s is 12.5 us, plus the 5 us floor
    t = bench.stream_terms(2500.0, 50_000_000, 35.0, {"floor_us": 5.0, "paged_read_gbps": 4000.0})
    assert "frac_of_stream" not in t and t["frac_of_paged_read"] == 0.625
    assert t["paged_model_us"] == pytest.approx(17.5) and t["over_paged_model"] == pytest.approx(2.0)


def _xor(t):
    a = t.view(torch.int32).reshape(-1).cpu().numpy().view(np.uint32)
    return int(np.bitwise_xor.reduce(a))


@pytest.mark.gpu
@pytest.mark.parametrize("unroll,wg", [(1, 7), (4, 64), (8, 300)])
def test_stream_read_reads_every_word(gpu_lib, unroll, wg):
    lib = bench.probe_library()
    n = (1 << 20) + 48  # a tail past the unrolled steps
    src = torch.randint(-2**31, 2**31 - 1, (n // 4,), dtype=torch.int32, device="cuda:0")
    out = torch.zeros(wg, dtype=torch.int32, device="cuda:0")
    print(f"[case] stream read unroll={unroll} wg={wg}", flush=True)
    h = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    assert lib.pa_probe_stream_read(src.data_ptr(), n, wg, unroll, out.data_ptr(), h) == 0
    torch.cuda.synchronize()
    assert _xor(out) == _xor(src)


@pytest.mark.gpu
@pytest.mark.parametrize("dependent", [0, 1])
def test_first_tile_reads_each_workgroups_first_blocks(gpu_lib, dependent):
    from workloads import make_case

    case = make_case("batch64", num_seqs=9)
    lib = bench.probe_library()
    n, hkv, bs, d = case.k_pool.shape
    g = {k: getattr(case, k).to("cuda:0") for k in ("k_pool", "v_pool", "block_tables", "seq_lens")}
    out = torch.zeros(9 * hkv, dtype=torch.int32, device="cuda:0")
    print(f"[case] first tile dependent={dependent}", flush=True)
    h = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    assert lib.pa_probe_first_tile(g["k_pool"].data_ptr(), g["v_pool"].data_ptr(), g["block_tables"].data_ptr(),
                                   g["seq_lens"].data_ptr(), 9, hkv, case.block_tables.shape[1], n, bs, d * 2,
                                   dependent, out.data_ptr(), h) == 0
    torch.cuda.synchronize()
    mb = case.block_tables.shape[1]
    for i in range(9):
        L = int(case.seq_lens[i])
        for h_ in range(hkv):
            want = 0
            for w in range(4):
                j = min(w, mb - 1) if not dependent else min(w, max(0, -(-L // bs) - 1), mb - 1)
                blk = min(int(case.block_tables[i, j]) & 0xFFFFFFFF, n - 1)
                want ^= _xor(case.k_pool[blk, h_]) ^ _xor(case.v_pool[blk, h_]) ^ (L & 0xFFFFFFFF)
            assert (int(out[i * hkv + h_]) & 0xFFFFFFFF) == want, (i, h_)


@pytest.mark.gpu
@pytest.mark.parametrize("bpw,unroll,nt", [(1, 1, 0), (3, 2, 1), (16, 4, 0)])
def test_paged_read_reads_every_block_once(gpu_lib, bpw, unroll, nt):
    """Each workgroup's XOR is the XOR of the K and V rows of exactly its blocks: blocks
    [4 * bpw * grp, 4 * bpw * (grp + 1)) of its sequence, cut at ceil(L / b)."""
    from workloads import make_case

    case = make_case("batch64", num_seqs=7)
    lib = bench.probe_library()
    n, hkv, bs, d = case.k_pool.shape
    mb = case.block_tables.shape[1]
    groups = -(-mb // (4 * bpw))
    g = {k: getattr(case, k).to("cuda:0") for k in ("k_pool", "v_pool", "block_tables", "seq_lens")}
    out = torch.zeros(7 * groups * hkv, dtype=torch.int32, device="cuda:0")
    print(f"[case] paged read bpw={bpw} unroll={unroll} nt={nt}", flush=True)
    h = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    assert lib.pa_probe_paged_read(g["k_pool"].data_ptr(), g["v_pool"].data_ptr(), g["block_tables"].data_ptr(),
                                   g["seq_lens"].data_ptr(), 7, hkv, mb, n, bs, d * 2, bpw, unroll, nt,
                                   out.data_ptr(), h) == 0
    torch.cuda.synchronize()
    got = out.cpu()
    for i in range(7):
        nb = min(-(-int(case.seq_lens[i]) // bs), mb)
        for grp in range(groups):
            for h_ in range(hkv):
                want = 0
                for j in range(4 * bpw * grp, min(nb, 4 * bpw * (grp + 1))):
                    blk = min(int(case.block_tables[i, j]) & 0xFFFFFFFF, n - 1)
                    want ^= _xor(case.k_pool[blk, h_]) ^ _xor(case.v_pool[blk, h_])
                assert (int(got[(i * groups + grp) * hkv + h_]) & 0xFFFFFFFF) == want, (i, grp, h_)


def _mfma_probe_expected(iters: int, nv: int) -> np.ndarray:
    """What every workgroup of pa_probe_mfma writes, thread by thread, in float64: the operands are
    A[r][k] = bf16(0.001 (lane + k % 8)) held by lane r + 16 (k // 8), B[k][c] = bf16(0.002 (lane - k % 8))
    held by lane c + 16 (k // 8); lane (g, c) keeps D[4g + e][c] of D = A B, e < 4, in each of its 8
    accumulators, iters times; its 8 FMA chains start at 0.01 lane + k and take nv steps per round each
    (v <- 0.9999 v + 0.5)."""
    def bf16(x):
        return torch.tensor(x, dtype=torch.float32).to(torch.bfloat16).to(torch.float64).numpy()

    k = np.arange(32)
    A = np.stack([bf16(0.001 * (r + 16 * (k // 8) + k % 8)) for r in range(16)])        # [16, 32]
    B = np.stack([bf16(0.002 * (c + 16 * (k // 8) - k % 8)) for c in range(16)], axis=1)  # [32, 16]
    D = A @ B
    out = np.zeros(256)
    for t in range(256):
        lane = t % 64
        g, c = lane // 16, lane % 16
        acc = 8 * iters * sum(D[4 * g + e, c] for e in range(4))
        steps = nv * iters
        v = sum(5000.0 + (0.01 * lane + kk - 5000.0) * 0.9999 ** steps for kk in range(8))
        out[t] = acc + v
    return out


@pytest.mark.gpu
@pytest.mark.parametrize("nv", [0, 2, 4])
def test_mfma_probe_computes_what_it_states(gpu_lib, nv):
    lib = bench.probe_library()
    wg, iters = 300, 7
    out = torch.full((wg * 256,), float("nan"), dtype=torch.float32, device="cuda:0")
    print(f"[case] mfma probe nv={nv}", flush=True)
    h = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    assert lib.pa_probe_mfma(wg, iters, nv, out.data_ptr(), h) == 0
    torch.cuda.synchronize()
    got = out.cpu().numpy().reshape(wg, 256).astype(np.float64)
    assert np.isfinite(got).all()
    assert (got == got[0]).all()  # every workgroup computes the same
    np.testing.assert_allclose(got[0], _mfma_probe_expected(iters, nv), rtol=1e-5)
