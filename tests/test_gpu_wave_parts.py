"""Split decode with two consecutive partitions per wave, on the GPU.

When B * Hkv * ceil(max_seq_len / partition_tokens) exceeds the waves the GPU holds at once, each wave of
the matrix-core split kernel walks two consecutive partitions (pa_decode_partitioned_schedule = 2). It
still writes one partial per partition, each with that partition's own reference maximum, so the merged
result must be the same bits as with one partition per wave. pa_dims.split_schedule forces either choice, so
the same call runs both ways. Both runs also meet the float64 oracle; nothing expected comes from the GPU.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from tests.helpers import assert_attention_close, bits, oracle_after_write, poison_case, to_f32_view
from workloads import build_case

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _gpu(case):
    return {k: getattr(case, k).to(DEV, copy=True) for k in ("q", "k_new", "v_new", "k_pool", "v_pool", "block_tables",
                                                    "seq_lens", "positions")}


def _both_ways(pa, g, case, pt, call):
    """call(kp) with one, then two partitions per wave (forced through pa_dims.split_schedule), at the case's
    own max_seq_len."""
    outs = []
    for kp in (1, 2):
        assert pa.split_schedule(g["q"], g["k_pool"], g["block_tables"], case.max_seq_len, pt, force=kp) == kp
        outs.append(call(kp))
    torch.cuda.synchronize()
    return outs


def _oracle_decode(case, kp_bits, vp_bits):
    kp = torch.from_numpy(kp_bits.view(np.int16)).view(case.k_pool.dtype).reshape(case.k_pool.shape)
    vp = torch.from_numpy(vp_bits.view(np.int16)).view(case.v_pool.dtype).reshape(case.v_pool.shape)
    return oracle.decode(to_f32_view(case.q), to_f32_view(kp), to_f32_view(vp), case.block_tables.numpy(),
                         case.seq_lens.numpy(), case.scale, case.block_size)


def _lengths(t):
    # one and several partitions, partition and tile boundaries, odd and even partition counts per sequence
    return sorted({max(t, x) for x in (1, 15, 16, 17, 31, 32, 33, 95, 96, 97, 200, 255, 256, 257, 520)})


@pytest.mark.parametrize("b", [4, 8, 16, 32])
@pytest.mark.parametrize("hq,hkv,t", [(32, 8, 1), (8, 2, 4), (12, 4, 3), (4, 1, 1)])
def test_two_partitions_per_wave_bitwise(gpu_lib, b, hq, hkv, t):
    """bf16 pools, separate append and fused append + decode: two partitions per wave give the bits of one
    per wave, and meet the oracle."""
    case = build_case(lengths=_lengths(t), num_q_heads=hq, num_kv_heads=hkv, head_dim=128, block_size=b,
                      q_tokens=t, dtype=torch.bfloat16, seed=7000 + b * 10 + hq + t, pool_slack=0.2)
    poison_case(case)
    kp, vp = oracle_after_write(case)
    ref = _oracle_decode(case, kp, vp)
    for pt in (32, 48 if 48 % b == 0 else 64, 512):
        print(f"[case] wave parts b={b} hq={hq} hkv={hkv} T={t} pt={pt}", flush=True)
        g = _gpu(case)
        gpu_lib.write_kv(g["k_new"], g["v_new"], g["k_pool"], g["v_pool"], g["block_tables"], g["positions"])
        outs = _both_ways(gpu_lib, g, case, pt, lambda kp: gpu_lib.decode_partitioned(
            g["q"], g["k_pool"], g["v_pool"], g["block_tables"], g["seq_lens"], case.scale, case.max_seq_len, pt,
            split_schedule=kp))
        fs = []

        def fused_call(kp):
            f = _gpu(case)
            fs.append(f)
            return gpu_lib.write_kv_decode(f["q"], f["k_new"], f["v_new"], f["k_pool"], f["v_pool"],
                                           f["block_tables"], f["seq_lens"], case.scale,
                                           max_seq_len=case.max_seq_len, partition_tokens=pt, split_schedule=kp)

        fused = _both_ways(gpu_lib, g, case, pt, fused_call)
        for f in fs:
            assert np.array_equal(bits(f["k_pool"]), kp) and np.array_equal(bits(f["v_pool"]), vp)
        assert torch.equal(outs[0], outs[1]), f"two partitions per wave changed the result (pt={pt})"
        assert torch.equal(fused[0], fused[1]), f"fused: two partitions per wave changed the result (pt={pt})"
        assert torch.equal(outs[0], fused[0])
        assert_attention_close(outs[1].cpu(), ref, kv_dtype=torch.bfloat16, out_dtype=torch.float32,
                               what=f"two per wave, pt={pt}")


def test_two_partitions_per_wave_reference_restarts(gpu_lib):
    """Scores that grow by about 130 base-2 units per 512-position partition make tiles outrun their
    partition's reference max (set by its first tile) several times inside each partition, the second
    partition of a wave included; each restart runs that partition again from its first tile. The bits
    equal those of one partition per wave, and the result meets the oracle. K rows and q point along
    head_dim 0 only, so every score is one exact bf16 product."""
    lengths = [40, 700, 1100, 1500, 2100]
    case = build_case(lengths=lengths, num_q_heads=32, num_kv_heads=8, head_dim=128, block_size=16,
                      dtype=torch.bfloat16, seed=7200, pool_slack=0.1)
    top = max(lengths)

    def ramp(pos):
        return float(torch.tensor(pos / top * 720.0).to(torch.bfloat16))

    for i, L in enumerate(lengths):
        for pos in range(L - 1):
            phys = int(case.block_tables[i, pos // 16])
            case.k_pool[phys, :, pos % 16] = 0.0
            case.k_pool[phys, :, pos % 16, 0] = ramp(pos)
        case.k_new[i] = 0.0
        case.k_new[i, :, :, 0] = ramp(L - 1)
    case.q[..., 0] = (6.0 + 0.1 * case.q[..., 0].float()).to(torch.bfloat16)
    kp, vp = oracle_after_write(case)
    ref = _oracle_decode(case, kp, vp)
    pt = 512
    g = _gpu(case)
    gpu_lib.write_kv(g["k_new"], g["v_new"], g["k_pool"], g["v_pool"], g["block_tables"], g["positions"])
    print("[case] wave parts reference restarts", flush=True)
    outs = _both_ways(gpu_lib, g, case, pt, lambda kp: gpu_lib.decode_partitioned(
        g["q"], g["k_pool"], g["v_pool"], g["block_tables"], g["seq_lens"], case.scale, case.max_seq_len, pt,
        split_schedule=kp))
    single = gpu_lib.decode(g["q"], g["k_pool"], g["v_pool"], g["block_tables"], g["seq_lens"], case.scale)
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1])
    for what, out in (("split", outs[1]), ("single pass", single)):
        assert_attention_close(out.cpu(), ref, kv_dtype=torch.bfloat16, out_dtype=torch.float32, what=what)


@pytest.mark.parametrize("t", [1, 4])
def test_fused_single_pass_short_wave_restarts(gpu_lib, t):
    """Fused append + single pass on sequences of 2 to 16 tiles, so every wave has at most four tiles and
    computes its first tile before it asks for its second. K points along head_dim 0 with a value that
    climbs about 2.6 per position (about 2 base-2 units of score per position), so a wave's later tiles
    outrun the reference its first tile set and it runs again from its first tile. The fused call gives the
    bits of the separate append + single pass, and both meet the oracle."""
    lengths = [max(t, x) for x in (20, 100, 180, 200, 250, 256)]
    case = build_case(lengths=lengths, num_q_heads=32, num_kv_heads=8, head_dim=128, block_size=16, q_tokens=t,
                      dtype=torch.bfloat16, seed=7300 + t, pool_slack=0.1)

    def ramp(pos):
        return float(torch.tensor(2.6 * pos).to(torch.bfloat16))

    for i, L in enumerate(lengths):
        for pos in range(L - t):
            phys = int(case.block_tables[i, pos // 16])
            case.k_pool[phys, :, pos % 16] = 0.0
            case.k_pool[phys, :, pos % 16, 0] = ramp(pos)
        for j in range(t):
            case.k_new[i, j] = 0.0
            case.k_new[i, j, :, 0] = ramp(L - t + j)
    case.q[..., 0] = (6.0 + 0.1 * case.q[..., 0].float()).to(torch.bfloat16)
    kp, vp = oracle_after_write(case)
    ref = _oracle_decode(case, kp, vp)
    f, s = _gpu(case), _gpu(case)
    print(f"[case] fused single pass short-wave restarts T={t}", flush=True)
    fused = gpu_lib.write_kv_decode(f["q"], f["k_new"], f["v_new"], f["k_pool"], f["v_pool"], f["block_tables"],
                                    f["seq_lens"], case.scale)
    gpu_lib.write_kv(s["k_new"], s["v_new"], s["k_pool"], s["v_pool"], s["block_tables"], s["positions"])
    separate = gpu_lib.decode(s["q"], s["k_pool"], s["v_pool"], s["block_tables"], s["seq_lens"], case.scale)
    torch.cuda.synchronize()
    assert torch.equal(fused, separate)
    for g in (f, s):  # bit patterns: the pools' unused slots hold NaN
        assert np.array_equal(bits(g["k_pool"]), kp) and np.array_equal(bits(g["v_pool"]), vp)
    for what, out in (("fused", fused), ("separate", separate)):
        assert_attention_close(out.cpu(), ref, kv_dtype=torch.bfloat16, out_dtype=torch.float32, what=what)
