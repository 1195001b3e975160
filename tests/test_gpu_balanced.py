"""The balanced split schedule (pa_dims.split_schedule = PA_SPLIT_BALANCED) against the float64 oracle, on
the GPU.

The tiles of every sequence of one kv head form one list cut into equal ranges, one per pair of waves,
so ranges cross sequences; the two waves of a pair share their range from its two ends, each leaves
one partial per sequence it touched (slot 2 (range - first range of the sequence) + side), and marks
the slots of the range's other sequences empty. The workspace is filled beforehand with
partials that look valid (m = 0, l = 1, acc = 1e6), so a slot the kernel failed to write would show in
the output. Every case meets the oracle at the bar of its pool type; the fused append under this
schedule writes the pools bit for bit like the separate append, and its output meets the oracle too
(the two waves of a pair meet where their timing puts them, so the pieces, and the rounding of their
probabilities, may differ from call to call).
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from tests.helpers import assert_attention_close, bits, oracle_after_write, poison_case, to_f32_view
from workloads import build_case, fp8_pools, int8_pools

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
BAL = 3


def _poisoned_workspace(pa, q, k_pool, tables, max_len, pt):
    n = pa.workspace_bytes(q, k_pool, tables, max_len, pt, split_schedule=BAL)
    ws = torch.empty(n, dtype=torch.uint8, device=DEV)
    f = ws.view(torch.float32)
    f.fill_(1.0e6)
    rows = q.shape[0] * q.shape[1] * q.shape[2]
    parts = -(-max_len // pt)
    ml = f[: rows * (2 * parts + 2) * 2].view(-1, 2)
    ml[:, 0] = 0.0
    ml[:, 1] = 1.0
    return ws


def _lengths(t, b):
    # short sequences (a range holds many), tails at tile and block edges, long ones cut by many ranges
    return sorted({max(t, x) for x in (1, 2, 15, 16, 17, b + 1, 40, 100, 257, 700, 1300, 2500)})


def _oracle_bf16(case, kp, vp):
    back = lambda x: torch.from_numpy(x.view(np.int16)).view(case.k_pool.dtype).reshape(case.k_pool.shape)  # noqa
    return oracle.decode(to_f32_view(case.q), to_f32_view(back(kp)), to_f32_view(back(vp)), case.block_tables.numpy(),
                         case.seq_lens.numpy(), case.scale, case.block_size)


@pytest.mark.parametrize("b", [16, 32])
@pytest.mark.parametrize("hq,hkv,t", [(32, 8, 1), (8, 2, 4), (12, 4, 3), (4, 1, 1), (16, 1, 1)])
@pytest.mark.parametrize("pt", [32, 64, 512])
def test_balanced_bf16(gpu_lib, b, hq, hkv, t, pt):
    if pt % b:
        pytest.skip("partition not a multiple of the block")
    case = build_case(lengths=_lengths(t, b), num_q_heads=hq, num_kv_heads=hkv, head_dim=128, block_size=b,
                      q_tokens=t, dtype=torch.bfloat16, seed=11000 + b + hq + t + pt, pool_slack=0.2)
    poison_case(case)
    kp, vp = oracle_after_write(case)
    ref = _oracle_bf16(case, kp, vp)
    g = {k: getattr(case, k).to(DEV, copy=True) for k in ("q", "k_new", "v_new", "k_pool", "v_pool", "block_tables",
                                                         "seq_lens", "positions")}
    gpu_lib.write_kv(g["k_new"], g["v_new"], g["k_pool"], g["v_pool"], g["block_tables"], g["positions"])
    print(f"[case] balanced bf16 b={b} hq={hq} hkv={hkv} T={t} pt={pt}", flush=True)
    assert gpu_lib.split_schedule(g["q"], g["k_pool"], g["block_tables"], case.max_seq_len, pt, force=BAL) == BAL
    ws = _poisoned_workspace(gpu_lib, g["q"], g["k_pool"], g["block_tables"], case.max_seq_len, pt)
    out = gpu_lib.decode_partitioned(g["q"], g["k_pool"], g["v_pool"], g["block_tables"], g["seq_lens"], case.scale,
                                     case.max_seq_len, pt, workspace=ws, split_schedule=BAL)
    torch.cuda.synchronize()
    assert_attention_close(out.cpu(), ref, kv_dtype=torch.bfloat16, out_dtype=torch.float32, what=f"balanced pt={pt}")
    # the fused append under the same schedule: the same pools and the same bits
    f = {k: getattr(case, k).to(DEV, copy=True) for k in g}
    fused = gpu_lib.write_kv_decode(f["q"], f["k_new"], f["v_new"], f["k_pool"], f["v_pool"], f["block_tables"],
                                    f["seq_lens"], case.scale, max_seq_len=case.max_seq_len, partition_tokens=pt,
                                    split_schedule=BAL)
    torch.cuda.synchronize()
    assert np.array_equal(bits(f["k_pool"]), kp) and np.array_equal(bits(f["v_pool"]), vp)
    # the pair's meeting point follows the waves' timing, so the two calls may cut the pieces (and round
    # their probabilities, relative to each piece's own reference) differently: each meets the oracle
    assert_attention_close(fused.cpu(), ref, kv_dtype=torch.bfloat16, out_dtype=torch.float32, what=f"fused pt={pt}")


@pytest.mark.parametrize("fmt", ["int8", "fp8"])
@pytest.mark.parametrize("b", [16, 32])
@pytest.mark.parametrize("hq,t", [(32, 1), (16, 4)])
def test_balanced_8bit(gpu_lib, fmt, b, hq, t):
    case = build_case(lengths=_lengths(t, b), num_q_heads=hq, num_kv_heads=8, head_dim=128, block_size=b,
                      q_tokens=t, dtype=torch.bfloat16, seed=12000 + b + hq + t, pool_slack=0.2)
    kc, vc, sc = (int8_pools if fmt == "int8" else fp8_pools)(case, seed=b + hq + t)

    def np_codes(x):
        return x.cpu().view(torch.uint8).numpy().view(np.int8 if fmt == "int8" else np.uint8)

    s = sc.cpu().numpy()
    ref = (oracle.decode_int8 if fmt == "int8" else oracle.decode_fp8)(
        case.q.float().numpy(), np_codes(kc), np.ascontiguousarray(s[..., 0]), np_codes(vc),
        np.ascontiguousarray(s[..., 1]), case.block_tables.numpy(), case.seq_lens.numpy(), case.scale, b)
    q, tab, lens = (getattr(case, k).to(DEV) for k in ("q", "block_tables", "seq_lens"))
    kc, vc, sc = (x.to(DEV) for x in (kc, vc, sc))
    dec = gpu_lib.decode_partitioned_int8 if fmt == "int8" else gpu_lib.decode_partitioned_fp8
    for pt in (32, 512):
        print(f"[case] balanced {fmt} b={b} hq={hq} T={t} pt={pt}", flush=True)
        ws = _poisoned_workspace(gpu_lib, q, kc.view(torch.int8), tab, case.max_seq_len, pt)
        out = dec(q, kc, vc, sc, tab, lens, case.scale, case.max_seq_len, pt, workspace=ws, split_schedule=BAL)
        torch.cuda.synchronize()
        assert_attention_close(out.cpu(), ref, kv_dtype=torch.int8, out_dtype=torch.float32, what=f"{fmt} pt={pt}")


def test_balanced_restarts(gpu_lib):
    """Scores climbing about 130 base-2 units per 512 positions: pieces restart inside partitions, in the
    middle of a wave's range as well as at its start."""
    lengths = [40, 700, 1100, 1500, 2100]
    case = build_case(lengths=lengths, num_q_heads=32, num_kv_heads=8, head_dim=128, block_size=16,
                      dtype=torch.bfloat16, seed=13000, pool_slack=0.1)
    top = max(lengths)
    for i, L in enumerate(lengths):
        for pos in range(L - 1):
            phys = int(case.block_tables[i, pos // 16])
            case.k_pool[phys, :, pos % 16] = 0.0
            case.k_pool[phys, :, pos % 16, 0] = float(torch.tensor(pos / top * 720.0).to(torch.bfloat16))
        case.k_new[i] = 0.0
        case.k_new[i, :, :, 0] = float(torch.tensor((L - 1) / top * 720.0).to(torch.bfloat16))
    case.q[..., 0] = (6.0 + 0.1 * case.q[..., 0].float()).to(torch.bfloat16)
    kp, vp = oracle_after_write(case)
    ref = _oracle_bf16(case, kp, vp)
    g = {k: getattr(case, k).to(DEV, copy=True) for k in ("q", "k_new", "v_new", "k_pool", "v_pool", "block_tables",
                                                         "seq_lens", "positions")}
    gpu_lib.write_kv(g["k_new"], g["v_new"], g["k_pool"], g["v_pool"], g["block_tables"], g["positions"])
    print("[case] balanced restarts", flush=True)
    for pt in (64, 512):
        out = gpu_lib.decode_partitioned(g["q"], g["k_pool"], g["v_pool"], g["block_tables"], g["seq_lens"],
                                         case.scale, case.max_seq_len, pt, split_schedule=BAL)
        torch.cuda.synchronize()
        assert_attention_close(out.cpu(), ref, kv_dtype=torch.bfloat16, out_dtype=torch.float32, what=f"pt={pt}")


def test_balanced_fewer_tiles_than_waves(gpu_lib):
    """Batches whose whole tile list holds fewer partitions than the launch has waves: the ranges shrink to
    at least one partition each and the surplus waves leave; one sequence of one tile included."""
    for lengths in ([1], [3, 5], [17, 40, 33]):
        case = build_case(lengths=lengths, num_q_heads=8, num_kv_heads=2, head_dim=128, block_size=16,
                          dtype=torch.bfloat16, seed=14000 + len(lengths))
        poison_case(case)
        kp, vp = oracle_after_write(case)
        g = {k: getattr(case, k).to(DEV, copy=True) for k in ("q", "k_new", "v_new", "k_pool", "v_pool",
                                                             "block_tables", "seq_lens", "positions")}
        gpu_lib.write_kv(g["k_new"], g["v_new"], g["k_pool"], g["v_pool"], g["block_tables"], g["positions"])
        print(f"[case] balanced small {lengths}", flush=True)
        ws = _poisoned_workspace(gpu_lib, g["q"], g["k_pool"], g["block_tables"], case.max_seq_len, 32)
        out = gpu_lib.decode_partitioned(g["q"], g["k_pool"], g["v_pool"], g["block_tables"], g["seq_lens"],
                                         case.scale, case.max_seq_len, 32, workspace=ws, split_schedule=BAL)
        torch.cuda.synchronize()
        assert_attention_close(out.cpu(), _oracle_bf16(case, kp, vp), kv_dtype=torch.bfloat16,
                               out_dtype=torch.float32, what=f"{lengths}")


@pytest.mark.parametrize("nseq", [1, 2, 32, 33, 48])
def test_balanced_scan_paths(gpu_lib, nseq):
    """Both ways the kernel finds its ranges: up to 63 sequences whose q rows fit four 16-byte pieces per
    thread (32 sequences of 4 rows here) scan the lengths in registers and fix each wave's first takes; 33
    and more scan in LDS, up to 48 (their q rows fill the 48 KiB the workgroup stages them in). Random lengths (a one-position sequence among them) at partitions of 64 tokens, the
    fused append and the plain decode, poisoned workspaces, against the oracle."""
    rng = np.random.default_rng(1400 + nseq)
    lengths = [int(x) for x in rng.integers(1, 700, size=nseq)]
    if nseq > 2:
        lengths[1] = 1  # a one-position sequence among long ones
    case = build_case(lengths=lengths, num_q_heads=32, num_kv_heads=8, head_dim=128, block_size=16, q_tokens=1,
                      dtype=torch.bfloat16, seed=1400 + nseq, pool_slack=0.2)
    poison_case(case)
    kp, vp = oracle_after_write(case)
    ref = _oracle_bf16(case, kp, vp)
    pt = 64
    print(f"[case] balanced scan paths B={nseq}", flush=True)
    g = {k: getattr(case, k).to(DEV, copy=True) for k in ("q", "k_new", "v_new", "k_pool", "v_pool", "block_tables",
                                                         "seq_lens", "positions")}
    assert gpu_lib.split_schedule(g["q"], g["k_pool"], g["block_tables"], case.max_seq_len, pt, force=BAL) == BAL
    ws = _poisoned_workspace(gpu_lib, g["q"], g["k_pool"], g["block_tables"], case.max_seq_len, pt)
    fused = gpu_lib.write_kv_decode(g["q"], g["k_new"], g["v_new"], g["k_pool"], g["v_pool"], g["block_tables"],
                                    g["seq_lens"], case.scale, max_seq_len=case.max_seq_len, partition_tokens=pt,
                                    workspace=ws, split_schedule=BAL)
    torch.cuda.synchronize()
    assert np.array_equal(bits(g["k_pool"]), kp) and np.array_equal(bits(g["v_pool"]), vp)
    assert_attention_close(fused.cpu(), ref, kv_dtype=torch.bfloat16, out_dtype=torch.float32, what="fused")
    ws = _poisoned_workspace(gpu_lib, g["q"], g["k_pool"], g["block_tables"], case.max_seq_len, pt)
    out = gpu_lib.decode_partitioned(g["q"], g["k_pool"], g["v_pool"], g["block_tables"], g["seq_lens"], case.scale,
                                     case.max_seq_len, pt, workspace=ws, split_schedule=BAL)
    torch.cuda.synchronize()
    assert_attention_close(out.cpu(), ref, kv_dtype=torch.bfloat16, out_dtype=torch.float32, what="decode")
