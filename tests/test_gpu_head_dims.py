"""Decode parity for every (dtype, head_dim) pair of the boundary, on the GPU.

[P1] "25. Paged attention and prefix caching", section "Attention that reads through the table", launches
its decode for any head_dim with the output in q's dtype; the library serves q/KV in bf16 or fp32 with
head_dim 64 or 128, b in {4, 8, 16, 32}, single pass and split, fp32 or bf16 out. bf16 with head_dim 128
runs on the matrix-core kernel by default; the other three pairs run on the vector-ALU kernel (a K/V row
of 8, 16 or 32 sixteen-byte chunks). Each case writes the step's new rows first (checked bit for bit),
poisons every unwritten slot with NaN, and compares the output with the float64 oracle on the same
values: 1e-5 relative per row for fp32 inputs, 2e-3 absolute for bf16.
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
PAIRS = [(torch.bfloat16, 64), (torch.bfloat16, 128), (torch.float32, 64), (torch.float32, 128)]


def _gpu(case):
    return {k: getattr(case, k).to(DEV, copy=True) for k in ("q", "k_new", "v_new", "k_pool", "v_pool", "block_tables",
                                                    "seq_lens", "positions")}


def _oracle(case, kp_bits, vp_bits):
    def back(x):
        return torch.from_numpy(x.view(np.int16 if x.dtype == np.uint16 else np.int32)).view(
            case.k_pool.dtype).reshape(case.k_pool.shape)

    return oracle.decode(to_f32_view(case.q), to_f32_view(back(kp_bits)), to_f32_view(back(vp_bits)),
                         case.block_tables.numpy(), case.seq_lens.numpy(), case.scale, case.block_size)


def _step(pa, case, *, partition_tokens=None, out_dtype=torch.float32, variant=0):
    g = _gpu(case)
    pa.write_kv(g["k_new"], g["v_new"], g["k_pool"], g["v_pool"], g["block_tables"], g["positions"])
    if partition_tokens:
        out = pa.decode_partitioned(g["q"], g["k_pool"], g["v_pool"], g["block_tables"], g["seq_lens"], case.scale,
                                    case.max_seq_len, partition_tokens, out_dtype=out_dtype, variant=variant)
    else:
        out = pa.decode(g["q"], g["k_pool"], g["v_pool"], g["block_tables"], g["seq_lens"], case.scale,
                        out_dtype=out_dtype, variant=variant)
    torch.cuda.synchronize()
    return g, out


@pytest.mark.parametrize("dtype,d", PAIRS)
@pytest.mark.parametrize("b", [4, 8, 16, 32])
@pytest.mark.parametrize("hq,hkv,t", [(8, 2, 1), (32, 8, 1), (12, 4, 3), (4, 1, 1), (16, 2, 2)])
def test_decode_every_dtype_and_head_dim(gpu_lib, dtype, d, b, hq, hkv, t):
    """GQA 1-8, 1-3 causal query tokens (up to 16 rows per kv head), lengths at tile and block edges and
    past several 16-position tiles; single pass, and split into 32- and 48/64-position partitions."""
    lengths = sorted({max(t, x) for x in (1, b - 1, b, b + 1, 15, 16, 17, 47, 100, 257)})
    case = build_case(lengths=lengths, num_q_heads=hq, num_kv_heads=hkv, head_dim=d, block_size=b, q_tokens=t,
                      dtype=dtype, seed=9000 + d + b * 3 + hq + t, pool_slack=0.2)
    poison_case(case)
    kp, vp = oracle_after_write(case)
    ref = _oracle(case, kp, vp)
    for pt in (None, 32, 48 if 48 % b == 0 else 64):
        print(f"[case] {dtype} D={d} b={b} hq={hq} hkv={hkv} T={t} split={pt}", flush=True)
        g, out = _step(gpu_lib, case, partition_tokens=pt)
        assert np.array_equal(bits(g["k_pool"]), kp) and np.array_equal(bits(g["v_pool"]), vp)
        assert_attention_close(out.cpu(), ref, kv_dtype=dtype, out_dtype=torch.float32, what=f"{dtype} D={d} pt={pt}")


@pytest.mark.parametrize("dtype,d", PAIRS)
def test_bf16_output_every_pair(gpu_lib, dtype, d):
    case = build_case(lengths=[3, 40, 129, 300], num_q_heads=16, num_kv_heads=4, head_dim=d, block_size=16,
                      dtype=dtype, seed=9100 + d)
    poison_case(case)
    kp, vp = oracle_after_write(case)
    ref = _oracle(case, kp, vp)
    print(f"[case] bf16 out {dtype} D={d}", flush=True)
    for pt in (None, 64):
        _, out = _step(gpu_lib, case, partition_tokens=pt, out_dtype=torch.bfloat16)
        assert_attention_close(out.cpu(), ref, kv_dtype=dtype, out_dtype=torch.bfloat16, what=f"bf16 out pt={pt}")


@pytest.mark.parametrize("dtype,d", PAIRS)
def test_single_position_gives_v0_bitwise_every_pair(gpu_lib, dtype, d):
    """L = 1: the one softmax weight is exactly 1, so the fp32 output is v_0 bit for bit."""
    case = build_case(lengths=[1, 1, 1], num_q_heads=8, num_kv_heads=2, head_dim=d, block_size=16, dtype=dtype,
                      seed=9200 + d)
    print(f"[case] v0 {dtype} D={d}", flush=True)
    for variant in (0, 1):
        _, out = _step(gpu_lib, case, variant=variant)
        want = case.v_new[:, 0].to(torch.float32).repeat_interleave(4, dim=1)
        assert torch.equal(out[:, 0].cpu(), want)


@pytest.mark.parametrize("dtype,d", [(torch.bfloat16, 64), (torch.float32, 128)])
def test_new_pairs_reference_restarts(gpu_lib, dtype, d):
    """Scores that climb by 0.13-0.18 base-2 units per position (up to about 125 units over a sequence)
    make later tiles outrun the vector-ALU kernel's lazy reference (2^8 slack) many times; each time
    it rescales. K rows and q point along head_dim 0 only, so every score is one exact product."""
    lengths = [40, 300, 700]
    case = build_case(lengths=lengths, num_q_heads=8, num_kv_heads=2, head_dim=d, block_size=16, dtype=dtype,
                      seed=9300 + d, pool_slack=0.1)
    for i, L in enumerate(lengths):
        for pos in range(L - 1):
            phys = int(case.block_tables[i, pos // 16])
            case.k_pool[phys, :, pos % 16] = 0.0
            case.k_pool[phys, :, pos % 16, 0] = float(torch.tensor(pos * 0.25).to(dtype))
        case.k_new[i] = 0.0
        case.k_new[i, :, :, 0] = float(torch.tensor((L - 1) * 0.25).to(dtype))
    case.q[..., 0] = (4.0 + 0.1 * case.q[..., 0].float()).to(dtype)
    kp, vp = oracle_after_write(case)
    ref = _oracle(case, kp, vp)
    print(f"[case] restarts {dtype} D={d}", flush=True)
    for pt in (None, 128):
        _, out = _step(gpu_lib, case, partition_tokens=pt)
        assert_attention_close(out.cpu(), ref, kv_dtype=dtype, out_dtype=torch.float32, what=f"restart pt={pt}")
