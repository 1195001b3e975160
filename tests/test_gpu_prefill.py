"""Parity of the paged prefill path (pa_write_kv_varlen, pa_prefill) against the prefill oracle, on
the GPU, through the C ABI.

The chunk scatter must match the oracle bit for bit. Attention must be within the bf16 bar (2e-3
absolute; plus half a bf16 ulp for bf16 output) of the oracle's float64 attention on the same
bf16 values. Inputs come from the seeded generators in workloads/; nothing expected comes from the
GPU.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from tests.helpers import assert_attention_close, bits, from_bits, to_f32_view
from workloads import build_prefill_case, make_prefill_case

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _poison_tails(case):
    """NaN in every slot at or past L_i of each sequence's blocks: they must never be read."""
    b = case.block_size
    for i, L in enumerate(case.seq_lens.tolist()):
        nblk = -(-L // b)
        for pos in range(L, nblk * b):
            phys = int(case.block_tables[i, pos // b])
            case.k_pool[phys, :, pos % b] = float("nan")
            case.v_pool[phys, :, pos % b] = float("nan")
    return case


def _gpu(*ts):
    return [t.to(DEV, copy=True) for t in ts]


def _oracle_pools(case):
    """Pools after the oracle's chunk scatter, as numpy bit arrays."""
    return oracle.write_kv_varlen(bits(case.k_pool), bits(case.v_pool), bits(case.k_new), bits(case.v_new),
                                  case.block_tables.numpy(), case.seq_lens.numpy(), case.q_start.numpy(),
                                  case.block_size)


def _as_float(arr, like):
    return to_f32_view(from_bits(arr, like.dtype).reshape(like.shape))


def _run(pa, case, out_dtype=torch.float32):
    kn, vn, kp, vp, tables, lens, qs, q = _gpu(case.k_new, case.v_new, case.k_pool, case.v_pool, case.block_tables,
                                               case.seq_lens, case.q_start, case.q)
    pa.write_kv_varlen(kn, vn, kp, vp, tables, lens, qs, case.max_chunk)
    out = pa.prefill(q, kp, vp, tables, lens, qs, case.scale, case.max_chunk, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return out, kp, vp


HISTS = [0, 15, 16, 47, 100, 7, 300, 1]
CHUNKS = [1, 31, 32, 33, 129, 0, 200, 64]


@pytest.mark.parametrize("b,dtype", [(16, torch.bfloat16), (4, torch.bfloat16), (32, torch.float32),
                                     (8, torch.float32)])
def test_write_kv_varlen_bit_exact(gpu_lib, b, dtype):
    case = build_prefill_case(histories=HISTS, chunks=CHUNKS, num_q_heads=4, num_kv_heads=2, head_dim=64,
                              block_size=b, dtype=dtype, seed=40 + b, pool_slack=0.2)
    print(f"[case] write_kv_varlen b={b} {dtype}", flush=True)
    kn, vn, kp, vp, tables, lens, qs = _gpu(case.k_new, case.v_new, case.k_pool, case.v_pool, case.block_tables,
                                            case.seq_lens, case.q_start)
    gpu_lib.write_kv_varlen(kn, vn, kp, vp, tables, lens, qs, case.max_chunk)
    torch.cuda.synchronize()
    want_k, want_v = _oracle_pools(case)
    assert np.array_equal(bits(kp), want_k)
    assert np.array_equal(bits(vp), want_v)


@pytest.mark.parametrize("b,hq,hkv", [(16, 32, 8), (16, 8, 8), (16, 16, 2), (16, 12, 4), (16, 64, 2),
                                      (16, 128, 1), (4, 32, 8), (8, 32, 8), (32, 32, 8)])
def test_prefill_shapes(gpu_lib, b, hq, hkv):
    """GQA groups 1, 3, 4, 8, 32 and 128; chunks of 0, 1, 31, 32, 33, 64, 129 and 200 tokens after
    histories of 0 .. 300 positions (query blocks with ragged tails, tiles crossing the diagonal)."""
    case = _poison_tails(build_prefill_case(histories=HISTS, chunks=CHUNKS, num_q_heads=hq, num_kv_heads=hkv,
                                            head_dim=128, block_size=b, seed=hq * 3 + b, pool_slack=0.2))
    print(f"[case] prefill b={b} hq={hq} hkv={hkv}", flush=True)
    out, _, _ = _run(gpu_lib, case)
    kp, vp = _oracle_pools(case)
    ref = oracle.prefill(case.q.float().numpy(), _as_float(kp, case.k_pool), _as_float(vp, case.v_pool),
                         case.block_tables.numpy(), case.seq_lens.numpy(), case.q_start.numpy(), case.scale, b)
    assert_attention_close(out.cpu(), ref, kv_dtype=torch.bfloat16, out_dtype=torch.float32, what="prefill")


def test_prefill_bf16_output(gpu_lib):
    case = make_prefill_case("prefill_small")
    print("[case] prefill bf16 out", flush=True)
    out, _, _ = _run(gpu_lib, case, out_dtype=torch.bfloat16)
    kp, vp = _oracle_pools(case)
    ref = oracle.prefill(case.q.float().numpy(), _as_float(kp, case.k_pool), _as_float(vp, case.v_pool),
                         case.block_tables.numpy(), case.seq_lens.numpy(), case.q_start.numpy(), case.scale, 16)
    assert_attention_close(out.cpu(), ref, kv_dtype=torch.bfloat16, out_dtype=torch.bfloat16, what="bf16 out")


def test_prefill_permuted_blocks_bitwise(gpu_lib):
    """Relabelling physical blocks (pool rows and table entries together) leaves the output bit-identical."""
    case = make_prefill_case("prefill_small")
    print("[case] prefill permuted blocks", flush=True)
    a, kp, vp = _run(gpu_lib, case)
    n = kp.shape[0]
    perm = torch.randperm(n, generator=torch.Generator().manual_seed(9)).to(DEV)
    kp2, vp2 = torch.empty_like(kp), torch.empty_like(vp)
    kp2[perm], vp2[perm] = kp, vp
    tab = case.block_tables.clone()
    valid = tab < n
    tab[valid] = perm.cpu()[tab[valid].long()].to(torch.int32)
    q, lens, qs = _gpu(case.q, case.seq_lens, case.q_start)
    b_out = gpu_lib.prefill(q, kp2, vp2, tab.to(DEV), lens, qs, case.scale, case.max_chunk)
    torch.cuda.synchronize()
    assert torch.equal(a, b_out)


def test_prefill_large_scores_rescale(gpu_lib):
    """Scores that grow along the history by about 550 base-2 units make later tiles outrun each row's
    reference max several times; the rescaled result still meets the bar. K rows and q point along
    head_dim 0 only, so every score is one exact bf16 product and the oracle and the kernel see the
    same scores up to the final scaling."""
    case = build_prefill_case(histories=[200, 0], chunks=[90, 150], num_q_heads=8, num_kv_heads=2, head_dim=128,
                              block_size=16, seed=77)
    ramp = torch.linspace(0.0, 60.0, 400)
    for i, L in enumerate(case.seq_lens.tolist()):
        for pos in range(L):
            phys = int(case.block_tables[i, pos // 16])
            case.k_pool[phys, :, pos % 16] = 0.0
            case.k_pool[phys, :, pos % 16, 0] = float(ramp[pos] * 12.0)
    case.k_new[:] = 0.0
    case.k_new[:, :, 0] = 8.0
    case.q[:, :, 0] = (6.0 + 0.1 * case.q[:, :, 0].float()).to(torch.bfloat16)
    print("[case] prefill rescale", flush=True)
    out, _, _ = _run(gpu_lib, case)
    kp, vp = _oracle_pools(case)
    ref = oracle.prefill(case.q.float().numpy(), _as_float(kp, case.k_pool), _as_float(vp, case.v_pool),
                         case.block_tables.numpy(), case.seq_lens.numpy(), case.q_start.numpy(), case.scale, 16)
    assert_attention_close(out.cpu(), ref, kv_dtype=torch.bfloat16, out_dtype=torch.float32, what="rescale")


def test_prefill_pa_check_rejects_bad_chunks(gpu_lib, monkeypatch):
    """Under PA_CHECK=1 a chunk longer than its sequence, or a q_start that does not start at 0, is
    refused before any launch."""
    case = make_prefill_case("prefill_small")
    q, kp, vp, tables, lens, qs = _gpu(case.q, case.k_pool, case.v_pool, case.block_tables, case.seq_lens,
                                       case.q_start)
    monkeypatch.setenv("PA_CHECK", "1")
    print("[case] prefill PA_CHECK", flush=True)
    out = gpu_lib.prefill(q, kp, vp, tables, lens, qs, case.scale, case.max_chunk)  # valid: accepted
    short = lens.clone()
    short[0] = int(case.chunks[0]) - 1
    with pytest.raises(gpu_lib.PaError) as err:
        gpu_lib.prefill(q, kp, vp, tables, short, qs, case.scale, case.max_chunk, out=out)
    assert err.value.status == -1
    shifted = qs.clone()
    shifted[0] = 1
    with pytest.raises(gpu_lib.PaError) as err:
        gpu_lib.prefill(q, kp, vp, tables, lens, shifted, case.scale, case.max_chunk, out=out)
    assert err.value.status == -1
    with pytest.raises(gpu_lib.PaError) as err:  # a chunk longer than the q_tokens bound
        gpu_lib.prefill(q, kp, vp, tables, lens, qs, case.scale, case.max_chunk - 1, out=out)
    assert err.value.status == -1
    torch.cuda.synchronize()


def test_prefill_unsupported_shapes_are_refused(gpu_lib):
    """fp32 pools and head_dim 64 have no prefill kernel: PA_ERR_UNSUPPORTED, nothing launched."""
    for kw in (dict(dtype=torch.float32, head_dim=128), dict(dtype=torch.bfloat16, head_dim=64)):
        case = build_prefill_case(histories=[5, 9], chunks=[3, 4], num_q_heads=4, num_kv_heads=2, block_size=16,
                                  seed=2, **kw)
        q, kp, vp, tables, lens, qs = _gpu(case.q, case.k_pool, case.v_pool, case.block_tables, case.seq_lens,
                                           case.q_start)
        with pytest.raises(gpu_lib.PaError) as err:
            gpu_lib.prefill(q, kp, vp, tables, lens, qs, case.scale, case.max_chunk)
        assert err.value.status == -2


def test_prefill_full_size_sampled(gpu_lib):
    """The benchmark's prefill workload (16 sequences, chunks of 512-2048 after histories of 0-4096),
    in the launch configuration the benchmark times: the whole scatter is compared bit for bit, then
    sampled output rows against the oracle row by row."""
    case = make_prefill_case("prefill")
    print(f"[case] prefill full size Q={case.q.shape[0]} pool={tuple(case.k_pool.shape)}", flush=True)
    out, kp_g, vp_g = _run(gpu_lib, case)
    kp, vp = _oracle_pools(case)
    assert np.array_equal(bits(kp_g), kp)
    assert np.array_equal(bits(vp_g), vp)
    del kp_g, vp_g
    kf, vf = _as_float(kp, case.k_pool), _as_float(vp, case.v_pool)
    got = out.cpu().double().numpy()
    qf = case.q.float().numpy()
    rng = np.random.default_rng(17)
    total, hq, _ = case.q.shape
    qs = case.q_start.numpy()
    rows = {(int(qs[i]), 0) for i in range(len(case.chunks))}                  # first token of each chunk
    rows |= {(int(qs[i + 1]) - 1, hq - 1) for i in range(len(case.chunks))}     # last token of each chunk
    rows |= {(int(rng.integers(total)), int(rng.integers(hq))) for _ in range(48)}
    rows = sorted(rows)
    ref = np.stack([oracle.prefill_row(qf, kf, vf, case.block_tables.numpy(), case.seq_lens.numpy(), qs,
                                       case.scale, 16, r, h) for r, h in rows])
    sel = np.stack([got[r, h] for r, h in rows])
    err = assert_attention_close(sel, ref, kv_dtype=torch.bfloat16, out_dtype=torch.float32, what="prefill full")
    print(f"[result] prefill: {len(rows)} sampled rows, max |err| = {err:.2e}", flush=True)
