"""Parity of the int8 KV path (pa_write_kv_int8, pa_decode_int8, pa_decode_partitioned_int8) against
the int8 oracle, on the GPU.

Codes and scales written by the append must match the oracle bit for bit (both decide every code in
float32 with the same operations). Attention over int8 pools must be within the bf16 bar (2e-3
absolute) of the oracle's float64 attention over the dequantised values. Inputs come from the seeded
generators in workloads/; nothing expected comes from the GPU.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from tests.helpers import assert_attention_close
from workloads import build_case, int8_pools, make_case

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _bits(t):
    t = t.detach().cpu().contiguous()
    return t.view(torch.int32).numpy() if t.dtype == torch.float32 else t.numpy()


def _gpu(*ts):
    return [t.to(DEV, copy=True) for t in ts]


def _write(pa, g):
    """g = [k_new, v_new, k_codes, v_codes, scales, block_tables, positions] on the GPU."""
    pa.write_kv_int8(*g)


def _split(pools):
    """(k_codes, v_codes, scales [N, Hkv, 2]) -> the oracle's (k_codes, k_scales, v_codes, v_scales) in numpy."""
    kc, vc, sc = [p.cpu().numpy() for p in pools]
    return kc, np.ascontiguousarray(sc[..., 0]), vc, np.ascontiguousarray(sc[..., 1])


def _append_ref(case, pools, k_new, v_new):
    return oracle.append_int8(*_split(pools), k_new.float().numpy(), v_new.float().numpy(),
                              case.block_tables.numpy(), case.positions.numpy(), case.block_size)


def _decode_ref(case, pools):
    return oracle.decode_int8(case.q.float().numpy(), *_split(pools), case.block_tables.numpy(),
                              case.seq_lens.numpy(), case.scale, case.block_size)


def _check_append(g, ref):
    """Pools and scales after the GPU append (g[2:5]) against the oracle's, bit for bit."""
    kc, ks, vc, vs = ref
    assert np.array_equal(_bits(g[2]), kc), "k codes"
    assert np.array_equal(_bits(g[3]), vc), "v codes"
    sc = _bits(g[4])
    assert np.array_equal(sc[..., 0], ks.view(np.int32)), "k scales"
    assert np.array_equal(sc[..., 1], vs.view(np.int32)), "v scales"


# ----------------------------------------------------------------------------- append

@pytest.mark.parametrize("b,t,dtype,hkv", [(16, 1, torch.bfloat16, 8), (16, 4, torch.bfloat16, 2),
                                           (32, 1, torch.bfloat16, 4), (32, 4, torch.float32, 2),
                                           (16, 3, torch.float32, 1)])
def test_write_kv_int8_bit_exact(gpu_lib, b, t, dtype, hkv):
    """Lengths put the new rows at offset 0 of a fresh block, in the middle of a block, and (T > 1)
    across two blocks; every other sequence's new rows are 20x larger, so their block's scale grows
    and its old codes are re-quantised."""
    lengths = sorted({max(t, x) for x in (1, b - 1, b, b + 1, 2 * b + 2, 3 * b, 70, 100, 257)})
    case = build_case(lengths=lengths, num_q_heads=hkv * 2, num_kv_heads=hkv, head_dim=128, block_size=b,
                      q_tokens=t, dtype=dtype, seed=300 + b + t, pool_slack=0.3)
    case.k_new[::2] *= 20
    case.v_new[1::2] *= 20
    print(f"[case] int8 append b={b} T={t} {dtype} Hkv={hkv} lengths={lengths}", flush=True)
    pools = int8_pools(case, seed=b * 10 + t)
    g = _gpu(case.k_new, case.v_new, *pools, case.block_tables, case.positions)
    _write(gpu_lib, g)
    torch.cuda.synchronize()
    _check_append(g, _append_ref(case, pools, case.k_new, case.v_new))


# ----------------------------------------------------------------------------- decode

@pytest.mark.parametrize("b", [16, 32])
@pytest.mark.parametrize("hq,hkv,t", [(4, 1, 1), (32, 8, 1), (8, 2, 4), (64, 8, 4), (16, 2, 1), (12, 4, 3)])
def test_decode_int8_shapes(gpu_lib, b, hq, hkv, t):
    """GQA groups 1-8, 1-4 causal query tokens (up to 32 rows per kv head), lengths at tile and block
    boundaries, single pass and with 32/48/64-position partitions."""
    lengths = sorted({max(t, x) for x in (1, 15, 16, 17, b - 1, b + 1, 47, 100, 257)})
    case = build_case(lengths=lengths, num_q_heads=hq, num_kv_heads=hkv, head_dim=128, block_size=b,
                      q_tokens=t, dtype=torch.bfloat16, seed=500 + b + hq + t, pool_slack=0.2)
    pools = int8_pools(case, seed=hq * 7 + t)
    ref = _decode_ref(case, pools)
    q, tables, lens = _gpu(case.q, case.block_tables, case.seq_lens)
    kc, vc, sc = _gpu(*pools)
    print(f"[case] int8 decode b={b} hq={hq} hkv={hkv} T={t}", flush=True)
    out = gpu_lib.decode_int8(q, kc, vc, sc, tables, lens, case.scale)
    torch.cuda.synchronize()
    assert_attention_close(out.cpu(), ref, kv_dtype=torch.int8, out_dtype=torch.float32, what="single pass")
    for pt in (32, 48 if 48 % b == 0 else 64):
        out = gpu_lib.decode_partitioned_int8(q, kc, vc, sc, tables, lens, case.scale, case.max_seq_len, pt)
        torch.cuda.synchronize()
        assert_attention_close(out.cpu(), ref, kv_dtype=torch.int8, out_dtype=torch.float32, what=f"split {pt}")


def test_decode_int8_bf16_output(gpu_lib):
    case = make_case("batch64", num_seqs=6)
    pools = int8_pools(case, seed=5)
    ref = _decode_ref(case, pools)
    q, tables, lens = _gpu(case.q, case.block_tables, case.seq_lens)
    kc, vc, sc = _gpu(*pools)
    out = gpu_lib.decode_int8(q, kc, vc, sc, tables, lens, case.scale, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert_attention_close(out.cpu(), ref, kv_dtype=torch.int8, out_dtype=torch.bfloat16, what="bf16 out")


def test_append_then_decode_step(gpu_lib):
    """One whole int8 decode step (append the new token, then attend) against the oracle's step."""
    case = make_case("batch64", num_seqs=12)
    pools = int8_pools(case, seed=9)
    g = _gpu(case.k_new, case.v_new, *pools, case.block_tables, case.positions)
    _write(gpu_lib, g)
    q, lens = _gpu(case.q, case.seq_lens)
    out = gpu_lib.decode_int8(q, g[2], g[3], g[4], g[5], lens, case.scale)
    torch.cuda.synchronize()
    kc, ks, vc, vs = _append_ref(case, pools, case.k_new, case.v_new)
    ref = oracle.decode_int8(case.q.float().numpy(), kc, ks, vc, vs, case.block_tables.numpy(),
                             case.seq_lens.numpy(), case.scale, case.block_size)
    assert_attention_close(out.cpu(), ref, kv_dtype=torch.int8, out_dtype=torch.float32, what="step")


def test_decode_int8_permuted_blocks_bitwise(gpu_lib):
    """Relabelling physical blocks (codes, scales and table entries together) leaves the output
    bit-identical."""
    case = make_case("batch64", num_seqs=8)
    kc, vc, sc = int8_pools(case, seed=11)
    q, tables, lens = _gpu(case.q, case.block_tables, case.seq_lens)
    a = gpu_lib.decode_int8(q, *_gpu(kc, vc, sc), tables, lens, case.scale)
    n = kc.shape[0]
    perm = torch.randperm(n, generator=torch.Generator().manual_seed(4))
    moved = []
    for x in (kc, vc, sc):
        y = torch.empty_like(x)
        y[perm] = x
        moved.append(y)
    tab = case.block_tables.clone()
    valid = tab < n
    tab[valid] = perm[tab[valid].long()].to(torch.int32)
    b_out = gpu_lib.decode_int8(q, *_gpu(*moved), tab.to(DEV), lens, case.scale)
    torch.cuda.synchronize()
    assert torch.equal(a, b_out)


def test_int8_unsupported_shapes_are_refused(gpu_lib):
    """b = 8 (a tile would span two blocks and two scales) and head_dim 64 have no int8 kernel: the
    call returns PA_ERR_UNSUPPORTED and launches nothing."""
    for kw in (dict(block_size=8, head_dim=128), dict(block_size=16, head_dim=64)):
        case = build_case(lengths=[20, 40], num_q_heads=8, num_kv_heads=2, dtype=torch.bfloat16, seed=1, **kw)
        pools = _gpu(*int8_pools(case, seed=2))
        q, tables, lens = _gpu(case.q, case.block_tables, case.seq_lens)
        with pytest.raises(gpu_lib.PaError) as err:
            gpu_lib.decode_int8(q, pools[0], pools[1], pools[2], tables, lens, case.scale)
        assert err.value.status == -2


# ----------------------------------------------------------------------------- full size, sampled

@pytest.mark.parametrize("name,partition_tokens", [("batch64", None), ("long", 512)])
def test_int8_full_size_sampled(gpu_lib, name, partition_tokens):
    """Full workload sizes with int8 pools, in the launch configuration the benchmark times: the whole
    append is compared bit for bit, then sampled output rows against the oracle row by row."""
    case = make_case(name, pool_device=DEV)
    pools = int8_pools(case, seed=21)
    print(f"[case] int8 full {name} pool={tuple(case.k_pool.shape)}", flush=True)
    g = _gpu(case.k_new, case.v_new, *pools, case.block_tables, case.positions)
    _write(gpu_lib, g)
    q, lens = _gpu(case.q, case.seq_lens)
    if partition_tokens:
        out = gpu_lib.decode_partitioned_int8(q, g[2], g[3], g[4], g[5], lens, case.scale, case.max_seq_len,
                                              partition_tokens)
    else:
        out = gpu_lib.decode_int8(q, g[2], g[3], g[4], g[5], lens, case.scale)
    torch.cuda.synchronize()
    kc, ks, vc, vs = _append_ref(case, pools, case.k_new, case.v_new)
    _check_append(g, (kc, ks, vc, vs))
    del g, pools
    got = out.cpu().double().numpy()
    qf = case.q.float().numpy()
    tables, lens_np = case.block_tables.numpy(), case.seq_lens.numpy()
    rng = np.random.default_rng(len(name) + 100)
    b, t, hq, _ = case.q.shape
    rows = sorted({(0, 0, h) for h in range(hq)} | {(b - 1, 0, h) for h in range(hq)}
                  | {(int(rng.integers(b)), int(rng.integers(t)), int(rng.integers(hq))) for _ in range(48)})
    ref = np.stack([oracle.decode_row_int8(qf, kc, ks, vc, vs, tables, lens_np, case.scale, case.block_size, i, tt, h)
                    for i, tt, h in rows])
    sel = np.stack([got[i, tt, h] for i, tt, h in rows])
    err = assert_attention_close(sel, ref, kv_dtype=torch.int8, out_dtype=torch.float32, what=name)
    print(f"[result] int8 {name}: {len(rows)} sampled rows, max |err| = {err:.2e}", flush=True)
