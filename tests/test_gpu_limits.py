"""Size limits of the decode path, on the GPU: table rows filled to their last slot, and pools whose byte
offsets pass 4 GiB.

A full row (L = MB * b) is checked against the float64 oracle. A pool past 4 GiB is checked by relabelling:
the same blocks moved to the top of a pool of about 5 GB (and the table rewritten to match) must give the bits of
the small pool, since physical block ids do not enter the arithmetic ([P1] section "Attention that reads
through the table") and that small case meets the oracle in the other tests. Nothing expected comes from
the GPU.
"""

from __future__ import annotations

import pytest
import torch

import oracle
from tests.helpers import assert_attention_close, oracle_after_write, poison_case, to_f32_view
from workloads import build_case, int8_pools, make_case

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
VALU, MFMA = 1, 2


def _gpu(case):
    return {k: getattr(case, k).to(DEV, copy=True) for k in ("q", "k_new", "v_new", "k_pool", "v_pool", "block_tables",
                                                    "seq_lens", "positions")}


@pytest.mark.parametrize("variant", [VALU, MFMA])
@pytest.mark.parametrize("b,t", [(4, 1), (16, 1), (32, 1), (16, 4)])
def test_full_table_rows(gpu_lib, variant, b, t):
    """The longest sequence fills every slot of its table row (L = MB * b, the last block full), beside a
    one-block sequence and one a slot short of full: single pass and split, against the oracle."""
    mb = 24
    lengths = [mb * b, max(t, 1), mb * b - 1, 3 * b]
    case = build_case(lengths=lengths, num_q_heads=32, num_kv_heads=8, head_dim=128, block_size=b, q_tokens=t,
                      dtype=torch.bfloat16, seed=8100 + b + t, pool_slack=0.25)
    assert case.block_tables.shape[1] == mb
    poison_case(case)
    kp, vp = oracle_after_write(case)
    kpool = torch.from_numpy(kp.view("int16")).view(torch.bfloat16).reshape(case.k_pool.shape)
    vpool = torch.from_numpy(vp.view("int16")).view(torch.bfloat16).reshape(case.v_pool.shape)
    ref = oracle.decode(to_f32_view(case.q), to_f32_view(kpool), to_f32_view(vpool), case.block_tables.numpy(),
                        case.seq_lens.numpy(), case.scale, b)
    g = _gpu(case)
    gpu_lib.write_kv(g["k_new"], g["v_new"], g["k_pool"], g["v_pool"], g["block_tables"], g["positions"])
    print(f"[case] full rows b={b} T={t} variant={variant}", flush=True)
    outs = {"single pass": gpu_lib.decode(g["q"], g["k_pool"], g["v_pool"], g["block_tables"], g["seq_lens"],
                                          case.scale, variant=variant)}
    for pt in (64, 512):
        outs[f"split {pt}"] = gpu_lib.decode_partitioned(g["q"], g["k_pool"], g["v_pool"], g["block_tables"],
                                                         g["seq_lens"], case.scale, case.max_seq_len, pt,
                                                         variant=variant)
    torch.cuda.synchronize()
    for what, out in outs.items():
        assert_attention_close(out.cpu(), ref, kv_dtype=torch.bfloat16, out_dtype=torch.float32, what=what)


def _relabel_high(case, big_n, pools):
    """Copies of the case's used blocks at the top of pools of big_n blocks, and the matching table."""
    tab = case.block_tables.clone()
    used = sorted({int(x) for row in case.table_rows for x in row})
    new_id = {old: big_n - 1 - i for i, old in enumerate(used)}
    for i, row in enumerate(case.table_rows):
        for j, old in enumerate(row):
            tab[i, j] = new_id[old]
    src = torch.tensor(used, dtype=torch.long, device=DEV)
    dst = torch.tensor([new_id[o] for o in used], dtype=torch.long, device=DEV)
    big = []
    for pool in pools:
        x = torch.empty((big_n,) + tuple(pool.shape[1:]), dtype=pool.dtype, device=DEV)
        x[dst] = pool[src]
        big.append(x)
    return big, tab.to(DEV)


def test_pool_past_4gib_bitwise(gpu_lib):
    """bf16 pools of 160,000 blocks (5.2 GB each; the used blocks, at the top, start past byte 2^32): single pass,
    split, fused append + decode, and the write itself all give the small pool's bits."""
    case = make_case("batch64", num_seqs=12)
    big_n = 160_000
    assert (big_n - 1000) * case.k_pool[0].numel() * 2 > 2 ** 32  # every used block starts past 4 GiB
    g = _gpu(case)
    (bk, bv), btab = _relabel_high(case, big_n, (g["k_pool"], g["v_pool"]))
    print("[case] pool past 4 GiB", flush=True)
    res = []
    for kp, vp, tab in ((g["k_pool"], g["v_pool"], g["block_tables"]), (bk, bv, btab)):
        kp, vp = kp.clone(), vp.clone()
        gpu_lib.write_kv(g["k_new"], g["v_new"], kp, vp, tab, g["positions"])
        single = gpu_lib.decode(g["q"], kp, vp, tab, g["seq_lens"], case.scale)
        split = gpu_lib.decode_partitioned(g["q"], kp, vp, tab, g["seq_lens"], case.scale, case.max_seq_len, 64)
        rows = torch.stack([kp[int(tab[i, (int(case.seq_lens[i]) - 1) // 16])] for i in range(case.q.shape[0])])
        res.append((single, split, rows))
        del kp, vp
    fk, fv = bk.clone(), bv.clone()
    fused = gpu_lib.write_kv_decode(g["q"], g["k_new"], g["v_new"], fk, fv, btab, g["seq_lens"], case.scale)
    torch.cuda.synchronize()
    (s0, p0, r0), (s1, p1, r1) = res
    assert torch.equal(s0, s1) and torch.equal(p0, p1)
    assert torch.equal(r0.view(torch.int16), r1.view(torch.int16)), "the append wrote other bits past 4 GiB"
    assert torch.equal(fused, s0)


def test_int8_pool_past_4gib_bitwise(gpu_lib):
    """int8 pools (and their per-(block, kv head) scales) of 300,000 blocks, 4.9 GB each: the top blocks give
    the small pool's bits, single pass and split."""
    case = make_case("batch64", num_seqs=12)
    kc, vc, sc = (x.to(DEV) for x in int8_pools(case, seed=31))
    big_n = 300_000
    assert (big_n - 1000) * kc[0].numel() > 2 ** 32  # every used block starts past 4 GiB
    (bkc, bvc, bsc), btab = _relabel_high(case, big_n, (kc, vc, sc))
    q, tab, lens = (case.q.to(DEV), case.block_tables.to(DEV), case.seq_lens.to(DEV))
    print("[case] int8 pool past 4 GiB", flush=True)
    a = gpu_lib.decode_int8(q, kc, vc, sc, tab, lens, case.scale)
    b = gpu_lib.decode_int8(q, bkc, bvc, bsc, btab, lens, case.scale)
    pa_ = gpu_lib.decode_partitioned_int8(q, kc, vc, sc, tab, lens, case.scale, case.max_seq_len, 64)
    pb = gpu_lib.decode_partitioned_int8(q, bkc, bvc, bsc, btab, lens, case.scale, case.max_seq_len, 64)
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(pa_, pb)
