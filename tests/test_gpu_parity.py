"""Parity of the HIP path (through the C ABI) against the float64 oracle, on the GPU.

KV writes must be bit-exact. Attention must be within 1e-5 relative per row for fp32
inputs, and within 2e-3 absolute for bf16 inputs against the oracle run on the same
bf16-rounded values (tests/helpers.assert_attention_close). Inputs come only from the
seeded generator (workloads/) and the oracle; nothing expected comes from the GPU.
"""

from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle
from tests.helpers import assert_attention_close, bits, oracle_after_write, poison_case, to_f32_view
from workloads import build_case, make_case

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
VALU, MFMA = 1, 2


def _to_gpu(case):
    """Fresh device copies: the case's own tensors stay the untouched inputs of the oracle."""
    return {k: getattr(case, k).to(DEV, copy=True) for k in ("q", "k_new", "v_new", "k_pool", "v_pool", "block_tables",
                                                    "seq_lens", "positions")}


def _oracle_decode(case, kp_bits, vp_bits):
    kp = torch.from_numpy(kp_bits.view(np.int16 if kp_bits.dtype == np.uint16 else np.int32))
    vp = torch.from_numpy(vp_bits.view(np.int16 if vp_bits.dtype == np.uint16 else np.int32))
    kp = kp.view(case.k_pool.dtype).reshape(case.k_pool.shape)
    vp = vp.view(case.v_pool.dtype).reshape(case.v_pool.shape)
    return oracle.decode(to_f32_view(case.q), to_f32_view(kp), to_f32_view(vp), case.block_tables.numpy(),
                         case.seq_lens.numpy(), case.scale, case.block_size)


def _run_step(pa, case, *, partitioned=False, partition_tokens=512, out_dtype=torch.float32, variant=0,
              max_seq_len=None):
    g = _to_gpu(case)
    pa.write_kv(g["k_new"], g["v_new"], g["k_pool"], g["v_pool"], g["block_tables"], g["positions"])
    if partitioned:
        out = pa.decode_partitioned(g["q"], g["k_pool"], g["v_pool"], g["block_tables"], g["seq_lens"], case.scale,
                                    max_seq_len or case.max_seq_len, partition_tokens, out_dtype=out_dtype,
                                    variant=variant)
    else:
        out = pa.decode(g["q"], g["k_pool"], g["v_pool"], g["block_tables"], g["seq_lens"], case.scale,
                        out_dtype=out_dtype, variant=variant)
    torch.cuda.synchronize()
    return g, out


def _check_step(pa, case, **kw):
    print(f"[case] {case.name} B={case.q.shape[0]} T={case.q.shape[1]} Hq={case.q.shape[2]} "
          f"Hkv={case.k_pool.shape[1]} b={case.block_size} kw={kw}", flush=True)
    poison_case(case)
    g, out = _run_step(pa, case, **kw)
    kp, vp = oracle_after_write(case)
    assert np.array_equal(bits(g["k_pool"]), kp), "K pool differs from the oracle's write"
    assert np.array_equal(bits(g["v_pool"]), vp), "V pool differs from the oracle's write"
    ref = _oracle_decode(case, kp, vp)
    return assert_attention_close(out.cpu(), ref, kv_dtype=case.k_pool.dtype,
                                  out_dtype=kw.get("out_dtype", torch.float32), what=case.name)


# ----------------------------------------------------------------------------- KV write

@pytest.mark.parametrize("name", ["tiny", "tiny_b4", "batch64"])
def test_write_kv_bit_exact(gpu_lib, name):
    case = make_case(name)
    g = _to_gpu(case)
    gpu_lib.write_kv(g["k_new"], g["v_new"], g["k_pool"], g["v_pool"], g["block_tables"], g["positions"])
    torch.cuda.synchronize()
    kp, vp = oracle_after_write(case)
    assert np.array_equal(bits(g["k_pool"]), kp)
    assert np.array_equal(bits(g["v_pool"]), vp)


def test_write_kv_worked_example(gpu_lib):
    """[P1] 'Paging': b = 4, table [5, 1, 7]; position 9 goes to physical block 7, offset 1."""
    case = make_case("tiny_b4")
    g = _to_gpu(case)
    before = bits(g["k_pool"]).copy()
    gpu_lib.write_kv(g["k_new"], g["v_new"], g["k_pool"], g["v_pool"], g["block_tables"], g["positions"])
    torch.cuda.synchronize()
    after = bits(g["k_pool"])
    assert np.array_equal(after[7, :, 1, :], bits(case.k_new)[0, 0])
    changed = np.argwhere((after != before).any(axis=-1))
    assert {(int(b), int(o)) for b, _, o in changed} == {(7, 1)}


def test_write_kv_multi_token_bf16(gpu_lib):
    case = build_case(lengths=[4, 17, 64, 33], num_q_heads=16, num_kv_heads=2, head_dim=128, block_size=8,
                      q_tokens=4, dtype=torch.bfloat16, seed=5)
    g = _to_gpu(case)
    gpu_lib.write_kv(g["k_new"], g["v_new"], g["k_pool"], g["v_pool"], g["block_tables"], g["positions"])
    torch.cuda.synchronize()
    kp, vp = oracle_after_write(case)
    assert np.array_equal(bits(g["k_pool"]), kp) and np.array_equal(bits(g["v_pool"]), vp)


# ----------------------------------------------------------------------------- decode, small cases

@pytest.mark.parametrize("name", ["tiny", "tiny_b4"])
@pytest.mark.parametrize("partitioned", [False, True])
def test_decode_tiny_fp32(gpu_lib, name, partitioned):
    _check_step(gpu_lib, make_case(name), partitioned=partitioned, partition_tokens=16)


@pytest.mark.parametrize("variant", [VALU, MFMA])
@pytest.mark.parametrize("name,num_seqs", [("batch64", 8), ("long", 2), ("prefix", 4), ("spec", 3)])
@pytest.mark.parametrize("partitioned", [False, True])
def test_decode_config_shapes_bf16(gpu_lib, name, num_seqs, partitioned, variant):
    """Each bf16 workload's shapes and length mix, on its first sequences (the oracle runs in full),
    through both kernel families."""
    _check_step(gpu_lib, make_case(name, num_seqs=num_seqs), partitioned=partitioned, partition_tokens=512,
                variant=variant)


@pytest.mark.parametrize("variant", [VALU, MFMA])
@pytest.mark.parametrize("b", [4, 8, 16, 32])
@pytest.mark.parametrize("hq,hkv,t", [(4, 4, 1), (8, 4, 1), (8, 2, 1), (16, 2, 1), (8, 2, 2), (12, 4, 3),
                                      (16, 2, 4), (4, 1, 4), (32, 4, 3), (64, 8, 4)])
def test_decode_shapes_and_tails_bf16(gpu_lib, b, hq, hkv, t, variant):
    """Block sizes 4-32, GQA groups 1-8, 1-4 causal query tokens (up to 32 rows per kv head),
    and lengths at block and tile boundaries (b-1, b, b+1, 15, 16, 17, ...) in one launch,
    single-pass and with 32- and 48-position partitions (the latter splits tile pairs)."""
    lengths = sorted({max(t, x) for x in (b - 1, b, b + 1, 15, 16, 17, 31, 33, 47, 100, 257)})
    for kw in (dict(), dict(partitioned=True, partition_tokens=32),
               dict(partitioned=True, partition_tokens=48 if 48 % b == 0 else 64)):
        case = build_case(lengths=lengths, num_q_heads=hq, num_kv_heads=hkv, head_dim=128, block_size=b,
                          q_tokens=t, dtype=torch.bfloat16, seed=b * 100 + hq * 10 + t, pool_slack=0.2)
        _check_step(gpu_lib, case, variant=variant, **kw)


@pytest.mark.parametrize("variant", [0, VALU])
@pytest.mark.parametrize("b", [4, 16])
@pytest.mark.parametrize("hq,hkv,t", [(8, 2, 5), (16, 4, 6), (8, 2, 8), (16, 2, 8), (32, 4, 8)])
def test_decode_five_to_eight_query_tokens(gpu_lib, b, hq, hkv, t, variant):
    """5-8 causal query tokens per sequence (10-64 query rows per kv head): the default choice (matrix
    cores up to 32 rows, the vector-ALU kernel's 8-row groups above) and the vector-ALU kernel forced,
    single pass and split, against the oracle. Forcing the matrix cores on more than 32 rows is refused."""
    lengths = sorted({max(t, x) for x in (t, b - 1, b, b + 1, 15, 16, 17, 31, 33, 47, 100, 257)})
    for kw in (dict(), dict(partitioned=True, partition_tokens=32), dict(partitioned=True, partition_tokens=48)):
        case = build_case(lengths=lengths, num_q_heads=hq, num_kv_heads=hkv, head_dim=128, block_size=b,
                          q_tokens=t, dtype=torch.bfloat16, seed=9100 + b * 100 + hq * 10 + t, pool_slack=0.2)
        _check_step(gpu_lib, case, variant=variant, **kw)
    if t * (hq // hkv) > 32:
        g = _to_gpu(case)
        with pytest.raises(gpu_lib.PaError) as err:
            gpu_lib.decode(g["q"], g["k_pool"], g["v_pool"], g["block_tables"], g["seq_lens"], case.scale,
                           variant=MFMA)
        assert err.value.status == -2


@pytest.mark.parametrize("variant", [VALU, MFMA])
@pytest.mark.parametrize("partition_tokens,msl_factor", [(16, 1), (48, 1), (16, 2), (32, 3)])
def test_many_partitions_per_sequence(gpu_lib, partition_tokens, msl_factor, variant):
    """Dozens of short partitions per sequence, with max_seq_len at 1-3x the longest sequence (partitions
    past a sequence's end are never written and never read)."""
    case = make_case("batch64", num_seqs=32)
    _check_step(gpu_lib, case, partitioned=True, partition_tokens=partition_tokens, variant=variant,
                max_seq_len=case.max_seq_len * msl_factor)


@pytest.mark.parametrize("t", [1, 3])
def test_decode_fp32_shapes(gpu_lib, t):
    case = build_case(lengths=[t, 5, 16, 47, 130], num_q_heads=8, num_kv_heads=2, head_dim=64, block_size=8,
                      q_tokens=t, dtype=torch.float32, seed=77 + t)
    _check_step(gpu_lib, case)


@pytest.mark.parametrize("variant", [VALU, MFMA])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_decode_bf16_output(gpu_lib, out_dtype, variant):
    _check_step(gpu_lib, make_case("batch64", num_seqs=6), out_dtype=out_dtype, variant=variant)
    _check_step(gpu_lib, make_case("batch64", num_seqs=6), out_dtype=out_dtype, partitioned=True,
                partition_tokens=64, variant=variant)


@pytest.mark.parametrize("variant", [VALU, MFMA])
def test_single_position_returns_v0_bitwise(gpu_lib, variant):
    """L = 1: softmax weight exactly 1, so fp32 output == v_0 bit for bit (bf16 and fp32 pools)."""
    for dtype, d in ((torch.float32, 64), (torch.bfloat16, 128)):
        if dtype == torch.float32 and variant == MFMA:
            continue
        case = build_case(lengths=[1, 1, 1], num_q_heads=8, num_kv_heads=2, head_dim=d, block_size=16,
                          dtype=dtype, seed=3)
        g, out = _run_step(gpu_lib, case, variant=variant)
        want = case.v_new[:, 0].to(torch.float32).repeat_interleave(4, dim=1)  # [B, Hq, D]
        assert torch.equal(out[:, 0].cpu(), want)


@pytest.mark.parametrize("variant", [VALU, MFMA])
def test_permuted_physical_blocks_bitwise(gpu_lib, variant):
    """Relabelling the physical blocks (pool rows + table entries) leaves the GPU output bit-identical."""
    case = make_case("batch64", num_seqs=8)
    g, out_a = _run_step(gpu_lib, case, variant=variant)
    n = case.k_pool.shape[0]
    perm = torch.randperm(n, generator=torch.Generator().manual_seed(9))
    kp2 = torch.empty_like(case.k_pool)
    vp2 = torch.empty_like(case.v_pool)
    kp2[perm] = case.k_pool
    vp2[perm] = case.v_pool
    tab = case.block_tables.clone()
    valid = tab < n
    tab[valid] = perm[tab[valid].long()].to(torch.int32)
    case.k_pool, case.v_pool, case.block_tables = kp2, vp2, tab
    _, out_b = _run_step(gpu_lib, case, variant=variant)
    assert torch.equal(out_a, out_b)


def test_shared_prefix_equals_private_copies_bitwise(gpu_lib):
    """Sequences whose first blocks are one shared physical copy give the same output, bit for bit,
    as the same data held in private blocks."""
    shared = make_case("prefix", num_seqs=4)
    g, out_shared = _run_step(gpu_lib, shared)
    kp, vp = shared.k_pool.clone(), shared.v_pool.clone()
    rows = [list(r) for r in shared.table_rows]
    extra = []
    next_id = kp.shape[0]
    for i in range(1, len(rows)):          # give every sequence but the first its own prefix copy
        for j in range(128):
            extra.append(rows[i][j])
            rows[i][j] = next_id
            next_id += 1
    idx = torch.tensor(extra, dtype=torch.int64)
    kp = torch.cat([kp, kp[idx]])
    vp = torch.cat([vp, vp[idx]])
    tab = shared.block_tables.clone()
    for i, r in enumerate(rows):
        tab[i, :len(r)] = torch.tensor(r, dtype=torch.int32)
    shared.k_pool, shared.v_pool, shared.block_tables = kp, vp, tab
    _, out_private = _run_step(gpu_lib, shared)
    assert torch.equal(out_shared, out_private)


def test_one_partition_equals_single_pass_bitwise(gpu_lib):
    """Vector-ALU kernel: a split run with one partition covering every sequence does the same
    arithmetic as the single pass (the merge of one partial is exact), so the two agree bit for bit."""
    case = make_case("batch64", num_seqs=8)
    big = ((case.max_seq_len + 15) // 16) * 16
    _, a = _run_step(gpu_lib, case, variant=VALU)
    _, b = _run_step(gpu_lib, case, partitioned=True, partition_tokens=big, variant=VALU)
    assert torch.equal(a, b)


def test_one_partition_mfma_matches_oracle(gpu_lib):
    """Matrix-core kernel: the single pass spreads a sequence's tiles over four waves, while one
    partition hands them all to one wave, so the two differ only in summation order; both meet the
    oracle bar."""
    case = make_case("batch64", num_seqs=8)
    big = ((case.max_seq_len + 15) // 16) * 16
    _check_step(gpu_lib, case, variant=MFMA)
    _check_step(gpu_lib, make_case("batch64", num_seqs=8), partitioned=True, partition_tokens=big, variant=MFMA)


@pytest.mark.parametrize("variant", [VALU, MFMA])
def test_partitioned_workspace_reuse(gpu_lib, variant):
    """One workspace, sized for the largest call and filled with garbage first, serves a sequence of
    calls with different batch sizes: each result matches the oracle, and repeating the first call
    reproduces its output bit for bit (nothing left in the workspace leaks into a result)."""
    msl, pt = 512, 64
    big = make_case("batch64", num_seqs=16)
    small = make_case("batch64", num_seqs=6, seed=4242)
    need = gpu_lib.workspace_bytes(big.q, big.k_pool, big.block_tables, msl, pt, variant=variant)
    ws = torch.full((need,), 0x7F, dtype=torch.uint8, device=DEV)  # every float in it reads as 3.4e38
    outs = []
    for case in (big, small, big):
        print(f"[case] reuse B={case.q.shape[0]} variant={variant}", flush=True)
        g = _to_gpu(case)
        out = gpu_lib.decode_partitioned(g["q"], g["k_pool"], g["v_pool"], g["block_tables"], g["seq_lens"],
                                         case.scale, msl, pt, workspace=ws, variant=variant)
        torch.cuda.synchronize()
        kp, vp = bits(case.k_pool), bits(case.v_pool)
        assert_attention_close(out.cpu(), _oracle_decode(case, kp, vp), kv_dtype=torch.bfloat16,
                               out_dtype=torch.float32, what=f"reuse B={case.q.shape[0]}")
        outs.append(out.cpu())
    assert torch.equal(outs[0], outs[2])


def test_pa_check_rejects_bad_table_before_launch(gpu_lib, monkeypatch):
    """PA_CHECK=1: valid inputs give the usual result; a table entry outside the pool is refused on the
    host with PA_ERR_INVALID_ARG. (The MFMA kernel is forced: it clamps block ids into the pool, so even
    an unchecked launch could not read outside it.)"""
    case = make_case("batch64", num_seqs=4)
    g = _to_gpu(case)
    ref = gpu_lib.decode(g["q"], g["k_pool"], g["v_pool"], g["block_tables"], g["seq_lens"], case.scale,
                         variant=MFMA)
    monkeypatch.setenv("PA_CHECK", "1")
    out = gpu_lib.decode(g["q"], g["k_pool"], g["v_pool"], g["block_tables"], g["seq_lens"], case.scale,
                         variant=MFMA)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
    bad = g["block_tables"].clone()
    bad[1, 0] = case.k_pool.shape[0]
    with pytest.raises(gpu_lib.PaError) as err:
        gpu_lib.decode(g["q"], g["k_pool"], g["v_pool"], bad, g["seq_lens"], case.scale, variant=MFMA)
    assert err.value.status == -1


def test_table_padding_never_read(gpu_lib):
    """Padding INT32_MAX (default) and 0 give identical results: padding is never dereferenced."""
    a = make_case("batch64", num_seqs=5)
    b = make_case("batch64", num_seqs=5, table_pad=0)
    _, oa = _run_step(gpu_lib, a)
    _, ob = _run_step(gpu_lib, b)
    assert torch.equal(oa, ob)


@pytest.mark.parametrize("b,hq,hkv,t", [(16, 32, 8, 1), (8, 16, 2, 4), (32, 64, 8, 4)])
def test_longest_first_batches(gpu_lib, b, hq, hkv, t):
    """Single passes over 128 to 512 sequences deal the sequences longest first (the j-th workgroup of a
    kv head takes length rank j, ties by index): lengths drawn from a few values, so most are tied, and
    every row still meets the oracle, separate and fused."""
    gen = torch.Generator().manual_seed(4100 + b + t)
    pool_of_lengths = torch.tensor([t, 5, 17, 64, 100, 150, 151, 300])
    lengths = pool_of_lengths[torch.randint(0, len(pool_of_lengths), (200,), generator=gen)].tolist()
    case = build_case(lengths=lengths, num_q_heads=hq, num_kv_heads=hkv, head_dim=128, block_size=b, q_tokens=t,
                      dtype=torch.bfloat16, seed=4200 + b + t, pool_slack=0.1)
    _check_step(gpu_lib, case, variant=MFMA)
    a, out_a, g, out_b = _fused_vs_separate(gpu_lib, case)
    assert torch.equal(out_a, out_b)
    assert np.array_equal(bits(a["k_pool"]), bits(g["k_pool"]))


def test_zero_query_averages_values(gpu_lib):
    case = build_case(lengths=[5, 40, 200], num_q_heads=8, num_kv_heads=2, head_dim=128, block_size=16,
                      q_tokens=2, dtype=torch.bfloat16, seed=12)
    case.q.zero_()
    g, out = _run_step(gpu_lib, case)
    kp, vp = oracle_after_write(case)
    vpool = torch.from_numpy(vp.view(np.int16)).view(torch.bfloat16).reshape(case.v_pool.shape).double().numpy()
    for i, L in enumerate([5, 40, 200]):
        for t in range(2):
            n = L - 2 + t + 1
            for h in range(8):
                vals = oracle.gather_positions(vpool, case.block_tables[i].numpy(), np.arange(n), h // 4, 16)
                np.testing.assert_allclose(out[i, t, h].cpu().double().numpy(), vals.mean(axis=0), atol=2e-6)


# ----------------------------------------------------------------------------- full-size workloads

def _sampled_rows(case, rng, n_random=48):
    b, t, hq, _ = case.q.shape
    rows = {(0, tt, h) for tt in range(t) for h in range(hq)} | {(b - 1, tt, h) for tt in range(t) for h in range(hq)}
    longest = int(torch.argmax(case.seq_lens))
    rows |= {(longest, t - 1, h) for h in range(hq)}
    while len(rows) < n_random + 3 * t * hq:
        rows.add((int(rng.integers(b)), int(rng.integers(t)), int(rng.integers(hq))))
    return sorted(rows)


@pytest.mark.parametrize("name,partitioned,variant", [("batch64", False, 0), ("batch64", True, 0), ("long", True, 0),
                                                      ("spec", False, 0),
                                                      ("prefix", True, 0), ("spec", True, 0), ("batch64", False, VALU),
                                                      ("long", True, VALU)])
def test_full_size_sampled(gpu_lib, name, partitioned, variant):
    """Full workload sizes in the launch configuration the benchmark times (512-token partitions for the
    long/prefix/speculative cases): the complete KV write is compared bit for bit, and sampled output rows
    against the oracle computed row by row."""
    case = make_case(name, pool_device=DEV)
    print(f"[case] full {name} partitioned={partitioned} pool={tuple(case.k_pool.shape)}", flush=True)
    g, out = _run_step(gpu_lib, case, partitioned=partitioned, partition_tokens=512, variant=variant)
    kp, vp = oracle_after_write(case)
    assert np.array_equal(bits(g["k_pool"]), kp)
    assert np.array_equal(bits(g["v_pool"]), vp)
    del g
    kpool = torch.from_numpy(kp.view(np.int16)).view(torch.bfloat16).reshape(case.k_pool.shape).float().numpy()
    vpool = torch.from_numpy(vp.view(np.int16)).view(torch.bfloat16).reshape(case.v_pool.shape).float().numpy()
    q = case.q.float().numpy()
    tables, lens = case.block_tables.numpy(), case.seq_lens.numpy()
    rng = np.random.default_rng(len(name))
    rows = _sampled_rows(case, rng)
    got = out.cpu().double().numpy()
    ref = np.stack([oracle.decode_row(q, kpool, vpool, tables, lens, case.scale, case.block_size, i, t, h)
                    for i, t, h in rows])
    sel = np.stack([got[i, t, h] for i, t, h in rows])
    err = assert_attention_close(sel, ref, kv_dtype=torch.bfloat16, out_dtype=torch.float32, what=name)
    print(f"[result] {name}: {len(rows)} sampled rows, max |err| = {err:.2e}", flush=True)


# ----------------------------------------------------------------------------- fused append + decode

def _fused_vs_separate(pa, case, *, partition_tokens=None, variant_sep=MFMA, split_schedule=0):
    """Run pa_write_kv + decode and pa_write_kv_decode on copies of the same inputs; return both
    (pools, out) so callers can require bit identity."""
    a = _to_gpu(case)
    pa.write_kv(a["k_new"], a["v_new"], a["k_pool"], a["v_pool"], a["block_tables"], a["positions"])
    if partition_tokens:
        out_a = pa.decode_partitioned(a["q"], a["k_pool"], a["v_pool"], a["block_tables"], a["seq_lens"], case.scale,
                                      case.max_seq_len, partition_tokens, variant=variant_sep,
                                      split_schedule=split_schedule)
    else:
        out_a = pa.decode(a["q"], a["k_pool"], a["v_pool"], a["block_tables"], a["seq_lens"], case.scale,
                          variant=variant_sep)
    b = _to_gpu(case)
    out_b = pa.write_kv_decode(b["q"], b["k_new"], b["v_new"], b["k_pool"], b["v_pool"], b["block_tables"],
                               b["seq_lens"], case.scale, max_seq_len=case.max_seq_len if partition_tokens else None,
                               partition_tokens=partition_tokens, split_schedule=split_schedule)
    torch.cuda.synchronize()
    return a, out_a, b, out_b


@pytest.mark.parametrize("b", [4, 8, 16, 32])
@pytest.mark.parametrize("hq,hkv,t", [(4, 4, 1), (32, 8, 1), (8, 2, 2), (32, 8, 2), (8, 2, 4), (16, 2, 4), (12, 4, 3), (64, 8, 4)])
def test_fused_append_decode_bitwise(gpu_lib, b, hq, hkv, t):
    """pa_write_kv_decode equals pa_write_kv followed by the MFMA decode, bit for bit (pools and out),
    single pass and split (new rows inside one partition and straddling two), and meets the oracle."""
    lengths = sorted({max(t, x) for x in (1, 2, b - 1, b, b + 1, 15, 16, 17, 31, 33, 47, 100, 257)})
    case = build_case(lengths=lengths, num_q_heads=hq, num_kv_heads=hkv, head_dim=128, block_size=b, q_tokens=t,
                      dtype=torch.bfloat16, seed=900 + b * 10 + hq + t, pool_slack=0.2)
    poison_case(case)
    print(f"[case] fused b={b} hq={hq} hkv={hkv} T={t}", flush=True)
    for pt in (None, 32, 48 if 48 % b == 0 else 64):
        a, out_a, g, out_b = _fused_vs_separate(gpu_lib, case, partition_tokens=pt)
        assert np.array_equal(bits(a["k_pool"]), bits(g["k_pool"])), f"K pool differs (pt={pt})"
        assert np.array_equal(bits(a["v_pool"]), bits(g["v_pool"])), f"V pool differs (pt={pt})"
        assert torch.equal(out_a, out_b), f"output differs (pt={pt})"
    kp, vp = oracle_after_write(case)
    assert np.array_equal(bits(g["k_pool"]), kp) and np.array_equal(bits(g["v_pool"]), vp)
    assert_attention_close(out_b.cpu(), _oracle_decode(case, kp, vp), kv_dtype=torch.bfloat16,
                           out_dtype=torch.float32, what="fused")


@pytest.mark.parametrize("name,pt,sched", [("batch64", None, 0), ("long", 512, 2), ("long", 512, 0), ("spec", None, 0)])
def test_fused_append_decode_full_size_bitwise(gpu_lib, name, pt, sched):
    """Full workload sizes: the fused step writes the pools bit for bit like the separate append, and its
    output equals the separate decode's bit for bit on the schedules that give the same bits on every
    call (single pass; long with two partitions per wave). Long under the library's choice runs balanced
    ranges, whose pairs of waves meet where their timing puts them: there both outputs agree to well
    inside the bf16 bar (every row of that call meets the oracle in the full-row tests)."""
    case = make_case(name, pool_device=DEV)
    print(f"[case] fused full {name} schedule={sched}", flush=True)
    a, out_a, g, out_b = _fused_vs_separate(gpu_lib, case, partition_tokens=pt, split_schedule=sched)
    assert torch.equal(a["k_pool"].view(torch.int16), g["k_pool"].view(torch.int16))
    assert torch.equal(a["v_pool"].view(torch.int16), g["v_pool"].view(torch.int16))
    if pt and sched == 0:
        assert gpu_lib.split_schedule(case.q, case.k_pool, case.block_tables, case.max_seq_len, pt) == \
            gpu_lib.SPLIT_BALANCED
        assert (out_a - out_b).abs().max().item() < 1e-4
    else:
        assert torch.equal(out_a, out_b)


def test_fused_append_decode_refuses_unsupported(gpu_lib):
    case = make_case("tiny")  # fp32 pools: no MFMA kernel, so no fused path
    g = _to_gpu(case)
    with pytest.raises(gpu_lib.PaError) as err:
        gpu_lib.write_kv_decode(g["q"], g["k_new"], g["v_new"], g["k_pool"], g["v_pool"], g["block_tables"],
                                g["seq_lens"], case.scale)
    assert err.value.status == -2
