"""Pins for the float64 oracle (CPU only).

Each oracle function is checked against something other than itself: the pages'
worked examples (tests/golden/slot_examples.json), a library routine (torch
index_put scatter, torch scaled_dot_product_attention in float64), closed forms,
invariants, or brute force. ``test_planted_mistakes_are_caught`` plants plausible
mistakes in a copy of the oracle and shows that these pins catch each one.
"""

from __future__ import annotations

import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from oracle import pa_oracle
from tests.helpers import bits, to_f64

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "slot_examples.json")


def _golden():
    with open(GOLDEN, encoding="utf-8") as fh:
        return json.load(fh)


# ----------------------------------------------------------------------------- slot mapping

@pytest.mark.parametrize("ex", _golden()["slots"], ids=lambda e: f"b{e['b']}-p{e['pos']}")
def test_physical_slot_worked_examples(ex):
    assert oracle.physical_slot(ex["table"], ex["pos"], ex["b"]) == tuple(ex["expect"]), ex["cite"]


@pytest.mark.parametrize("ex", _golden()["slots"], ids=lambda e: f"b{e['b']}-p{e['pos']}")
def test_gather_positions_worked_examples(ex):
    """gather_positions on a pool whose every slot stores its own (block, offset)."""
    b, table = ex["b"], ex["table"]
    n_blocks = max(table) + 1
    pool = np.zeros((n_blocks, 2, b, 2))
    pool[:, :, :, 0] = np.arange(n_blocks)[:, None, None]
    pool[:, :, :, 1] = np.arange(b)[None, None, :]
    rows = oracle.gather_positions(pool, table, [ex["pos"]], kv_head=1, block_size=b)
    assert tuple(rows[0].astype(int)) == tuple(ex["expect"]), ex["cite"]


@pytest.mark.parametrize("ex", _golden()["blocks"], ids=lambda e: f"L{e['tokens']}")
def test_blocks_needed_and_waste_printed_numbers(ex):
    assert oracle.blocks_needed(ex["tokens"], ex["b"]) == ex["blocks"], ex["cite"]
    assert oracle.tail_waste(ex["tokens"], ex["b"]) == ex["waste"], ex["cite"]


def _brute_force_blocks(length, b):
    """Append tokens one at a time, taking a new block whenever the count is a multiple of b
    ([P2] task 09.1 rule: a new physical block only when len % 16 == 0)."""
    blocks = 0
    for n in range(length):
        if n % b == 0:
            blocks += 1
    return blocks


@pytest.mark.parametrize("b", [1, 4, 8, 16, 32])
def test_blocks_needed_brute_force(b):
    for length in range(0, 300):
        nb = _brute_force_blocks(length, b)
        assert oracle.blocks_needed(length, b) == nb
        waste = oracle.tail_waste(length, b)
        assert waste == nb * b - length
        assert 0 <= waste <= b - 1  # at most b - 1 wasted slots ([P1] "Paging"; [P2] section 2)


def test_demo_utilisation_arithmetic():
    """[P1] 'Reserved memory is wasted memory': 9,924 tokens, 32 x 1,024 static slots, 10,144 paged slots.
    The per-request lengths are not printed, so only the arithmetic is consistent-checked."""
    assert 10144 % 16 == 0 and 10144 // 16 == 634
    assert round(9924 / 32768, 3) == 0.303
    assert round(9924 / 10144, 3) == 0.978
    assert 10144 - 9924 < 32 * 16  # under b - 1 waste for each of the 32 requests


def test_visible_length_against_full_causal_mask():
    """Token t of T new tokens sits at position L - T + t; the number of ones in that row of a
    lower-triangular L x L causal mask (torch.tril) is the count it may attend to."""
    for seq_len in (1, 2, 5, 17, 40):
        mask = torch.ones(seq_len, seq_len).tril()
        for n_tok in range(1, min(seq_len, 5) + 1):
            for t in range(n_tok):
                row = seq_len - n_tok + t
                assert oracle.visible_length(seq_len, n_tok, t) == int(mask[row].sum())
    assert oracle.visible_length(37, 1, 0) == 37


# ----------------------------------------------------------------------------- KV write

def _random_write_case(rng, dtype, n_blocks=24, hkv=3, b=4, d=8, n_seq=3, n_tok=2):
    lengths = rng.integers(n_tok, 4 * b, size=n_seq)
    perm = rng.permutation(n_blocks)
    tables = np.full((n_seq, 4), 2**31 - 1, dtype=np.int32)
    cursor = 0
    for i, length in enumerate(lengths):
        nb = -(-int(length) // b)
        tables[i, :nb] = perm[cursor:cursor + nb]
        cursor += nb
    positions = np.stack([np.arange(L - n_tok, L) for L in lengths]).astype(np.int32)
    pool = torch.randn(2, n_blocks, hkv, b, d, dtype=torch.float32).to(dtype)
    new = torch.randn(2, n_seq, n_tok, hkv, d, dtype=torch.float32).to(dtype)
    # NaNs with distinct payloads must survive the copy bit for bit
    if dtype == torch.float32:
        nv = new.view(torch.int32)
        nv[0, 0, 0, 0, 0] = 0x7FC00123
        nv[1, -1, -1, -1, -1] = 0x7FA00042
    return pool, new, tables, positions


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_write_kv_matches_torch_index_put(dtype):
    """The oracle scatter equals torch's advanced-index assignment that [P1] 'The paged cache'
    (update) uses, bit for bit, and leaves every other slot untouched."""
    rng = np.random.default_rng(3)
    pool, new, tables, positions = _random_write_case(rng, dtype)
    b = pool.shape[3]
    kp, vp = oracle.write_kv(bits(pool[0]), bits(pool[1]), bits(new[0]), bits(new[1]),
                             tables, positions, b)
    tab = torch.from_numpy(tables.astype(np.int64))
    pos = torch.from_numpy(positions.astype(np.int64))
    blocks = tab[torch.arange(tab.shape[0])[:, None], pos // b]
    offsets = pos % b
    ref = pool.clone()
    ref[0][blocks, :, offsets] = new[0]
    ref[1][blocks, :, offsets] = new[1]
    assert np.array_equal(kp, bits(ref[0]))
    assert np.array_equal(vp, bits(ref[1]))
    # untouched slots: compare against the input pools with the written slots masked out
    touched = np.zeros(pool.shape[1:4], dtype=bool)
    touched[blocks.numpy(), :, offsets.numpy()] = True
    assert np.array_equal(kp[~touched], bits(pool[0])[~touched])
    assert touched.sum() == positions.size * pool.shape[2]


def test_write_kv_does_not_modify_inputs():
    rng = np.random.default_rng(5)
    pool, new, tables, positions = _random_write_case(rng, torch.float32)
    k_before = bits(pool[0]).copy()
    oracle.write_kv(bits(pool[0]), bits(pool[1]), bits(new[0]), bits(new[1]), tables, positions, 4)
    assert np.array_equal(bits(pool[0]), k_before)


# ----------------------------------------------------------------------------- attention

def _history_case(rng, *, lengths, hq, hkv, d, b, n_tok=1, n_blocks=None, dtype=np.float64):
    """Contiguous per-sequence K/V histories, placed into a shuffled pool block by block:
    logical block j of a sequence holds its tokens j*b .. j*b + b - 1 ([P5] section 3.2 step 1)."""
    need = [-(-L // b) for L in lengths]
    n_blocks = n_blocks or sum(need) + 3
    perm = rng.permutation(n_blocks)
    k_pool = rng.standard_normal((n_blocks, hkv, b, d)).astype(dtype)
    v_pool = rng.standard_normal((n_blocks, hkv, b, d)).astype(dtype)
    tables = np.full((len(lengths), max(need)), 2**31 - 1, dtype=np.int64)
    hist_k, hist_v = [], []
    cursor = 0
    for i, L in enumerate(lengths):
        hk = rng.standard_normal((L, hkv, d)).astype(dtype)
        hv = rng.standard_normal((L, hkv, d)).astype(dtype)
        for j in range(need[i]):
            phys = int(perm[cursor])
            cursor += 1
            tables[i, j] = phys
            chunk = slice(j * b, min(L, (j + 1) * b))
            n = chunk.stop - chunk.start
            k_pool[phys, :, :n] = hk[chunk].transpose(1, 0, 2)
            v_pool[phys, :, :n] = hv[chunk].transpose(1, 0, 2)
            k_pool[phys, :, n:] = np.nan      # slots past L: never read
            v_pool[phys, :, n:] = np.nan
        hist_k.append(hk)
        hist_v.append(hv)
    q = rng.standard_normal((len(lengths), n_tok, hq, d)).astype(dtype)
    return q, k_pool, v_pool, tables, np.array(lengths), hist_k, hist_v


def _sdpa_reference(q, hist_k, hist_v, scale, rng):
    """torch SDPA in float64 over the contiguous histories. For T > 1 the queries are the last T
    rows of a full-length causal self-attention (is_causal=True), so the mask comes from torch."""
    n_seq, n_tok, hq, d = q.shape
    out = np.zeros_like(q, dtype=np.float64)
    for i in range(n_seq):
        L = hist_k[i].shape[0]
        k = torch.from_numpy(hist_k[i]).permute(1, 0, 2)[None].to(torch.float64)
        v = torch.from_numpy(hist_v[i]).permute(1, 0, 2)[None].to(torch.float64)
        if n_tok == 1:
            qq = torch.from_numpy(q[i]).permute(1, 0, 2)[None].to(torch.float64)
            o = F.scaled_dot_product_attention(qq, k, v, scale=scale, enable_gqa=True)
            out[i] = o[0].permute(1, 0, 2).numpy()
        else:
            q_full = rng.standard_normal((L, hq, d))
            q_full[L - n_tok:] = q[i]
            qq = torch.from_numpy(q_full).permute(1, 0, 2)[None]
            o = F.scaled_dot_product_attention(qq, k, v, scale=scale, is_causal=True, enable_gqa=True)
            out[i] = o[0].permute(1, 0, 2).numpy()[L - n_tok:]
    return out


@pytest.mark.parametrize("b,hq,hkv,d,n_tok,lengths", [
    (16, 4, 2, 8, 1, [40]),                      # [P2] task 09.2: L = 40, GQA 4/2, d = 8
    (16, 4, 2, 64, 1, [1, 17, 33, 64]),          # the tiny workload's shape
    (4, 4, 2, 64, 1, [10, 3, 4, 5]),
    (16, 8, 8, 16, 1, [15, 16, 17, 31, 32, 33]), # tail boundaries b-1, b, b+1 in one batch
    (8, 6, 2, 16, 2, [9, 2, 23]),
    (16, 16, 2, 32, 4, [4, 19, 64, 70]),         # speculative: 4 causal tokens, GQA 8:1
    (32, 3, 1, 8, 3, [3, 100]),
])
def test_decode_matches_library_attention(b, hq, hkv, d, n_tok, lengths):
    rng = np.random.default_rng(sum(lengths) + b)
    q, kp, vp, tables, lens, hk, hv = _history_case(rng, lengths=lengths, hq=hq, hkv=hkv, d=d, b=b, n_tok=n_tok)
    scale = 1.0 / math.sqrt(d)
    got = oracle.decode(q, kp, vp, tables, lens, scale, b)
    ref = _sdpa_reference(q, hk, hv, scale, rng)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)
    assert np.isfinite(got).all()
    # and the pages' own bar for task 09.2 (atol 1e-5)
    assert np.abs(got - ref).max() < 1e-5


def test_decode_row_equals_decode():
    rng = np.random.default_rng(11)
    q, kp, vp, tables, lens, _, _ = _history_case(rng, lengths=[7, 30], hq=4, hkv=2, d=8, b=4, n_tok=2)
    full = oracle.decode(q, kp, vp, tables, lens, 0.25, 4)
    for i in range(2):
        for t in range(2):
            for h in range(4):
                row = oracle.decode_row(q, kp, vp, tables, lens, 0.25, 4, i, t, h)
                np.testing.assert_allclose(row, full[i, t, h], rtol=0, atol=1e-14)


def test_permuting_physical_blocks_changes_nothing():
    """Relabelling physical blocks (pool rows and table entries together) leaves every output
    bit-identical: physical ids never enter the arithmetic ([P1]: kernel checked with scrambled tables)."""
    rng = np.random.default_rng(21)
    q, kp, vp, tables, lens, _, _ = _history_case(rng, lengths=[5, 33, 48], hq=4, hkv=2, d=16, b=16)
    base = oracle.decode(q, kp, vp, tables, lens, 0.3, 16)
    perm = rng.permutation(kp.shape[0])           # new id of old block x is perm[x]
    kp2 = np.empty_like(kp)
    vp2 = np.empty_like(vp)
    kp2[perm] = kp
    vp2[perm] = vp
    tables2 = tables.copy()
    valid = tables < kp.shape[0]
    tables2[valid] = perm[tables[valid]]
    again = oracle.decode(q, kp2, vp2, tables2, lens, 0.3, 16)
    assert np.array_equal(base, again)


def test_single_position_returns_v0_exactly():
    """With L = 1 the softmax of a single score is exactly 1, so o = v_0 bit for bit."""
    rng = np.random.default_rng(2)
    q, kp, vp, tables, lens, hk, hv = _history_case(rng, lengths=[1, 1], hq=4, hkv=2, d=8, b=16)
    out = oracle.decode(q, kp, vp, tables, lens, 0.35, 16)
    for i in range(2):
        for h in range(4):
            assert np.array_equal(out[i, 0, h], hv[i][0, h // 2])


def test_zero_query_averages_visible_values():
    """q = 0 gives equal weights, so o is the mean of the visible V rows (closed form),
    including the causal cut for T > 1."""
    rng = np.random.default_rng(4)
    q, kp, vp, tables, lens, hk, hv = _history_case(rng, lengths=[9, 26], hq=4, hkv=2, d=8, b=8, n_tok=3)
    q[:] = 0.0
    out = oracle.decode(q, kp, vp, tables, lens, 0.125, 8)
    for i, L in enumerate([9, 26]):
        for t in range(3):
            n = L - 3 + t + 1
            for h in range(4):
                np.testing.assert_allclose(out[i, t, h], hv[i][:n, h // 2].mean(axis=0), rtol=0, atol=1e-14)


def test_huge_scale_selects_the_best_key():
    """As scale grows the softmax becomes one-hot on the highest-scoring position, so o equals
    that position's V row (the other weights underflow to exactly 0)."""
    rng = np.random.default_rng(8)
    q, kp, vp, tables, lens, hk, hv = _history_case(rng, lengths=[37], hq=2, hkv=1, d=8, b=16)
    out = oracle.decode(q, kp, vp, tables, lens, 1e6, 16)
    for h in range(2):
        best = int(np.argmax(hk[0][:, 0] @ q[0, 0, h]))
        assert np.array_equal(out[0, 0, h], hv[0][best, 0])


def test_padding_entries_are_never_read():
    """Table entries past ceil(L/b) hold INT32_MAX; the oracle never dereferences them."""
    rng = np.random.default_rng(9)
    q, kp, vp, tables, lens, _, _ = _history_case(rng, lengths=[3, 64], hq=2, hkv=1, d=8, b=16)
    assert tables[0, 1] == 2**31 - 1
    out = oracle.decode(q, kp, vp, tables, lens, 0.3, 16)
    assert np.isfinite(out).all()


def test_generated_workloads_respect_block_arithmetic():
    """Every generated table row has exactly ceil(L/b) blocks; the tail waste is < b; the pool
    never hands one physical block to two sequences outside the shared prefix."""
    from workloads import make_case

    for name in ("tiny", "tiny_b4", "batch64"):
        case = make_case(name)
        seen = set()
        for i, row in enumerate(case.table_rows):
            L = int(case.seq_lens[i])
            assert len(row) == oracle.blocks_needed(L, case.block_size)
            assert 0 <= oracle.tail_waste(L, case.block_size) < case.block_size
            assert not (set(row) & seen)
            seen |= set(row)
            assert (case.block_tables[i, len(row):] == 2**31 - 1).all()
    tb4 = make_case("tiny_b4")
    assert oracle.physical_slot(tb4.table_rows[0], int(tb4.positions[0, 0]), 4) == (7, 1)


# ----------------------------------------------------------------------------- planted mistakes

def _pin_suite(mod):
    """Run the main pins against oracle module ``mod``; return the names of pins that fail."""
    failed = []
    for ex in _golden()["slots"]:
        b, table = ex["b"], ex["table"]
        n_blocks = max(table) + 1
        pool = np.zeros((n_blocks, 1, b, 2))
        pool[:, :, :, 0] = np.arange(n_blocks)[:, None, None]
        pool[:, :, :, 1] = np.arange(b)[None, None, :]
        if tuple(mod.gather_positions(pool, table, [ex["pos"]], 0, b)[0].astype(int)) != tuple(ex["expect"]):
            failed.append("golden-gather")
            break
    for b, hq, hkv, d, n_tok, lengths in [(4, 4, 2, 8, 1, [10, 3]), (8, 6, 2, 8, 3, [9, 23])]:
        rng = np.random.default_rng(1)
        q, kp, vp, tables, lens, hk, hv = _history_case(rng, lengths=lengths, hq=hq, hkv=hkv, d=d, b=b, n_tok=n_tok)
        try:
            got = mod.decode(q, kp, vp, tables, lens, 0.3, b)
            ref = _sdpa_reference(q, hk, hv, 0.3, rng)
            if not np.allclose(got, ref, rtol=0, atol=1e-12):
                failed.append(f"sdpa-T{n_tok}")
        except Exception:  # a broken oracle may also crash
            failed.append(f"sdpa-T{n_tok}-crash")
    return failed


def test_planted_mistakes_are_caught(monkeypatch):
    import importlib
    import types

    assert _pin_suite(pa_oracle) == []

    def fresh():
        src = importlib.util.find_spec("oracle.pa_oracle")
        mod = importlib.util.module_from_spec(src)
        src.loader.exec_module(mod)
        return mod

    mutants = {}

    m = fresh()  # offset and block swapped in the gather
    def bad_gather(pool, table_row, positions, kv_head, block_size):
        positions = np.asarray(positions)
        return np.asarray(pool[np.asarray(table_row)[positions % block_size % len(table_row)], kv_head,
                               positions // block_size % pool.shape[2]], dtype=np.float64)
    m.gather_positions = bad_gather
    mutants["gather-swapped"] = m

    m = fresh()  # causal limit off by one
    m.visible_length = lambda L, T, t: L - T + t
    mutants["causal-off-by-one"] = m

    m = fresh()  # scale dropped
    orig = m.attend_rows
    m.attend_rows = lambda q, k, v, scale: orig(q, k, v, 1.0)
    mutants["scale-dropped"] = m

    m = fresh()  # GQA mapping h % Hkv instead of h // G
    def bad_decode(q, k_pool, v_pool, block_tables, seq_lens, scale, block_size):
        n_seq, n_tok, hq, dim = q.shape
        hkv = k_pool.shape[1]
        out = np.zeros(q.shape)
        for i in range(n_seq):
            for h in range(hq):
                for t in range(n_tok):
                    n = m.visible_length(int(seq_lens[i]), n_tok, t)
                    pos = np.arange(n)
                    k = m.gather_positions(k_pool, block_tables[i], pos, h % hkv, block_size)
                    v = m.gather_positions(v_pool, block_tables[i], pos, h % hkv, block_size)
                    out[i, t, h] = m.attend_rows(q[i, t, h][None], k, v, scale)[0]
        return out
    m.decode = bad_decode
    mutants["gqa-modulo"] = m

    m = fresh()  # values weighted but not normalised
    def unnormalised(q, k, v, scale):
        s = scale * (np.asarray(q, np.float64) @ np.asarray(k, np.float64).T)
        return np.exp(s - s.max(axis=1, keepdims=True)) @ np.asarray(v, np.float64)
    m.attend_rows = unnormalised
    mutants["no-normalise"] = m

    for name, mod in mutants.items():
        assert isinstance(mod, types.ModuleType)
        assert _pin_suite(mod), f"planted mistake '{name}' was not caught by the pins"
