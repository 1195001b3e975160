"""Pins of the paged-prefill oracle (oracle/pa_oracle_prefill.py) against what the pages and the
mathematics fix: torch's float64 causal scaled_dot_product_attention on the contiguous histories
(a library routine, with the mask from torch's is_causal), torch's index_put for the scatter,
closed forms, and invariants. ``test_planted_mistakes_are_caught`` plants mistakes in copies of the
oracle and checks that these pins catch each one."""

from __future__ import annotations

import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from oracle import pa_oracle_prefill

P = pa_oracle_prefill


def _case(rng, *, lengths, chunks, hq, hkv, d, b, extra_blocks=3):
    """Contiguous histories of the given lengths placed block by block into a shuffled pool (slots
    past a length hold NaN), plus packed chunk queries: sequence i's last ``chunks[i]`` positions."""
    need = [-(-L // b) for L in lengths]
    n_blocks = sum(need) + extra_blocks
    perm = rng.permutation(n_blocks)
    k_pool = rng.standard_normal((n_blocks, hkv, b, d))
    v_pool = rng.standard_normal((n_blocks, hkv, b, d))
    tables = np.full((len(lengths), max(need)), 2**31 - 1, dtype=np.int64)
    hist_k, hist_v = [], []
    cursor = 0
    for i, L in enumerate(lengths):
        hk = rng.standard_normal((L, hkv, d))
        hv = rng.standard_normal((L, hkv, d))
        for j in range(need[i]):
            phys = int(perm[cursor])
            cursor += 1
            tables[i, j] = phys
            n = min(L, (j + 1) * b) - j * b
            k_pool[phys, :, :n] = hk[j * b:j * b + n].transpose(1, 0, 2)
            v_pool[phys, :, :n] = hv[j * b:j * b + n].transpose(1, 0, 2)
            k_pool[phys, :, n:] = np.nan
            v_pool[phys, :, n:] = np.nan
        hist_k.append(hk)
        hist_v.append(hv)
    q_start = np.concatenate([[0], np.cumsum(chunks)]).astype(np.int64)
    q = rng.standard_normal((int(q_start[-1]), hq, d))
    return q, k_pool, v_pool, tables, np.array(lengths), q_start, hist_k, hist_v


def _sdpa_causal(q, q_start, hist_k, hist_v, scale, rng):
    """Each chunk's queries are the last n rows of a full causal self-attention over the sequence's
    L positions (torch's is_causal mask); the other query rows are random fillers."""
    out = np.zeros(q.shape)
    for i in range(len(hist_k)):
        lo, hi = int(q_start[i]), int(q_start[i + 1])
        if hi == lo:
            continue
        L, hq, d = hist_k[i].shape[0], q.shape[1], q.shape[2]
        q_full = rng.standard_normal((L, hq, d))
        q_full[L - (hi - lo):] = q[lo:hi]
        qq = torch.from_numpy(q_full).permute(1, 0, 2)[None]
        k = torch.from_numpy(hist_k[i]).permute(1, 0, 2)[None]
        v = torch.from_numpy(hist_v[i]).permute(1, 0, 2)[None]
        o = F.scaled_dot_product_attention(qq, k, v, scale=scale, is_causal=True, enable_gqa=True)
        out[lo:hi] = o[0].permute(1, 0, 2).numpy()[L - (hi - lo):]
    return out


CASES = [
    # b, hq, hkv, d, lengths, chunks
    (16, 4, 2, 8, [40, 17, 5], [8, 17, 1]),          # history + chunk; whole sequence; one token
    (4, 8, 2, 16, [10, 3, 33, 20], [10, 0, 5, 13]),  # b = 4 (the [P1] block size), an empty chunk
    (16, 6, 2, 16, [64, 65, 31], [32, 33, 31]),      # chunk edges at 31 / 32 / 33 tokens, GQA 3:1
    (32, 8, 8, 8, [100, 1], [40, 1]),                # MHA (G = 1), a one-position sequence
]


@pytest.mark.parametrize("b,hq,hkv,d,lengths,chunks", CASES)
def test_prefill_matches_library_causal_attention(b, hq, hkv, d, lengths, chunks):
    rng = np.random.default_rng(sum(lengths) + b)
    q, kp, vp, tables, lens, qs, hk, hv = _case(rng, lengths=lengths, chunks=chunks, hq=hq, hkv=hkv, d=d, b=b)
    scale = 1.0 / math.sqrt(d)
    got = P.prefill(q, kp, vp, tables, lens, qs, scale, b)
    ref = _sdpa_causal(q, qs, hk, hv, scale, rng)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)
    assert np.isfinite(got).all()


def test_prefill_without_history_is_causal_self_attention():
    """L_i = n_i: the chunk is the whole sequence, and the result is textbook causal attention of
    the chunk over itself (torch's is_causal on the chunk alone)."""
    rng = np.random.default_rng(3)
    lengths = [23, 16, 1]
    q, kp, vp, tables, lens, qs, hk, hv = _case(rng, lengths=lengths, chunks=lengths, hq=4, hkv=1, d=16, b=8)
    got = P.prefill(q, kp, vp, tables, lens, qs, 0.25, 8)
    for i, L in enumerate(lengths):
        lo, hi = int(qs[i]), int(qs[i + 1])
        qq = torch.from_numpy(q[lo:hi]).permute(1, 0, 2)[None]
        k = torch.from_numpy(hk[i]).permute(1, 0, 2)[None]
        v = torch.from_numpy(hv[i]).permute(1, 0, 2)[None]
        o = F.scaled_dot_product_attention(qq, k, v, scale=0.25, is_causal=True, enable_gqa=True)
        np.testing.assert_allclose(got[lo:hi], o[0].permute(1, 0, 2).numpy(), rtol=0, atol=1e-12)


def test_first_token_of_a_fresh_sequence_returns_v0_exactly():
    """With no history, token 0 sees one position: its softmax weight is exactly 1."""
    rng = np.random.default_rng(4)
    q, kp, vp, tables, lens, qs, hk, hv = _case(rng, lengths=[9, 30], chunks=[9, 30], hq=2, hkv=2, d=8, b=4)
    got = P.prefill(q, kp, vp, tables, lens, qs, 0.5, 4)
    for i in range(2):
        assert np.array_equal(got[int(qs[i])], hv[i][0])


def test_zero_queries_average_the_visible_values():
    """q = 0 gives equal weights: token j's output is the mean of V[0 .. L - n + j]."""
    rng = np.random.default_rng(5)
    q, kp, vp, tables, lens, qs, hk, hv = _case(rng, lengths=[50, 12], chunks=[20, 12], hq=4, hkv=2, d=8, b=16)
    q[:] = 0.0
    got = P.prefill(q, kp, vp, tables, lens, qs, 1.0, 16)
    for i, (L, n) in enumerate([(50, 20), (12, 12)]):
        for j in range(n):
            mean = hv[i][:L - n + j + 1].mean(axis=0)  # [Hkv, D]
            want = np.repeat(mean, 2, axis=0)           # heads 2h, 2h+1 read kv head h
            np.testing.assert_allclose(got[int(qs[i]) + j], want, rtol=0, atol=1e-12)


def test_equal_chunks_equal_decode_with_that_many_tokens():
    """With every n_i = T the packed layout is decode's [B, T, Hq, D], and the result is the decode
    oracle's (pinned on its own in test_oracle.py)."""
    rng = np.random.default_rng(6)
    q, kp, vp, tables, lens, qs, hk, hv = _case(rng, lengths=[40, 70, 9], chunks=[5, 5, 5], hq=8, hkv=2, d=8, b=16)
    got = P.prefill(q, kp, vp, tables, lens, qs, 0.3, 16)
    dec = oracle.decode(q.reshape(3, 5, 8, 8), kp, vp, tables, lens, 0.3, 16)
    np.testing.assert_array_equal(got, dec.reshape(got.shape))


def test_permuting_physical_blocks_changes_nothing():
    rng = np.random.default_rng(7)
    q, kp, vp, tables, lens, qs, hk, hv = _case(rng, lengths=[33, 18], chunks=[17, 6], hq=4, hkv=2, d=8, b=4)
    a = P.prefill(q, kp, vp, tables, lens, qs, 0.4, 4)
    perm = rng.permutation(kp.shape[0])
    kp2, vp2 = np.empty_like(kp), np.empty_like(vp)
    kp2[perm], vp2[perm] = kp, vp
    t2 = tables.copy()
    valid = t2 < kp.shape[0]
    t2[valid] = perm[t2[valid]]
    assert np.array_equal(a, P.prefill(q, kp2, vp2, t2, lens, qs, 0.4, 4))


def test_prefill_row_equals_prefill():
    rng = np.random.default_rng(8)
    q, kp, vp, tables, lens, qs, hk, hv = _case(rng, lengths=[33, 5, 18], chunks=[17, 0, 6], hq=4, hkv=2, d=8, b=4)
    full = P.prefill(q, kp, vp, tables, lens, qs, 0.4, 4)
    for r in range(q.shape[0]):
        for h in range(4):
            np.testing.assert_allclose(P.prefill_row(q, kp, vp, tables, lens, qs, 0.4, 4, r, h), full[r, h],
                                       rtol=0, atol=1e-13)


# ----------------------------------------------------------------------------- the chunk's scatter

def _write_case(rng, dtype):
    b, hkv, d = 4, 3, 8
    lengths, chunks = [10, 7, 4, 13], [6, 0, 4, 1]
    need = [-(-L // b) for L in lengths]
    n_blocks = sum(need) + 2
    perm = rng.permutation(n_blocks)
    tables = np.full((4, max(need)), 2**31 - 1, dtype=np.int64)
    c = 0
    for i, n in enumerate(need):
        tables[i, :n] = perm[c:c + n]
        c += n
    pools = [rng.standard_normal((n_blocks, hkv, b, d)).astype(dtype) for _ in range(2)]
    qs = np.concatenate([[0], np.cumsum(chunks)]).astype(np.int64)
    new = [rng.standard_normal((int(qs[-1]), hkv, d)).astype(dtype) for _ in range(2)]
    return pools, new, tables, np.array(lengths), qs, b


@pytest.mark.parametrize("dtype", [np.float32, np.float64])
def test_write_kv_varlen_matches_torch_index_put(dtype):
    rng = np.random.default_rng(11)
    (kp, vp), (kn, vn), tables, lens, qs, b = _write_case(rng, dtype)
    got_k, got_v = P.write_kv_varlen(kp, vp, kn, vn, tables, lens, qs, b)
    for pool, new, got in ((kp, kn, got_k), (vp, vn, got_v)):
        ref = torch.from_numpy(pool.copy())
        for i in range(len(lens)):
            n = int(qs[i + 1] - qs[i])
            pos = torch.arange(int(lens[i]) - n, int(lens[i]))
            blocks = torch.from_numpy(tables[i])[pos // b]
            # pool[blocks, :, offsets] is [n, Hkv, D]; the chunk rows are [n, Hkv, D] too
            ref[blocks, :, pos % b] = torch.from_numpy(new[int(qs[i]):int(qs[i + 1])])
        assert np.array_equal(got, ref.numpy())


def test_write_kv_varlen_equal_chunks_is_write_kv():
    """Equal chunks T: the packed rows are decode's [B, T, Hkv, D] new rows at positions L - T .. L - 1."""
    rng = np.random.default_rng(12)
    b, hkv, d, T = 8, 2, 4, 3
    lengths = [5, 17, 3]
    need = [-(-L // b) for L in lengths]
    n_blocks = sum(need)
    tables = np.full((3, max(need)), 2**31 - 1, dtype=np.int64)
    perm, c = rng.permutation(n_blocks), 0
    for i, n in enumerate(need):
        tables[i, :n] = perm[c:c + n]
        c += n
    kp, vp = (rng.standard_normal((n_blocks, hkv, b, d)) for _ in range(2))
    kn, vn = (rng.standard_normal((3 * T, hkv, d)) for _ in range(2))
    qs = np.arange(4) * T
    lens = np.array(lengths)
    positions = np.stack([np.arange(L - T, L) for L in lengths])
    a = P.write_kv_varlen(kp, vp, kn, vn, tables, lens, qs, b)
    w = oracle.write_kv(kp, vp, kn.reshape(3, T, hkv, d), vn.reshape(3, T, hkv, d), tables, positions, b)
    assert all(np.array_equal(x, y) for x, y in zip(a, w))


def test_chunk_positions_reject_chunks_longer_than_the_sequence():
    with pytest.raises(ValueError):
        P.chunk_positions([3, 4], [0, 4, 5])


# ----------------------------------------------------------------------------- planted mistakes

def _pin_suite(mod):
    failed = []
    for b, hq, hkv, d, lengths, chunks in CASES[:3]:
        rng = np.random.default_rng(100 + b)
        q, kp, vp, tables, lens, qs, hk, hv = _case(rng, lengths=lengths, chunks=chunks, hq=hq, hkv=hkv, d=d, b=b)
        try:
            got = mod.prefill(q, kp, vp, tables, lens, qs, 0.35, b)
            if not np.allclose(got, _sdpa_causal(q, qs, hk, hv, 0.35, rng), rtol=0, atol=1e-12):
                failed.append(f"sdpa-{b}")
        except Exception:
            failed.append(f"sdpa-{b}-crash")
    rng = np.random.default_rng(11)
    (kp, vp), (kn, vn), tables, lens, qs, b = _write_case(rng, np.float64)
    try:
        got_k, _ = mod.write_kv_varlen(kp, vp, kn, vn, tables, lens, qs, b)
        ref = torch.from_numpy(kp.copy())
        for i in range(len(lens)):
            n = int(qs[i + 1] - qs[i])
            pos = torch.arange(int(lens[i]) - n, int(lens[i]))
            ref[torch.from_numpy(tables[i])[pos // b], :, pos % b] = torch.from_numpy(kn[int(qs[i]):int(qs[i + 1])])
        if not np.array_equal(got_k, ref.numpy()):
            failed.append("write")
    except Exception:
        failed.append("write-crash")
    return failed


def test_planted_mistakes_are_caught():
    import importlib

    assert _pin_suite(P) == []

    def fresh():
        spec = importlib.util.find_spec("oracle.pa_oracle_prefill")
        mod = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(mod)
        return mod

    mutants = {}
    orig_cp = P.chunk_positions

    m = fresh()  # history ignored: the chunk's token j taken as position j
    def from_zero(seq_lens, q_start):
        seq, pos = orig_cp(seq_lens, q_start)
        qs = np.asarray(q_start)
        return seq, pos - (np.asarray(seq_lens)[seq] - (qs[seq + 1] - qs[seq]))
    m.chunk_positions = from_zero
    mutants["history-ignored"] = m

    m = fresh()  # causal limit one short (a token does not see itself)
    m.chunk_positions = lambda seq_lens, q_start: (orig_cp(seq_lens, q_start)[0], orig_cp(seq_lens, q_start)[1] - 1)
    mutants["causal-off-by-one"] = m

    m = fresh()  # rows assigned to sequences as if every chunk had the same length
    def even_split(seq_lens, q_start):
        seq, pos = orig_cp(seq_lens, q_start)
        per = max(1, len(seq) // len(seq_lens))
        s2 = np.minimum(np.arange(len(seq)) // per, len(seq_lens) - 1)
        return s2, pos
    m.chunk_positions = even_split
    mutants["q_start-ignored"] = m

    m = fresh()  # kv head h % Hkv instead of h // G
    def gqa_mod(q, k_pool, v_pool, block_tables, seq_lens, q_start, scale, block_size):
        hkv = k_pool.shape[1]
        seq, pos = m.chunk_positions(seq_lens, q_start)
        out = np.zeros(q.shape)
        for r in range(q.shape[0]):
            for h in range(q.shape[1]):
                every = np.arange(int(pos[r]) + 1)
                k = oracle.gather_positions(k_pool, block_tables[int(seq[r])], every, h % hkv, block_size)
                v = oracle.gather_positions(v_pool, block_tables[int(seq[r])], every, h % hkv, block_size)
                out[r, h] = oracle.attend_rows(q[r, h][None], k, v, scale)[0]
        return out
    m.prefill = gqa_mod
    mutants["gqa-modulo"] = m

    for name, mod in mutants.items():
        assert _pin_suite(mod), f"planted mistake '{name}' was not caught by the pins"
