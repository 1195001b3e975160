"""Float64 CPU oracle: the paged-KV decode step written out from its definition.

TEST INFRASTRUCTURE ONLY (see the package docstring): no product code imports it.

Notation: B sequences, T query tokens per sequence (the T newest positions), Hq
query heads, Hkv kv heads, G = Hq / Hkv, D head_dim, b block size, N pool blocks,
MB block-table width. Pools are ``[N, Hkv, b, D]``, as in [P1] "Paging". Block
tables are ``[B, MB]`` integers, and only entries ``j < ceil(L_i / b)`` of row i
are meaningful. ``seq_lens[i] = L_i`` counts every position of sequence i,
including the T just written.

What this computes, and why it is a plain definition rather than the method:
[P5] §4.2 and [P4] "KV cache in Transformers (reminder)" both state that
blockwise online-softmax attention through the block table equals ordinary
softmax attention over the sequence's K/V in logical order. So the oracle
gathers K and V position by position through the table and applies the
two-pass, numerically stable softmax. It does not use the online recurrence,
blocks or partitions, so it shares no structure with the kernels it checks.
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "physical_slot",
    "blocks_needed",
    "tail_waste",
    "visible_length",
    "write_kv",
    "gather_positions",
    "attend_rows",
    "decode",
    "decode_row",
]

_UINT_OF_SIZE = {1: np.uint8, 2: np.uint16, 4: np.uint32, 8: np.uint64}


def physical_slot(table_row, pos: int, block_size: int) -> tuple[int, int]:
    """Where logical position ``pos`` lives: (physical block, offset in block).

    [P1] "Paging": position p sits in physical block ``table[p // b]`` at offset
    ``p % b``. [P5] §3.1-3.2 (token -> logical block number by division, then
    the Block Table, then the slot) and [P4] "Paged KV layouts (kernel writer
    view)" say the same.
    """
    if pos < 0:
        raise ValueError(f"negative position {pos}")
    return int(table_row[pos // block_size]), int(pos % block_size)


def blocks_needed(length: int, block_size: int) -> int:
    """Blocks a sequence of ``length`` tokens occupies: ceil(L / b).

    [P1] "The paged cache" (blocks_needed); [P2] §2, where a length-L
    sequence takes ceil(L/16) blocks.
    """
    return -(-int(length) // int(block_size))


def tail_waste(length: int, block_size: int) -> int:
    """Unused slots in a sequence's last block: b * ceil(L / b) - L.

    [P2] §2 bounds this residual loss below one block. [P1] "Paging" puts it
    at no more than b - 1 slots.
    """
    return int(block_size) * blocks_needed(length, block_size) - int(length)


def visible_length(seq_len: int, q_tokens: int, t: int) -> int:
    """How many positions query token ``t`` (0 <= t < T) attends to.

    [P5] §4.1: the causally masked score keeps position p for query position i
    only if p <= i. The T query tokens of a decode step are the sequence's T
    newest positions ([P4] "KV cache in Transformers (reminder)": decode
    appends the new (k, v) and attends with q_t, or a small speculative set of
    them). So token t sits at i = L - T + t and sees positions 0 .. L - T + t,
    which is L - T + t + 1 of them. For T = 1 that is all L positions.
    """
    return int(seq_len) - int(q_tokens) + int(t) + 1


def write_kv(k_pool, v_pool, k_new, v_new, block_tables, positions, block_size):
    """KV-append scatter; returns new pools and leaves the inputs unchanged.

    For every sequence i and new token t, with ``pos = positions[i, t]``, the
    rows ``k_new[i, t, h, :]`` and ``v_new[i, t, h, :]`` are copied, for every
    kv head h, to ``pool[table[i][pos // b], h, pos % b, :]``. This is the scatter
    half of ``update`` in [P1] "The paged cache", ``Sequence.append`` in [P2]
    (without its copy-on-write), and the step of the decode-step sketch in [P4]
    "Block table and allocator" that stores the new token's K and V at the fill
    offset of the sequence's last block.

    The copy is done on unsigned-integer views of the arrays, so every bit is
    kept, NaN payloads included. For bf16, pass the raw uint16 bits.
    Shapes: pools ``[N, Hkv, b, D]``, new rows ``[B, T, Hkv, D]``,
    ``block_tables [B, MB]``, ``positions [B, T]``.
    """
    if k_pool.dtype != k_new.dtype or v_pool.dtype != v_new.dtype:
        raise TypeError("pool and new rows must share a dtype")
    utype = _UINT_OF_SIZE[k_pool.dtype.itemsize]
    kp = np.array(k_pool, copy=True).view(utype)
    vp = np.array(v_pool, copy=True).view(utype)
    kn = np.ascontiguousarray(k_new).view(utype)
    vn = np.ascontiguousarray(v_new).view(utype)
    n_seq, n_tok = positions.shape
    for i in range(n_seq):
        for t in range(n_tok):
            phys, off = physical_slot(block_tables[i], int(positions[i, t]), block_size)
            kp[phys, :, off, :] = kn[i, t]
            vp[phys, :, off, :] = vn[i, t]
    return kp.view(k_pool.dtype), vp.view(v_pool.dtype)


def gather_positions(pool, table_row, positions, kv_head: int, block_size: int):
    """Rows ``pool[table[p // b], kv_head, p % b, :]`` for each p in ``positions``.

    This is the explicit per-position gather: ``gather_kv`` in [P2] and the
    gather half of ``update`` in [P1] "The paged cache". The result is float64
    with shape ``[len(positions), D]``.
    """
    positions = np.asarray(positions, dtype=np.int64)
    table_row = np.asarray(table_row, dtype=np.int64)
    blocks = table_row[positions // block_size]
    offsets = positions % block_size
    return np.asarray(pool[blocks, kv_head, offsets, :], dtype=np.float64)


def attend_rows(q_rows, keys, values, scale: float):
    """Softmax attention of each query row over the same keys and values, in float64.

    ``s[r, p] = scale * q[r] . k[p]``; ``o[r] = sum_p softmax_p(s[r]) v[p]``
    ([P2] §5: scores are q.K scaled by one over root head_dim, the output is their softmax
    applied to V; [P4] "KV cache in Transformers (reminder)"; [P5] §4.2: the output row is the
    softmax-weighted sum of the value rows).

    Softmax is done in the usual two passes ([P5] §4.2): subtract the row
    maximum, exponentiate, normalise. Shapes: ``q_rows [R, D]``,
    ``keys``/``values [P, D]``, result ``[R, D]``.
    """
    q = np.asarray(q_rows, dtype=np.float64)
    k = np.asarray(keys, dtype=np.float64)
    v = np.asarray(values, dtype=np.float64)
    if k.shape[0] == 0:
        raise ValueError("attention over zero positions is undefined")
    s = float(scale) * (q @ k.T)                      # [R, P]
    m = s.max(axis=1, keepdims=True)
    w = np.exp(s - m)
    return (w @ v) / w.sum(axis=1, keepdims=True)


def decode(q, k_pool, v_pool, block_tables, seq_lens, scale, block_size):
    """Paged decode attention for every (sequence, query token, query head).

    ``q`` is ``[B, T, Hq, D]`` and the result is float64 of the same shape. Query
    head h reads kv head ``h // G`` with ``G = Hq // Hkv`` ([P1] "Attention that
    reads through the table": query head h reads KV head h // group). Token t
    of sequence i attends to positions ``0 .. visible_length(L_i, T, t) - 1``,
    each gathered through the block table.
    """
    n_seq, n_tok, hq, dim = q.shape
    hkv = k_pool.shape[1]
    if hq % hkv:
        raise ValueError("num_q_heads must be a multiple of num_kv_heads")
    group = hq // hkv
    out = np.zeros((n_seq, n_tok, hq, dim), dtype=np.float64)
    for i in range(n_seq):
        seq_len = int(seq_lens[i])
        if visible_length(seq_len, n_tok, 0) < 1:
            raise ValueError(f"sequence {i}: length {seq_len} < {n_tok} query tokens")
        every_pos = np.arange(seq_len)
        for kvh in range(hkv):
            keys = gather_positions(k_pool, block_tables[i], every_pos, kvh, block_size)
            values = gather_positions(v_pool, block_tables[i], every_pos, kvh, block_size)
            heads = np.arange(kvh * group, (kvh + 1) * group)
            for t in range(n_tok):
                n = visible_length(seq_len, n_tok, t)
                out[i, t, heads] = attend_rows(q[i, t, heads], keys[:n], values[:n], scale)
    return out


def decode_row(q, k_pool, v_pool, block_tables, seq_lens, scale, block_size, i, t, h):
    """One output row ``o[i, t, h, :]`` of :func:`decode`, for sampled checks at full size."""
    n_tok, hq = q.shape[1], q.shape[2]
    group = hq // k_pool.shape[1]
    n = visible_length(int(seq_lens[i]), n_tok, t)
    if n < 1:
        raise ValueError("no visible positions")
    pos = np.arange(n)
    keys = gather_positions(k_pool, block_tables[i], pos, h // group, block_size)
    values = gather_positions(v_pool, block_tables[i], pos, h // group, block_size)
    return attend_rows(np.asarray(q[i, t, h])[None, :], keys, values, scale)[0]
