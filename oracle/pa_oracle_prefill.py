"""Float64 CPU oracle for paged prefill: a chunk of new query tokens per sequence.

TEST INFRASTRUCTURE ONLY (see the package docstring): no product code imports it.

What is computed. [P1] "25. Paged attention and prefix caching", stretch
exercise 4, defines the paged prefill kernel: a block of query tokens of one
sequence attends, causally, to that sequence's paged history and to the new
tokens themselves. [P4] "Prefill vs decode under paging" describes the phase:
many tokens are written left to right into the sequence's blocks, and
attention runs over those blocks. [P5] §4.1 fixes the mask: the query at
position i keeps position p only if p <= i.

Layout (variable chunk lengths, packed): sequence i owns query rows
``q_start[i] .. q_start[i+1] - 1`` of ``q [Q, Hq, D]``, with
``n_i = q_start[i+1] - q_start[i]`` new tokens. ``seq_lens[i] = L_i`` counts
the history and the chunk, so the chunk occupies positions ``L_i - n_i ..
L_i - 1`` and its token j sits at position ``L_i - n_i + j``.

Readings taken where the pages leave a step open:

* The chunk is the sequence's newest n_i positions, as the T new tokens of a
  decode step are. Its K/V rows are in the pools before attention runs: the
  chunk is written first (``write_kv_varlen``), then attended, the order [P4]
  gives for decode.
* n_i = 0 is allowed (that sequence has no query rows); n_i <= L_i.
* Query head h reads kv head h // G, as in decode ([P1] "Attention that reads
  through the table").

The attention itself is the decode oracle's: K/V gathered position by
position through the table, then the two-pass softmax of ``attend_rows``.
"""

from __future__ import annotations

import numpy as np

from .pa_oracle import _UINT_OF_SIZE, attend_rows, gather_positions, physical_slot

__all__ = ["chunk_positions", "write_kv_varlen", "prefill", "prefill_row"]


def chunk_positions(seq_lens, q_start):
    """Position of every packed query row: ``L_i - n_i + j`` for row ``q_start[i] + j``.

    Returns ``(seq_of_row, pos_of_row)``, int64 arrays of length ``q_start[-1]``.
    """
    q_start = np.asarray(q_start, dtype=np.int64)
    seq_lens = np.asarray(seq_lens, dtype=np.int64)
    total = int(q_start[-1])
    seq = np.empty(total, dtype=np.int64)
    pos = np.empty(total, dtype=np.int64)
    for i in range(len(seq_lens)):
        lo, hi = int(q_start[i]), int(q_start[i + 1])
        n = hi - lo
        if n < 0 or n > int(seq_lens[i]):
            raise ValueError(f"sequence {i}: chunk of {n} tokens with length {int(seq_lens[i])}")
        seq[lo:hi] = i
        pos[lo:hi] = int(seq_lens[i]) - n + np.arange(n)
    return seq, pos


def write_kv_varlen(k_pool, v_pool, k_new, v_new, block_tables, seq_lens, q_start, block_size):
    """Scatter of a prefill chunk's K/V rows; returns new pools, inputs unchanged.

    Row r of ``k_new``/``v_new`` (``[Q, Hkv, D]``), which belongs to sequence i
    at position ``p = L_i - n_i + (r - q_start[i])``, is copied bit for bit, for
    every kv head, to ``pool[table[i][p // b], :, p % b, :]``: the slot rule of
    [P1] "Paging", applied to each new token as in [P1] "The paged cache"
    (``update``) and [P4] "Prefill vs decode under paging".
    """
    if k_pool.dtype != k_new.dtype or v_pool.dtype != v_new.dtype:
        raise TypeError("pool and new rows must share a dtype")
    utype = _UINT_OF_SIZE[k_pool.dtype.itemsize]
    kp = np.array(k_pool, copy=True).view(utype)
    vp = np.array(v_pool, copy=True).view(utype)
    kn = np.ascontiguousarray(k_new).view(utype)
    vn = np.ascontiguousarray(v_new).view(utype)
    seq, pos = chunk_positions(seq_lens, q_start)
    for r in range(len(seq)):
        phys, off = physical_slot(block_tables[int(seq[r])], int(pos[r]), block_size)
        kp[phys, :, off, :] = kn[r]
        vp[phys, :, off, :] = vn[r]
    return kp.view(k_pool.dtype), vp.view(v_pool.dtype)


def prefill(q, k_pool, v_pool, block_tables, seq_lens, q_start, scale, block_size):
    """Causal paged attention of every packed query row; float64 ``[Q, Hq, D]``.

    Row ``q_start[i] + j``, head h, attends to positions ``0 .. L_i - n_i + j``
    of sequence i, kv head ``h // G``, each gathered through the block table.
    """
    q = np.asarray(q)
    total, hq, dim = q.shape
    hkv = k_pool.shape[1]
    if hq % hkv:
        raise ValueError("num_q_heads must be a multiple of num_kv_heads")
    group = hq // hkv
    seq, pos = chunk_positions(seq_lens, q_start)
    if len(seq) != total:
        raise ValueError("q_start[-1] must equal the number of query rows")
    out = np.zeros((total, hq, dim), dtype=np.float64)
    for i in range(len(seq_lens)):
        lo, hi = int(q_start[i]), int(q_start[i + 1])
        if hi == lo:
            continue
        every_pos = np.arange(int(seq_lens[i]))
        for kvh in range(hkv):
            keys = gather_positions(k_pool, block_tables[i], every_pos, kvh, block_size)
            values = gather_positions(v_pool, block_tables[i], every_pos, kvh, block_size)
            heads = np.arange(kvh * group, (kvh + 1) * group)
            for r in range(lo, hi):
                n = int(pos[r]) + 1
                out[r, heads] = attend_rows(q[r, heads], keys[:n], values[:n], scale)
    return out


def prefill_row(q, k_pool, v_pool, block_tables, seq_lens, q_start, scale, block_size, r, h):
    """One output row ``o[r, h, :]`` of :func:`prefill`, for sampled checks at full size."""
    q_start = np.asarray(q_start, dtype=np.int64)
    i = int(np.searchsorted(q_start, r, side="right")) - 1
    n_i = int(q_start[i + 1] - q_start[i])
    p = int(seq_lens[i]) - n_i + (r - int(q_start[i]))
    group = q.shape[1] // k_pool.shape[1]
    every = np.arange(p + 1)
    keys = gather_positions(k_pool, block_tables[i], every, h // group, block_size)
    values = gather_positions(v_pool, block_tables[i], every, h // group, block_size)
    return attend_rows(np.asarray(q[r, h])[None, :], keys, values, scale)[0]
