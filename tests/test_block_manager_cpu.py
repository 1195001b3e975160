"""The native host block manager (libpa.so's pa_bm_*, through paged_kv_cache_69_amd.blocks) against
the block-manager oracle: the pages' worked examples, and seeded random workloads replayed on both
with every returned value and the whole state (free count, reference counts, tables, lengths, cache
size) compared after every operation. Host code only: runs without a GPU."""

from __future__ import annotations

import json
import os
import random

import pytest

import paged_kv_cache_69_amd as pa
from oracle import pa_oracle_blocks as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "block_examples.json")


@pytest.fixture(scope="module")
def blocks():
    if not os.path.exists(pa.LIB_PATH):
        pytest.fail("libpa.so is not built: run __graft_entry__.build() first")
    from paged_kv_cache_69_amd import blocks as B

    return B


def _golden():
    with open(GOLDEN, encoding="utf-8") as fh:
        return json.load(fh)

def test_fork_cow_example(blocks):
    ex = _golden()["fork_cow"]
    m = blocks.BlockManager(64, ex["block_size"])
    m.add_seq(0)
    assert m.reserve(0, ex["prompt_tokens"]) == []
    m.commit(0, ex["prompt_tokens"])
    used = 64 - m.num_free
    assert used == ex["parent_blocks"]
    for k in range(1, ex["forks"] + 1):
        m.fork(0, k)
    assert 64 - m.num_free - used == ex["new_blocks_after_4_forks"]
    last = m.table(0)[-1]
    for k in range(1, ex["forks"] + 1):
        copies = m.reserve(k, 1)
        assert len(copies) == 1 and copies[0][0] == last  # the shared, partly filled block is copied
        m.commit(k, ex["prompt_tokens"] + 1)
    assert 64 - m.num_free - used == ex["new_blocks_after_each_sample_writes_a_token"]
    assert m.table(0)[-1] == last and m.refcount(last) == 1

def test_prefix_cache_example(blocks):
    ex = _golden()["prefix_cache"]
    m = blocks.BlockManager(256, ex["block_size"])
    system = list(range(1000, 1000 + ex["shared_tokens"]))
    total = prefilled = 0
    for r in range(ex["requests"]):
        prompt = system + [5000 + 100 * r + j for j in range(ex["own_tokens"])]
        reused = m.attach(r, prompt)
        m.reserve(r, len(prompt) - reused)
        m.commit(r, len(prompt))
        m.remember(r, prompt)
        total += len(prompt)
        prefilled += len(prompt) - reused
    assert (total, prefilled, 256 - m.num_free) == (ex["prompt_tokens"], ex["tokens_prefilled"], ex["blocks_in_use"])

def test_task_09_3_example(blocks):
    ex = _golden()["task_09_3"]
    m = blocks.BlockManager(1024, ex["block_size"])
    m.add_seq(100)
    m.reserve(100, ex["prompt_tokens"])
    m.commit(100, ex["prompt_tokens"])
    assert len(m.table(100)) == ex["prompt_blocks"]
    for i in range(ex["forks"]):
        m.fork(100, i)
        m.reserve(i, ex["tokens_per_fork"])
        m.commit(i, ex["prompt_tokens"] + ex["tokens_per_fork"])
    assert len(set(m.table(0)) & set(m.table(1))) == ex["shared_blocks_req0_req1"]
    assert 1024 - m.num_free == ex["blocks_used"]
    m.free(100)
    assert 1024 - m.num_free == ex["used_after_base_free"]

def test_errors_change_nothing(blocks):
    m = blocks.BlockManager(3, 4)
    m.add_seq(0)
    m.reserve(0, 8)
    m.commit(0, 8)
    m.fork(0, 1)
    state = (m.table(1), m.refcounts(), m.num_free)
    with pytest.raises(blocks.PoolExhausted):
        m.reserve(1, 9)
    assert (m.table(1), m.refcounts(), m.num_free) == state
    for bad in (lambda: m.add_seq(0), lambda: m.fork(0, 1), lambda: m.free(7), lambda: m.truncate(0, 9),
                lambda: m.commit(0, 13), lambda: m.build_tables([0, 1], 1)):
        with pytest.raises(pa.PaError):
            bad()
    assert (m.table(1), m.refcounts(), m.num_free) == state

def _state(m_cpp, o):
    cpp = (m_cpp.num_free, m_cpp.refcounts(), m_cpp.num_seqs, m_cpp.num_entries,
           {s: (m_cpp.table(s), m_cpp.length(s)) for s in o.seqs})
    ref = (o.num_free, list(o.refcount), len(o.seqs), o.num_entries,
           {s: (o.table(s), o.length(s)) for s in o.seqs})
    return cpp, ref

@pytest.mark.parametrize("seed", range(8))
def test_random_workloads_match_the_oracle(blocks, seed):
    rng = random.Random(1000 + seed)
    n_blocks, b = rng.choice([(24, 2), (40, 4), (64, 3)])
    m = blocks.BlockManager(n_blocks, b)
    o = O.BlockLedger(n_blocks, b)
    next_id = 0
    for step in range(400):
        seqs = sorted(o.seqs)
        op = rng.random()
        if op < 0.25 or not seqs:
            prompt = [rng.randrange(3) for _ in range(rng.randrange(1, 4 * b))]
            s = next_id
            next_id += 1
            assert m.attach(s, prompt) == o.attach(s, prompt)
            n = len(prompt) - o.length(s)
            try:
                want = o.reserve(s, n)
            except O.PoolExhausted:
                with pytest.raises(blocks.PoolExhausted):
                    m.reserve(s, n)
                m.free(s)
                o.free(s)
            else:
                assert m.reserve(s, n) == want
                m.commit(s, len(prompt))
                o.commit(s, len(prompt))
                assert m.remember(s, prompt) == o.remember(s, prompt)
        elif op < 0.5:
            s = rng.choice(seqs)
            n = rng.randrange(0, 2 * b + 1)
            try:
                want = o.reserve(s, n)
            except O.PoolExhausted:
                with pytest.raises(blocks.PoolExhausted):
                    m.reserve(s, n)
            else:
                assert m.reserve(s, n) == want
                new_len = o.length(s) + rng.randrange(0, n + 1)
                m.commit(s, new_len)
                o.commit(s, new_len)
        elif op < 0.65:
            s = rng.choice(seqs)
            m.fork(s, next_id)
            o.fork(s, next_id)
            next_id += 1
        elif op < 0.8:
            s = rng.choice(seqs)
            m.free(s)
            o.free(s)
        elif op < 0.9:
            s = rng.choice(seqs)
            n = rng.randrange(0, o.length(s) + 1)
            m.truncate(s, n)
            o.truncate(s, n)
        else:
            want = rng.randrange(n_blocks + 1)
            assert m.evict(want) == o.evict(want)
        cpp, ref = _state(m, o)
        assert cpp == ref, f"step {step}"
    width = max([len(o.table(s)) for s in o.seqs] + [1])
    seqs = sorted(o.seqs)
    assert m.build_tables(seqs, width, pad=-7) == tuple(map(list, o.build_tables(seqs, width, -7)))


def test_zero_token_reserve_and_multi_block_copies(blocks):
    """The two copy-on-write edge cases the oracle pins: a reserve of no tokens copies nothing, and a
    write that spans two shared blocks copies both."""
    m = blocks.BlockManager(8, 4)
    m.add_seq(0)
    m.reserve(0, 6)
    m.commit(0, 6)
    m.fork(0, 1)
    assert m.reserve(1, 0) == [] and m.num_free == 6
    assert m.reserve(1, 1) == [(1, 2)] and m.num_free == 5
    m = blocks.BlockManager(8, 4)
    m.add_seq(0)
    m.reserve(0, 8)
    m.commit(0, 1)
    m.fork(0, 1)
    assert m.reserve(1, 7) == [(0, 2), (1, 3)]
    assert (m.table(0), m.table(1), m.num_free) == ([0, 1], [2, 3], 4)
