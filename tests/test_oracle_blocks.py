"""Pins of the block-manager reference model (oracle/pa_oracle_blocks.py): the worked examples the
pages print (tests/golden/block_examples.json, each with its citation), closed forms of the
allocator and of the prefix cache's rules, invariants checked after every operation of seeded random
workloads, and a data-level check that copy-on-write keeps every sequence's history intact.
``test_planted_mistakes_are_caught`` plants mistakes in copies of the model and checks that these
pins catch each one."""

from __future__ import annotations

import importlib
import json
import os
import random

import pytest

from oracle import pa_oracle_blocks

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "block_examples.json")
M = pa_oracle_blocks


def _golden():
    with open(GOLDEN, encoding="utf-8") as fh:
        return json.load(fh)


def _used(m) -> int:
    return len(m.refcount) - m.num_free


# ----------------------------------------------------------------------------- worked examples

def fork_cow_example(mod, ex):
    m = mod.BlockLedger(64, ex["block_size"])
    m.add_seq(0)
    m.reserve(0, ex["prompt_tokens"])
    m.commit(0, ex["prompt_tokens"])
    parent_blocks = _used(m)
    for k in range(1, ex["forks"] + 1):
        m.fork(0, k)
    after_forks = _used(m) - parent_blocks
    for k in range(1, ex["forks"] + 1):
        m.reserve(k, 1)
        m.commit(k, ex["prompt_tokens"] + 1)
    after_writes = _used(m) - parent_blocks
    return parent_blocks, after_forks, after_writes


def test_fork_cow_worked_example():
    ex = _golden()["fork_cow"]
    assert fork_cow_example(M, ex) == (ex["parent_blocks"], ex["new_blocks_after_4_forks"],
                                       ex["new_blocks_after_each_sample_writes_a_token"])


def prefix_cache_example(mod, ex):
    m = mod.BlockLedger(256, ex["block_size"])
    system = list(range(1000, 1000 + ex["shared_tokens"]))
    prompt_tokens = prefilled = 0
    for r in range(ex["requests"]):
        prompt = system + [5000 + 100 * r + j for j in range(ex["own_tokens"])]
        reused = m.attach(r, prompt)
        m.reserve(r, len(prompt) - reused)
        m.commit(r, len(prompt))
        m.remember(r, prompt)
        prompt_tokens += len(prompt)
        prefilled += len(prompt) - reused
    without = ex["requests"] * -(-(ex["shared_tokens"] + ex["own_tokens"]) // ex["block_size"])
    return prompt_tokens, prefilled, _used(m), without


def test_prefix_cache_worked_example():
    ex = _golden()["prefix_cache"]
    assert prefix_cache_example(M, ex) == (ex["prompt_tokens"], ex["tokens_prefilled"], ex["blocks_in_use"],
                                           ex["blocks_without_sharing"])


def task_09_3(mod, ex):
    b = ex["block_size"]
    m = mod.BlockLedger(1024, b)
    m.add_seq("base")
    m.reserve("base", ex["prompt_tokens"])
    m.commit("base", ex["prompt_tokens"])
    prompt_blocks = len(m.table("base"))
    for i in range(ex["forks"]):
        m.fork("base", f"req{i}")
        m.reserve(f"req{i}", ex["tokens_per_fork"])
        m.commit(f"req{i}", ex["prompt_tokens"] + ex["tokens_per_fork"])
    shared = len(set(m.table("req0")) & set(m.table("req1")))
    used = _used(m)
    without = ex["forks"] * -(-(ex["prompt_tokens"] + ex["tokens_per_fork"]) // b)
    block_bytes = ex["n_layers"] * ex["n_kv_heads"] * ex["head_dim"] * ex["bytes_per_value"] * 2 * b
    saved_mib = (without - used) * block_bytes // 2**20
    m.free("base")
    return prompt_blocks, shared, used, without, without - used, saved_mib, _used(m)


def test_task_09_3_worked_example():
    ex = _golden()["task_09_3"]
    assert task_09_3(M, ex) == (ex["prompt_blocks"], ex["shared_blocks_req0_req1"], ex["blocks_used"],
                                ex["blocks_without_sharing"], ex["blocks_saved"], ex["mib_saved"],
                                ex["used_after_base_free"])


# ----------------------------------------------------------------------------- closed forms

def allocator_order(mod):
    """Blocks of a 4-block pool as handed out around releases and shared holds."""
    m = mod.BlockLedger(4, 1)
    m.add_seq("a")
    m.reserve("a", 2)  # blocks 0, 1
    m.commit("a", 2)
    out = [m.table("a")]
    m.truncate("a", 1)  # block 1 becomes unused
    m.add_seq("b")
    m.reserve("b", 3)  # never-used 2, 3 come before the just-released 1
    m.commit("b", 3)
    out.append(m.table("b"))
    m.fork("b", "c")
    m.free("b")  # still held by c: nothing becomes unused
    out.append(m.num_free)
    m.free("a")
    m.free("c")  # 0 first, then c's blocks in table order
    m.add_seq("d")
    m.reserve("d", 4)
    out.append(m.table("d"))
    return out


def test_allocator_hands_out_the_longest_unused_block():
    """The block handed out next is the one unused the longest ([P1] "The allocator"): fresh blocks
    in id order, a released block after every block released before it; a held block stays out."""
    assert allocator_order(M) == [[0, 1], [2, 3, 1], 0, [0, 2, 3, 1]]


def test_over_release_and_exhaustion_raise():
    m = M.BlockLedger(2, 4)
    m.add_seq(0)
    m.reserve(0, 8)
    m.commit(0, 8)
    with pytest.raises(M.PoolExhausted):
        m.reserve(0, 1)
    m._release(0)
    with pytest.raises(RuntimeError):
        m._release(0)


def test_blocks_and_waste_closed_form():
    """A sequence of L tokens holds ceil(L / b) blocks: waste under one block ([P1] "Paging")."""
    for b in (1, 4, 16):
        for L in range(0, 70):
            m = M.BlockLedger(200, b)
            m.add_seq(0)
            m.reserve(0, L)
            m.commit(0, L)
            assert len(m.table(0)) == -(-L // b)
            assert 0 <= b * len(m.table(0)) - L < b or L == 0


def cached_prompt_reuse(mod):
    m = mod.BlockLedger(64, 16)
    prompt = list(range(96))
    m.attach(0, prompt)
    m.reserve(0, 96)
    m.commit(0, 96)
    m.remember(0, prompt)
    return m.attach(1, prompt), m.attach(2, prompt + [7])


def test_fully_cached_prompt_still_prefills_its_last_token():
    """attach leaves at least one prompt token to prefill: a cached 96-token prompt (b = 16) reuses
    80 tokens, and a 97-token one reuses all 96 cached."""
    assert cached_prompt_reuse(M) == (80, 96)


def prefix_key_case(mod):
    m = mod.BlockLedger(64, 4)
    a = [1, 2, 3, 4, 9, 9, 9, 9, 5]
    m.attach(0, a)
    m.reserve(0, len(a))
    m.commit(0, len(a))
    m.remember(0, a)
    b = [0, 2, 3, 4, 9, 9, 9, 9, 5]  # second block identical, first differs
    return m.attach(1, b), m.attach(2, a), m.attach(3, [9, 9, 9, 9, 5])


def test_prefix_key_is_the_whole_prefix():
    """A block whose own tokens match a cached block but whose history differs is not reused: the
    cached (9, 9, 9, 9) block follows (1, 2, 3, 4), so a prompt that starts with it reuses nothing."""
    assert prefix_key_case(M) == (0, 8, 0)


def truncate_case(mod):
    """Rolling 40 tokens (b = 16) back to 17 keeps ceil(17/16) = 2 blocks and frees one; back to 0
    frees the rest; a shared block only loses this table's reference."""
    m = mod.BlockLedger(8, 16)
    m.add_seq(0)
    m.reserve(0, 40)
    m.commit(0, 40)
    m.fork(0, 1)
    out = [m.num_free]
    m.truncate(0, 17)
    out += [len(m.table(0)), m.num_free, m.refcount[m.table(1)[2]]]
    m.truncate(1, 0)
    out += [len(m.table(1)), m.num_free]
    return out


def test_truncate_releases_the_tail():
    assert truncate_case(M) == [5, 2, 5, 1, 0, 6]


def evict_case(mod):
    m = mod.BlockLedger(6, 2)
    for s, base in ((0, 10), (1, 20)):  # two cached 2-block prompts, then both freed
        p = [base, base + 1, base + 2, base + 3, 99]
        m.attach(s, p)
        m.reserve(s, len(p))
        m.commit(s, len(p))
        m.remember(s, p)
        m.free(s)
    out = [m.num_free]
    m.attach(2, [10, 11, 12, 13, 98])  # touches prompt 0's entries: prompt 1's are now the oldest
    out.append(m.evict(3))  # one block wanted: prompt 1's first block, the oldest entry, goes
    out.append(m.cached_prefixes())
    out.append(m.evict(6))  # prompt 0's blocks are referenced by sequence 2: kept
    out.append(m.cached_prefixes())
    m.free(2)
    out.append(m.evict(6))
    return out


def test_evict_is_lru_and_spares_blocks_in_use():
    assert evict_case(M) == [2, 3, [(20, 21, 22, 23), (10, 11), (10, 11, 12, 13)], 4,
                             [(10, 11), (10, 11, 12, 13)], 6]


def zero_token_reserve_case(mod):
    """A reserve of no tokens writes nothing, so a shared partly filled block is not copied."""
    m = mod.BlockLedger(8, 4)
    m.add_seq(0)
    m.reserve(0, 6)
    m.commit(0, 6)
    m.fork(0, 1)
    return m.reserve(1, 0), m.num_free, m.reserve(1, 1), m.num_free


def test_zero_token_reserve_copies_nothing():
    assert zero_token_reserve_case(M) == ([], 6, [(1, 2)], 5)


def multi_block_cow_case(mod):
    """A write that spans two shared blocks copies both: blocks reserved past the committed length
    are shared by a fork too, and the child's 7-token write touches both list entries."""
    m = mod.BlockLedger(8, 4)
    m.add_seq(0)
    m.reserve(0, 8)
    m.commit(0, 1)
    m.fork(0, 1)
    return m.reserve(1, 7), m.table(0), m.table(1), m.num_free


def test_write_across_shared_blocks_copies_each():
    assert multi_block_cow_case(M) == ([(0, 2), (1, 3)], [0, 1], [2, 3], 4)


# ----------------------------------------------------------------------------- invariants, data

def check_invariants(mod, m):
    counts = [0] * len(m.refcount)
    for rec in m.seqs.values():
        assert len(set(rec.blocks)) == len(rec.blocks)
        for blk in rec.blocks:
            counts[blk] += 1
    for rec in m.cache.values():
        counts[rec.block] += 1
    assert counts == m.refcount
    assert set(m.unused_since) == {i for i, r in enumerate(m.refcount) if r == 0}
    assert len(set(m.unused_since.values())) == len(m.unused_since)
    for rec in m.seqs.values():
        assert rec.length <= len(rec.blocks) * m.block_size
    assert len({rec.block for rec in m.cache.values()}) == len(m.cache)


def random_workload(mod, seed, steps=300, n_blocks=40, b=4, check=None, data=True):
    """Seeded random mix of attach/reserve+write/fork/free/truncate/evict. With ``data``, a token
    store (block, slot) -> token applies the returned copies and the writes, and every sequence's
    history is read back through its table after every step."""
    rng = random.Random(seed)
    m = mod.BlockLedger(n_blocks, b)
    store = {}
    hist = {}
    log = []
    next_id = 0

    def write(seq, toks):
        start = m.length(seq)
        copies = m.reserve(seq, len(toks))
        for src, dst in copies:
            for o in range(b):
                if (src, o) in store:
                    store[(dst, o)] = store[(src, o)]
        table = m.table(seq)
        for j, tok in enumerate(toks):
            pos = start + j
            store[(table[pos // b], pos % b)] = tok
        m.commit(seq, start + len(toks))
        hist[seq] = hist[seq][:start] + list(toks)
        return copies

    for _ in range(steps):
        op = rng.random()
        seqs = sorted(m.seqs, key=str)
        if op < 0.25 or not seqs:
            prompt = [rng.randrange(3) for _ in range(rng.randrange(1, 14))]
            seq = next_id
            next_id += 1
            reused = m.attach(seq, prompt)
            hist[seq] = list(prompt[:reused])
            try:
                copies = write(seq, prompt[reused:])
                m.remember(seq, prompt)
                log.append(("attach", seq, reused, copies))
            except mod.PoolExhausted:
                m.free(seq)
                del hist[seq]
                log.append(("attach-full", seq))
        elif op < 0.55:
            seq = rng.choice(seqs)
            toks = [rng.randrange(3) for _ in range(rng.randrange(1, 6))]
            try:
                log.append(("write", seq, write(seq, toks)))
            except mod.PoolExhausted:
                log.append(("write-full", seq))
        elif op < 0.7:
            parent = rng.choice(seqs)
            child = next_id
            next_id += 1
            m.fork(parent, child)
            hist[child] = list(hist[parent])
            log.append(("fork", parent, child))
        elif op < 0.85:
            seq = rng.choice(seqs)
            m.free(seq)
            del hist[seq]
            log.append(("free", seq))
        elif op < 0.93:
            seq = rng.choice(seqs)
            n = rng.randrange(0, m.length(seq) + 1)
            m.truncate(seq, n)
            hist[seq] = hist[seq][:n]
            log.append(("truncate", seq, n))
        else:
            log.append(("evict", m.evict(rng.randrange(n_blocks + 1))))
        if check:
            check(mod, m)
        if data:
            for s, h in hist.items():
                table = m.table(s)
                got = [store.get((table[p // b], p % b)) for p in range(m.length(s))]
                assert got == h, f"history of sequence {s} corrupted"
        log.append((m.num_free, tuple(m.refcount)))
    return log


@pytest.mark.parametrize("seed", range(6))
def test_random_workloads_keep_invariants_and_histories(seed):
    random_workload(M, seed, check=check_invariants)


def test_everything_returns_to_the_pool():
    m = M.BlockLedger(30, 4)
    for s in range(3):
        p = [s, 1, 2, 3, 4, 5, 6, 7, 8]
        m.attach(s, p)
        m.reserve(s, len(p) - m.length(s))
        m.commit(s, len(p))
        m.remember(s, p)
        m.fork(s, 10 + s)
    for s in list(m.seqs):
        m.free(s)
    m.evict(30)
    assert m.num_free == 30 and not m.cache


def test_reserve_is_all_or_nothing():
    m = M.BlockLedger(3, 4)
    m.add_seq(0)
    m.reserve(0, 8)
    m.commit(0, 8)
    m.fork(0, 1)
    before = (m.table(1), list(m.refcount), m.num_free)
    with pytest.raises(M.PoolExhausted):
        m.reserve(1, 9)  # would need a copy of block 1 and two new blocks; only one is unused
    assert (m.table(1), m.refcount, m.num_free) == before


# ----------------------------------------------------------------------------- planted mistakes

def _fresh():
    spec = importlib.util.find_spec("oracle.pa_oracle_blocks")
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _pins_fail(mod) -> bool:
    g = _golden()
    checks = [
        lambda: fork_cow_example(mod, g["fork_cow"]) == (3, 0, 4),
        lambda: prefix_cache_example(mod, g["prefix_cache"]) == (832, 160, 14, 56),
        lambda: task_09_3(mod, g["task_09_3"]) == (32, 31, 42, 320, 278, 556, 41),
        lambda: allocator_order(mod) == [[0, 1], [2, 3, 1], 0, [0, 2, 3, 1]],
        lambda: cached_prompt_reuse(mod) == (80, 96),
        lambda: prefix_key_case(mod) == (0, 8, 0),
        lambda: truncate_case(mod) == [5, 2, 5, 1, 0, 6],
        lambda: evict_case(mod) == [2, 3, [(20, 21, 22, 23), (10, 11), (10, 11, 12, 13)], 4,
                                    [(10, 11), (10, 11, 12, 13)], 6],
        lambda: zero_token_reserve_case(mod) == ([], 6, [(1, 2)], 5),
        lambda: multi_block_cow_case(mod) == ([(0, 2), (1, 3)], [0, 1], [2, 3], 4),
    ]
    for seed in range(3):
        checks.append(lambda seed=seed: random_workload(mod, seed, check=check_invariants) is not None)
    for chk in checks:
        try:
            if not chk():
                return True
        except Exception:  # a broken model may also crash or trip an invariant
            return True
    return False


def test_planted_mistakes_are_caught():
    assert not _pins_fail(M)
    L = "BlockLedger"
    mutants = {}

    m = _fresh()  # no copy-on-write: shared blocks are written in place
    def reserve_no_cow(self, seq, new_tokens):
        rec = self.seqs[seq]
        need = self.blocks_covering(rec.length + new_tokens)
        if max(0, need - len(rec.blocks)) > self.num_free:
            raise m.PoolExhausted("full")
        while len(rec.blocks) < need:
            rec.blocks.append(self._claim())
        return []
    setattr(getattr(m, L), "reserve", reserve_no_cow)
    mutants["no-cow"] = m

    m = _fresh()  # fork without taking references
    def fork_no_hold(self, parent, child):
        src = self.seqs[parent]
        self.seqs[child] = m.SeqRecord(list(src.blocks), src.length)
    setattr(getattr(m, L), "fork", fork_no_hold)
    mutants["fork-no-hold"] = m

    m = _fresh()  # allocator hands out the most recently released block (a stack, not a queue)
    def claim_lifo(self):
        blk = max(self.unused_since, key=self.unused_since.__getitem__)
        del self.unused_since[blk]
        self.refcount[blk] = 1
        return blk
    setattr(getattr(m, L), "_claim", claim_lifo)
    mutants["claim-lifo"] = m

    m = _fresh()  # attach reuses the whole prompt (no token left to prefill)
    orig_attach = getattr(m, L).attach
    def attach_all(self, seq, prompt):
        return orig_attach(self, seq, list(prompt) + [None])
    setattr(getattr(m, L), "attach", attach_all)
    mutants["attach-no-last-token"] = m

    m = _fresh()  # cache keyed by the block's own tokens only
    def key_own(self, tokens, nblocks):
        b = self.block_size
        return tuple(tokens[(nblocks - 1) * b:nblocks * b])
    setattr(getattr(m, L), "_key", key_own)
    setattr(getattr(m, L), "cached_prefixes",
            lambda self: [k for k, _ in sorted(self.cache.items(), key=lambda kv: kv[1].last_use)])
    mutants["key-own-block"] = m

    m = _fresh()  # attach does not refresh the entries it reuses (no LRU touch)
    def attach_no_touch(self, seq, prompt):
        self.add_seq(seq)
        rec = self.seqs[seq]
        usable = max(0, (len(prompt) - 1) // self.block_size)
        hits = 0
        while hits < usable and self._key(prompt, hits + 1) in self.cache:
            hits += 1
        for n in range(1, hits + 1):
            entry = self.cache[self._key(prompt, n)]
            self._hold(entry.block)
            rec.blocks.append(entry.block)
        rec.length = hits * self.block_size
        return rec.length
    setattr(getattr(m, L), "attach", attach_no_touch)
    mutants["attach-no-touch"] = m

    m = _fresh()  # evict ignores other users of a block
    def evict_any(self, blocks_wanted):
        while self.num_free < blocks_wanted and self.cache:
            key = min(self.cache, key=lambda k: self.cache[k].last_use)
            self._release(self.cache.pop(key).block)
        return self.num_free
    setattr(getattr(m, L), "evict", evict_any)
    mutants["evict-in-use"] = m

    m = _fresh()  # truncate keeps every block
    def truncate_keep(self, seq, length):
        self.seqs[seq].length = length
    setattr(getattr(m, L), "truncate", truncate_keep)
    mutants["truncate-keeps-blocks"] = m

    m = _fresh()  # copy-on-write looks only at the block the first new token lands in
    def reserve_first_only(self, seq, new_tokens):
        rec = self.seqs[seq]
        if new_tokens == 0:
            return []
        b = self.block_size
        first, last = rec.length // b, (rec.length + new_tokens - 1) // b
        shared = [j for j in range(first, min(first + 1, len(rec.blocks))) if self.refcount[rec.blocks[j]] > 1]
        missing = max(0, last + 1 - len(rec.blocks))
        if len(shared) + missing > self.num_free:
            raise m.PoolExhausted("full")
        pairs = []
        for j in shared:
            source = rec.blocks[j]
            rec.blocks[j] = self._claim()
            self._release(source)
            pairs.append((source, rec.blocks[j]))
        rec.blocks.extend(self._claim() for _ in range(missing))
        return pairs
    setattr(getattr(m, L), "reserve", reserve_first_only)
    mutants["cow-first-block-only"] = m

    for name, mod in mutants.items():
        assert _pins_fail(mod), f"planted mistake '{name}' was not caught by the pins"
