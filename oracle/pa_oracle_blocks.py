"""Reference model of the host-side block manager: who holds which physical block, each sequence's
block table, copy-on-write, and the prefix cache.

TEST INFRASTRUCTURE ONLY (see the package docstring): no product code imports it.

The rules it models, stated from the pages' prose:

* [P1] "25. Paged attention and prefix caching", "The allocator"; [P2] "Модуль 09: PagedAttention:
  пейджинг KV-кэша", section 4: blocks are handed out from the set of unused blocks and carry a
  reference count. A block is unused again once nothing references it; the one handed out next is
  the one that has been unused the longest. Releasing a block nobody holds is an error.
* [P1] "The paged cache": a sequence is a list of physical blocks plus a length; position p lives in
  list entry p // b. Before new tokens are written, blocks are made to exist for them; the length
  is recorded after the write.
* [P1] "Sharing blocks: forks and copy-on-write"; [P2] section 4: a fork shares every block of the
  parent (one more reference each). A block that is about to receive a token while someone else
  also references it is first replaced, in this sequence's list only, by a private copy.
* [P1] "Prefix caching": a full block is cached under the whole token prefix that ends with it, the
  cache holds one reference of its own, and entries are dropped least recently used first, and only
  while nobody else holds their block. A new prompt reuses the leading run of its full blocks that
  the cache holds, but always leaves its last token to be computed.

Design (this model's own): the state is a few flat tables, and every operation is a short edit of
them.

* ``refcount[blk]``: references to a block, one per list entry holding it and one per cache record.
* ``unused_since[blk]``: for every block without references, the clock tick at which it lost its
  last one (blocks that were never used get ticks below zero, in id order). Handing out a block is a
  minimum over this table.
* ``seqs[seq]``: a record of the sequence's block list and length.
* ``cache[key]``: a record of the cached block and the tick of its last use, where ``key`` is the
  tuple of the prefix's per-block token tuples. Eviction is a minimum over the last-use ticks of
  the records whose block has no other holder.
* One clock, advanced by every release to the unused set and every cache use, orders both.

Readings where the pages leave a step open:

* ``reserve`` is all-or-nothing: if the pool cannot supply every block the call needs (copies and
  new blocks), it raises before changing anything. It returns the (source, destination) block pairs
  whose data the caller copies before writing; a reserve of zero tokens copies nothing.
* ``commit`` never shortens a sequence; ``truncate`` does.
* The padding of a batch's table rows is a parameter.
"""

from __future__ import annotations

from dataclasses import dataclass, field

__all__ = ["BlockLedger", "PoolExhausted"]


class PoolExhausted(MemoryError):
    """The pool has fewer unused blocks than a request needs."""


@dataclass
class SeqRecord:
    blocks: list = field(default_factory=list)
    length: int = 0


@dataclass
class CacheRecord:
    block: int
    last_use: int


class BlockLedger:
    def __init__(self, num_blocks: int, block_size: int):
        if num_blocks < 1 or block_size < 1:
            raise ValueError("a pool needs at least one block of at least one slot")
        self.block_size = block_size
        self.refcount = [0] * num_blocks
        self.unused_since = {blk: blk - num_blocks for blk in range(num_blocks)}
        self.seqs: dict = {}
        self.cache: dict = {}
        self._clock = 0

    # ------------------------------------------------------------------ references

    def _now(self) -> int:
        self._clock += 1
        return self._clock

    @property
    def num_free(self) -> int:
        return len(self.unused_since)

    def _claim(self) -> int:
        blk = min(self.unused_since, key=self.unused_since.__getitem__)
        del self.unused_since[blk]
        self.refcount[blk] = 1
        return blk

    def _hold(self, blk: int):
        self.refcount[blk] += 1

    def _release(self, blk: int):
        if self.refcount[blk] < 1:
            raise RuntimeError(f"block {blk} released more often than it was held")
        self.refcount[blk] -= 1
        if self.refcount[blk] == 0:
            self.unused_since[blk] = self._now()

    # ------------------------------------------------------------------ sequences

    def blocks_covering(self, tokens: int) -> int:
        return -(-tokens // self.block_size)

    def table(self, seq) -> list:
        return list(self.seqs[seq].blocks)

    def length(self, seq) -> int:
        return self.seqs[seq].length

    def add_seq(self, seq):
        if seq in self.seqs:
            raise KeyError(f"sequence {seq} exists")
        self.seqs[seq] = SeqRecord()

    def reserve(self, seq, new_tokens: int) -> list:
        """Blocks for positions [length, length + new_tokens); returns the (source, destination) copies."""
        rec = self.seqs[seq]
        if new_tokens < 0:
            raise ValueError("negative token count")
        if new_tokens == 0:
            return []
        b = self.block_size
        first, last = rec.length // b, (rec.length + new_tokens - 1) // b  # list entries written
        shared = [j for j in range(first, min(last + 1, len(rec.blocks))) if self.refcount[rec.blocks[j]] > 1]
        missing = max(0, last + 1 - len(rec.blocks))
        if len(shared) + missing > self.num_free:
            raise PoolExhausted(f"need {len(shared) + missing} blocks, {self.num_free} unused")
        pairs = []
        for j in shared:
            source = rec.blocks[j]
            rec.blocks[j] = self._claim()
            self._release(source)
            pairs.append((source, rec.blocks[j]))
        rec.blocks.extend(self._claim() for _ in range(missing))
        return pairs

    def commit(self, seq, new_length: int):
        rec = self.seqs[seq]
        if new_length < 0 or new_length > len(rec.blocks) * self.block_size:
            raise ValueError("length beyond the reserved blocks")
        rec.length = max(rec.length, new_length)

    def fork(self, parent, child):
        if child in self.seqs or child == parent:
            raise KeyError(f"sequence {child} exists")
        src = self.seqs[parent]
        for blk in src.blocks:
            self._hold(blk)
        self.seqs[child] = SeqRecord(list(src.blocks), src.length)

    def free(self, seq):
        for blk in self.seqs.pop(seq).blocks:
            self._release(blk)

    def truncate(self, seq, length: int):
        rec = self.seqs[seq]
        if not 0 <= length <= rec.length:
            raise ValueError("truncate only rolls a sequence back")
        keep = self.blocks_covering(length)
        dropped, rec.blocks = rec.blocks[keep:], rec.blocks[:keep]
        for blk in dropped:
            self._release(blk)
        rec.length = length

    def build_tables(self, seqs, width: int, pad: int):
        recs = [self.seqs[s] for s in seqs]
        if any(len(r.blocks) > width for r in recs):
            raise ValueError("table wider than the requested width")
        return [r.blocks + [pad] * (width - len(r.blocks)) for r in recs], [r.length for r in recs]

    # ------------------------------------------------------------------ prefix cache

    def _key(self, tokens, nblocks: int) -> tuple:
        b = self.block_size
        return tuple(tuple(tokens[k * b:(k + 1) * b]) for k in range(nblocks))

    @property
    def num_entries(self) -> int:
        return len(self.cache)

    def cached_prefixes(self) -> list:
        """Every cached prefix as one flat token tuple, least recently used first."""
        order = sorted(self.cache.items(), key=lambda kv: kv[1].last_use)
        return [sum(key, ()) for key, _ in order]

    def attach(self, seq, prompt) -> int:
        """A new sequence that reuses the leading cached full blocks of its prompt; returns the
        number of prompt tokens it starts with."""
        self.add_seq(seq)
        rec = self.seqs[seq]
        usable = max(0, (len(prompt) - 1) // self.block_size)  # the last prompt token is always computed
        hits = 0
        while hits < usable and self._key(prompt, hits + 1) in self.cache:
            hits += 1
        for n in range(1, hits + 1):
            entry = self.cache[self._key(prompt, n)]
            entry.last_use = self._now()
            self._hold(entry.block)
            rec.blocks.append(entry.block)
        rec.length = hits * self.block_size
        return rec.length

    def remember(self, seq, tokens) -> int:
        """Cache the sequence's full blocks under their prefixes; returns how many were new."""
        rec = self.seqs[seq]
        full = len(tokens) // self.block_size
        if full > len(rec.blocks):
            raise ValueError("more full blocks than the sequence holds")
        new = 0
        for n in range(1, full + 1):
            key = self._key(tokens, n)
            if key not in self.cache:
                self._hold(rec.blocks[n - 1])
                self.cache[key] = CacheRecord(rec.blocks[n - 1], self._now())
                new += 1
        return new

    def evict(self, blocks_wanted: int) -> int:
        """Drop cache records nobody else uses, least recently used first, until blocks_wanted blocks
        are unused or no such record is left; returns the unused count."""
        while self.num_free < blocks_wanted:
            idle = [(rec.last_use, key) for key, rec in self.cache.items() if self.refcount[rec.block] == 1]
            if not idle:
                break
            _, key = min(idle)
            self._release(self.cache.pop(key).block)
        return self.num_free
