"""Reference model of the host-side block manager: block pool, per-sequence tables,
fork with copy-on-write, and the prefix cache.

TEST INFRASTRUCTURE ONLY (see the package docstring): no product code imports it.

It follows the behaviour [P1] "25. Paged attention and prefix caching" gives in
"The allocator", "The paged cache", "Sharing blocks: forks and copy-on-write" and
"Prefix caching", and [P2] "Модуль 09: PagedAttention: пейджинг KV-кэша", §4
(prefix sharing, reference counts, copy-on-write):

* The pool hands out blocks from a first-in first-out free list; each block has a
  reference count (tables and cache entries that point to it). A block returns to
  the free list when its count reaches zero; releasing below zero is an error.
* A sequence owns a table of blocks and a length. Before new tokens are written,
  ``reserve`` makes blocks exist for positions [length, length + n): any block in
  that range that is shared (count > 1) is first replaced by a fresh copy (the
  caller copies the data: the (source, destination) pairs are returned), then
  missing blocks are appended. ``commit`` records the new length after the write.
* ``fork`` gives a new sequence the parent's table and length, sharing every block.
* ``free`` releases a sequence's blocks; ``truncate`` rolls a sequence back to a
  shorter length and releases the blocks it no longer needs.
* The prefix cache maps a full block to the whole token prefix that ends with it,
  holds its own reference on each cached block, and keeps entries in
  least-recently-used order. ``attach`` reuses the longest cached run of full
  blocks of a prompt but leaves at least one prompt token to prefill; ``remember``
  publishes a sequence's full blocks after its prefill; ``evict`` drops entries
  nobody else references, oldest first, until enough blocks are free.

Readings where the pages leave a step open:

* ``reserve`` is all-or-nothing here: if the pool cannot supply every block the
  call needs (copies and new blocks), it raises before changing anything. The
  page's version may allocate some blocks before it runs out.
* The padding of a batch's table rows is a parameter (the page pads with 0).
"""

from __future__ import annotations

from collections import OrderedDict, deque

__all__ = ["BlockPool", "PagedCache", "PrefixCache", "PoolExhausted"]


class PoolExhausted(MemoryError):
    """The pool has fewer free blocks than a request needs."""


class BlockPool:
    def __init__(self, num_blocks: int):
        self.free_list = deque(range(num_blocks))
        self.refs = [0] * num_blocks

    @property
    def num_free(self) -> int:
        return len(self.free_list)

    def take(self) -> int:
        if not self.free_list:
            raise PoolExhausted("no free block")
        blk = self.free_list.popleft()
        self.refs[blk] = 1
        return blk

    def share(self, blk: int):
        self.refs[blk] += 1

    def drop(self, blk: int):
        if self.refs[blk] <= 0:
            raise RuntimeError(f"block {blk} released more often than referenced")
        self.refs[blk] -= 1
        if self.refs[blk] == 0:
            self.free_list.append(blk)


class PagedCache:
    def __init__(self, num_blocks: int, block_size: int):
        self.pool = BlockPool(num_blocks)
        self.b = block_size
        self.tables: dict[int, list[int]] = {}
        self.lengths: dict[int, int] = {}

    def blocks_for(self, tokens: int) -> int:
        return -(-tokens // self.b)

    def add_seq(self, seq: int):
        if seq in self.tables:
            raise KeyError(f"sequence {seq} exists")
        self.tables[seq] = []
        self.lengths[seq] = 0

    def reserve(self, seq: int, new_tokens: int) -> list[tuple[int, int]]:
        """Blocks for positions [length, length + new_tokens); returns the (src, dst) block copies."""
        table = self.tables[seq]
        start = self.lengths[seq]
        end = start + new_tokens
        want = self.blocks_for(end)
        touched = range(start // self.b, min(len(table), want))
        shared = [j for j in touched if self.pool.refs[table[j]] > 1]
        grow = max(0, want - len(table))
        if len(shared) + grow > self.pool.num_free:
            raise PoolExhausted(f"need {len(shared) + grow} blocks, {self.pool.num_free} free")
        copies = []
        for j in shared:
            fresh = self.pool.take()
            copies.append((table[j], fresh))
            self.pool.drop(table[j])
            table[j] = fresh
        for _ in range(grow):
            table.append(self.pool.take())
        return copies

    def commit(self, seq: int, new_length: int):
        if new_length > len(self.tables[seq]) * self.b:
            raise ValueError("length beyond the reserved blocks")
        self.lengths[seq] = max(self.lengths[seq], new_length)

    def fork(self, parent: int, child: int):
        self.add_seq(child)
        self.tables[child] = list(self.tables[parent])
        self.lengths[child] = self.lengths[parent]
        for blk in self.tables[child]:
            self.pool.share(blk)

    def free(self, seq: int):
        for blk in self.tables.pop(seq):
            self.pool.drop(blk)
        del self.lengths[seq]

    def truncate(self, seq: int, length: int):
        if not 0 <= length <= self.lengths[seq]:
            raise ValueError("truncate only rolls a sequence back")
        keep = self.blocks_for(length)
        for blk in self.tables[seq][keep:]:
            self.pool.drop(blk)
        del self.tables[seq][keep:]
        self.lengths[seq] = length

    def build_tables(self, seqs, width: int, pad: int):
        rows, lens = [], []
        for s in seqs:
            t = self.tables[s]
            if len(t) > width:
                raise ValueError("table wider than the requested width")
            rows.append(t + [pad] * (width - len(t)))
            lens.append(self.lengths[s])
        return rows, lens


class PrefixCache:
    """Full blocks keyed by the entire token prefix that ends with them; LRU order."""

    def __init__(self, cache: PagedCache):
        self.cache = cache
        self.entries: OrderedDict[tuple, int] = OrderedDict()

    def attach(self, seq: int, prompt) -> int:
        c = self.cache
        c.add_seq(seq)
        b = c.b
        reused = 0
        while reused + b <= len(prompt) - 1:  # keep one prompt token to prefill
            key = tuple(prompt[:reused + b])
            blk = self.entries.get(key)
            if blk is None:
                break
            self.entries.move_to_end(key)
            c.pool.share(blk)
            c.tables[seq].append(blk)
            reused += b
        c.lengths[seq] = reused
        return reused

    def remember(self, seq: int, tokens) -> int:
        c = self.cache
        published = 0
        for j in range(len(tokens) // c.b):
            key = tuple(tokens[:(j + 1) * c.b])
            if key in self.entries:
                continue
            blk = c.tables[seq][j]
            c.pool.share(blk)
            self.entries[key] = blk
            published += 1
        return published

    def evict(self, blocks_wanted: int) -> int:
        c = self.cache
        for key in list(self.entries):
            if c.pool.num_free >= blocks_wanted:
                break
            blk = self.entries[key]
            if c.pool.refs[blk] == 1:
                del self.entries[key]
                c.pool.drop(blk)
        return c.pool.num_free
