"""The five synthetic decode workloads plus a general case builder.

Each workload has the shapes, sizes and length mix of the pages' examples:

* ``tiny``: fp32; 4 q heads / 2 kv heads; head_dim 64; b = 16; lengths
  {1, 17, 33, 64}; a 32-block pool handed out as a seeded permutation.
  ``tiny_b4`` replays the worked example of [P1] "Paging": b = 4, table
  [5, 1, 7], and the token at position 9 written and attended, so L = 10.
* ``batch64``: bf16; a Llama-3-8B-shaped layer (32 q / 8 kv heads, head_dim
  128, b = 16); 64 sequences with L ~ U{20..500}. This scales up the chapter
  demo's mix of 32 requests of 20-500 tokens ([P1] "Reserved memory is wasted
  memory"). The pool has 4096 shuffled blocks.
* ``long``: bf16; same heads; 16 sequences with L log-uniform on
  [4096, 32768]; the pool holds every block the sequences need plus 10%,
  shuffled.
* ``prefix``: bf16; 128 sequences share their first 2048 tokens (128 physical
  blocks), each followed by a private suffix of U{64..1024} tokens.
* ``spec``: bf16; 4 query tokens per sequence; 64 q / 8 kv heads;
  256 sequences with L ~ U{1024..8192}.

No public dataset is involved; every value is drawn from a seeded
``torch.Generator``. Floating values are N(0, 1) drawn in fp32, then rounded to
the case dtype. For bf16 that rounding is torch's round-to-nearest-even.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch

CONFIG_NAMES = ("tiny", "tiny_b4", "batch64", "long", "prefix", "spec")
INT32_MAX = 2**31 - 1
_SEEDS = {"tiny": 1000, "batch64": 1001, "long": 1002, "prefix": 1003, "spec": 1004, "tiny_b4": 1005}
_FILL_CHUNK = 1 << 25  # elements drawn per randn call when filling big pools


@dataclass
class Case:
    """One decode step's inputs, as tensors on the CPU (pools: on the device they were drawn on).

    Layouts: ``q [B, T, Hq, D]``; ``k_new``/``v_new [B, T, Hkv, D]``;
    ``k_pool``/``v_pool [N, Hkv, b, D]``; ``block_tables [B, MB]`` int32, where
    entries past a sequence's block count are ``table_pad``;
    ``seq_lens [B]`` int32, counting the T new tokens; ``positions [B, T]``
    int32, holding the new tokens' positions L - T .. L - 1.
    """

    name: str
    q: torch.Tensor
    k_new: torch.Tensor
    v_new: torch.Tensor
    k_pool: torch.Tensor
    v_pool: torch.Tensor
    block_tables: torch.Tensor
    seq_lens: torch.Tensor
    positions: torch.Tensor
    block_size: int
    scale: float
    table_rows: list = field(default_factory=list)  # per sequence: its physical blocks
    unused_blocks: torch.Tensor | None = None        # physical blocks no table references

    @property
    def dims(self):
        b, t, hq, d = self.q.shape
        return dict(num_seqs=b, q_tokens=t, num_q_heads=hq, num_kv_heads=self.k_pool.shape[1],
                    head_dim=d, block_size=self.block_size, num_blocks=self.k_pool.shape[0],
                    max_blocks_per_seq=self.block_tables.shape[1])

    @property
    def max_seq_len(self) -> int:
        return int(self.seq_lens.max()) if self.seq_lens.numel() else 0

    def kv_tokens(self) -> int:
        """Total positions attended over: sum of L_i."""
        return int(self.seq_lens.to(torch.int64).sum())


def _randn(shape, gen, dtype):
    return torch.randn(shape, generator=gen, dtype=torch.float32).to(dtype)


def _fill_pool(shape, gen, dtype):
    """N(0,1) pool drawn in bounded chunks, so big pools never need a full fp32 copy.
    ``gen`` is a CPU or CUDA torch.Generator; the pool lives on the generator's device."""
    out = torch.empty(shape, dtype=dtype, device=gen.device)
    flat = out.view(-1)
    for start in range(0, flat.numel(), _FILL_CHUNK):
        n = min(_FILL_CHUNK, flat.numel() - start)
        flat[start:start + n] = torch.randn(n, generator=gen, dtype=torch.float32, device=gen.device).to(dtype)
    return out


def _ceil_div(a: int, b: int) -> int:
    return -(-a // b)


def build_case(*, name="custom", lengths, num_q_heads, num_kv_heads, head_dim, block_size,
               q_tokens=1, dtype=torch.bfloat16, seed=0, num_blocks=None, shared_prefix_blocks=0,
               table_pad=INT32_MAX, pool_slack=0.0, explicit_tables=None, poison_unused=True,
               pool_device="cpu"):
    """General builder used by every named workload.

    Blocks are handed out like a free list over a seeded permutation of the
    pool: each sequence takes the next ``ceil(L/b)`` entries, as in [P1] "The
    allocator". If ``shared_prefix_blocks`` > 0, the first that many logical
    blocks of every sequence map to the same physical blocks. Their refcount
    equals the number of sequences, as in a forked or prefix-cached prompt
    ([P1] "Sharing blocks"). When ``explicit_tables`` is given, those rows are
    used as they are.

    The pools are drawn on ``pool_device``: CPU by default, or a GPU, where a seeded torch
    CUDA generator makes multi-GB pools in moments. All other tensors are always drawn on
    the CPU.
    """
    gen = torch.Generator().manual_seed(int(seed))
    lengths = [int(x) for x in lengths]
    n_seq = len(lengths)
    need = [_ceil_div(max(L, 0), block_size) for L in lengths]
    if explicit_tables is not None:
        rows = [list(map(int, r)) for r in explicit_tables]
        if num_blocks is None:
            num_blocks = max(max(r) for r in rows if r) + 1
        perm_unused = sorted(set(range(num_blocks)) - {b for r in rows for b in r})
    else:
        private = [n - shared_prefix_blocks for n in need]
        if min(private) < 0:
            raise ValueError("a sequence is shorter than the shared prefix")
        used = shared_prefix_blocks + sum(private)
        if num_blocks is None:
            num_blocks = max(1, math.ceil(used * (1.0 + pool_slack)))
        if used > num_blocks:
            raise MemoryError("KV block pool exhausted")
        perm = torch.randperm(num_blocks, generator=gen).tolist()
        prefix = perm[:shared_prefix_blocks]
        cursor = shared_prefix_blocks
        rows = []
        for n in private:
            rows.append(prefix + perm[cursor:cursor + n])
            cursor += n
        perm_unused = perm[cursor:]
    width = max(1, max(len(r) for r in rows))
    tables = torch.full((n_seq, width), table_pad, dtype=torch.int32)
    for i, r in enumerate(rows):
        if r:
            tables[i, :len(r)] = torch.tensor(r, dtype=torch.int32)

    hq, hkv, d, t = num_q_heads, num_kv_heads, head_dim, q_tokens
    q = _randn((n_seq, t, hq, d), gen, dtype)
    k_new = _randn((n_seq, t, hkv, d), gen, dtype)
    v_new = _randn((n_seq, t, hkv, d), gen, dtype)
    pool_shape = (num_blocks, hkv, block_size, d)
    pool_gen = gen
    if torch.device(pool_device).type != "cpu":
        pool_gen = torch.Generator(device=pool_device).manual_seed(int(seed) + 1)
    k_pool = _fill_pool(pool_shape, pool_gen, dtype)
    v_pool = _fill_pool(pool_shape, pool_gen, dtype)
    unused = torch.tensor(perm_unused, dtype=torch.int64)
    if poison_unused and unused.numel():
        k_pool[unused.to(k_pool.device)] = float("nan")
        v_pool[unused.to(v_pool.device)] = float("nan")
    seq_lens = torch.tensor(lengths, dtype=torch.int32)
    positions = torch.stack([torch.arange(L - t, L, dtype=torch.int32) for L in lengths]) \
        if n_seq else torch.empty((0, t), dtype=torch.int32)
    return Case(name=name, q=q, k_new=k_new, v_new=v_new, k_pool=k_pool, v_pool=v_pool,
                block_tables=tables, seq_lens=seq_lens, positions=positions,
                block_size=block_size, scale=1.0 / math.sqrt(d), table_rows=rows,
                unused_blocks=unused)


def config_lengths(name: str, gen: torch.Generator, num_seqs: int | None = None):
    """Draw the length mix of a named workload (its first ``num_seqs`` sequences if given)."""
    if name == "tiny":
        lens = [1, 17, 33, 64]
    elif name == "tiny_b4":
        lens = [10]
    elif name == "batch64":
        lens = torch.randint(20, 501, (64,), generator=gen).tolist()
    elif name == "long":
        u = torch.rand(16, generator=gen, dtype=torch.float64)
        lo, hi = math.log(4096.0), math.log(32768.0)
        lens = [int(round(math.exp(lo + float(x) * (hi - lo)))) for x in u]
    elif name == "prefix":
        lens = [2048 + int(s) for s in torch.randint(64, 1025, (128,), generator=gen)]
    elif name == "spec":
        lens = torch.randint(1024, 8193, (256,), generator=gen).tolist()
    else:
        raise KeyError(name)
    if num_seqs is not None:
        lens = lens[:num_seqs]
    return lens


def make_case(name: str, *, num_seqs: int | None = None, seed: int | None = None,
              table_pad: int = INT32_MAX, poison_unused: bool = True, pool_device="cpu") -> Case:
    """Build a named workload; ``num_seqs`` keeps only its first sequences."""
    seed = _SEEDS[name] if seed is None else seed
    gen = torch.Generator().manual_seed(seed)
    lens = config_lengths(name, gen, num_seqs)
    common = dict(name=name, lengths=lens, seed=seed + 7919, table_pad=table_pad,
                  poison_unused=poison_unused, pool_device=pool_device)
    if name == "tiny":
        return build_case(num_q_heads=4, num_kv_heads=2, head_dim=64, block_size=16,
                          dtype=torch.float32, num_blocks=32, **common)
    if name == "tiny_b4":
        return build_case(num_q_heads=4, num_kv_heads=2, head_dim=64, block_size=4,
                          dtype=torch.float32, num_blocks=8, explicit_tables=[[5, 1, 7]], **common)
    if name == "batch64":
        return build_case(num_q_heads=32, num_kv_heads=8, head_dim=128, block_size=16,
                          dtype=torch.bfloat16, num_blocks=4096, **common)
    if name == "long":
        return build_case(num_q_heads=32, num_kv_heads=8, head_dim=128, block_size=16,
                          dtype=torch.bfloat16, pool_slack=0.10, **common)
    if name == "prefix":
        return build_case(num_q_heads=32, num_kv_heads=8, head_dim=128, block_size=16,
                          dtype=torch.bfloat16, shared_prefix_blocks=128, pool_slack=0.10, **common)
    if name == "spec":
        return build_case(num_q_heads=64, num_kv_heads=8, head_dim=128, block_size=16,
                          q_tokens=4, dtype=torch.bfloat16, **common)
    raise KeyError(name)


def int8_pools(case: Case, *, seed: int | None = None, device=None):
    """Seeded int8 K/V pools of the case's pool shape, for the int8 entry points.

    Codes are round(N(0, 40^2)) clipped to [-127, 127]; each (block, kv head) gets a scale drawn from
    U[0.02, 0.04] (about what max|x| / 127 gives for a block of N(0, 1) values). No quantiser runs
    here: codes and scales are drawn directly. Blocks no table references get NaN scales, so a read
    of one would show in the output. Returns ``(k_codes, v_codes, scales)`` on ``device`` (the case's
    pool device by default), ``scales [N, Hkv, 2]`` holding the (K, V) scale pair of each (block, kv
    head).
    """
    device = torch.device(device) if device is not None else case.k_pool.device
    gen = torch.Generator(device=device).manual_seed(int(seed if seed is not None else 7777))
    n, hkv, b, d = case.k_pool.shape
    codes, scales = [], torch.empty((n, hkv, 2), dtype=torch.float32, device=device)
    for side in range(2):
        c = torch.empty((n, hkv, b, d), dtype=torch.int8, device=device)
        flat = c.view(-1)
        for start in range(0, flat.numel(), _FILL_CHUNK):
            m = min(_FILL_CHUNK, flat.numel() - start)
            x = torch.randn(m, generator=gen, dtype=torch.float32, device=device) * 40.0
            flat[start:start + m] = x.round().clamp(-127, 127).to(torch.int8)
        scales[:, :, side] = torch.rand((n, hkv), generator=gen, dtype=torch.float32, device=device) * 0.02 + 0.02
        codes.append(c)
    if case.unused_blocks is not None and case.unused_blocks.numel():
        scales[case.unused_blocks.to(device)] = float("nan")
    return codes[0], codes[1], scales


def fp8_pools(case: Case, *, seed: int | None = None, device=None):
    """Seeded FP8 (E4M3) K/V pools of the case's pool shape, for the fp8 entry points.

    Codes are N(0, 120^2) draws clipped to +-448 and rounded to E4M3 by torch's float8_e4m3fn cast
    (round to nearest even), as the float pools round N(0, 1) draws to bf16; each (block, kv head)
    gets a scale drawn from U[0.004, 0.008] (about what max|x| / 448 gives for a block of N(0, 1)
    values). Blocks no table references get NaN scales. Returns ``(k_codes, v_codes, scales)`` with
    float8_e4m3fn codes and ``scales [N, Hkv, 2]`` (the (K, V) pair of each (block, kv head)), on
    ``device`` (the case's pool device by default).
    """
    device = torch.device(device) if device is not None else case.k_pool.device
    gen = torch.Generator(device=device).manual_seed(int(seed if seed is not None else 8888))
    n, hkv, b, d = case.k_pool.shape
    codes, scales = [], torch.empty((n, hkv, 2), dtype=torch.float32, device=device)
    for side in range(2):
        c = torch.empty((n, hkv, b, d), dtype=torch.float8_e4m3fn, device=device)
        flat = c.view(-1)
        for start in range(0, flat.numel(), _FILL_CHUNK):
            m = min(_FILL_CHUNK, flat.numel() - start)
            x = torch.randn(m, generator=gen, dtype=torch.float32, device=device) * 120.0
            flat[start:start + m] = x.clamp(-448.0, 448.0).to(torch.float8_e4m3fn)
        scales[:, :, side] = torch.rand((n, hkv), generator=gen, dtype=torch.float32, device=device) * 0.004 + 0.004
        codes.append(c)
    if case.unused_blocks is not None and case.unused_blocks.numel():
        scales[case.unused_blocks.to(device)] = float("nan")
    return codes[0], codes[1], scales


# ----------------------------------------------------------------------------- paged prefill

@dataclass
class PrefillCase:
    """One (chunked) prefill step's inputs, packed: sequence i owns rows ``q_start[i] .. q_start[i+1]-1``
    of ``q [Q, Hq, D]`` and ``k_new``/``v_new [Q, Hkv, D]``, its newest ``n_i`` positions after a history
    of ``L_i - n_i``. Pools and tables as in :class:`Case`; the chunk's slots hold stale values until
    the chunk is written."""

    name: str
    q: torch.Tensor
    k_new: torch.Tensor
    v_new: torch.Tensor
    k_pool: torch.Tensor
    v_pool: torch.Tensor
    block_tables: torch.Tensor
    seq_lens: torch.Tensor
    q_start: torch.Tensor
    block_size: int
    scale: float
    histories: list
    chunks: list

    @property
    def max_chunk(self) -> int:
        return max(self.chunks) if self.chunks else 0

    def attended_pairs(self) -> int:
        """Sum over chunk tokens of the positions each attends to: sum_i sum_j (h_i + j + 1)."""
        return sum(n * h + n * (n + 1) // 2 for h, n in zip(self.histories, self.chunks))


def build_prefill_case(*, name="custom", histories, chunks, num_q_heads, num_kv_heads, head_dim, block_size,
                       dtype=torch.bfloat16, seed=0, pool_slack=0.0, pool_device="cpu") -> PrefillCase:
    """Histories and chunk lengths per sequence; the pools come from :func:`build_case` over the total
    lengths (blocks from a seeded free-list permutation, unused blocks NaN), then q and the chunk's new
    K/V rows are drawn N(0, 1) in fp32 and rounded to ``dtype``."""
    histories = [int(h) for h in histories]
    chunks = [int(n) for n in chunks]
    lengths = [h + n for h, n in zip(histories, chunks)]
    base = build_case(name=name, lengths=lengths, num_q_heads=num_q_heads, num_kv_heads=num_kv_heads,
                      head_dim=head_dim, block_size=block_size, dtype=dtype, seed=seed, pool_slack=pool_slack,
                      pool_device=pool_device)
    gen = torch.Generator().manual_seed(int(seed) + 3)
    total = sum(chunks)
    q = _randn((total, num_q_heads, head_dim), gen, dtype)
    k_new = _randn((total, num_kv_heads, head_dim), gen, dtype)
    v_new = _randn((total, num_kv_heads, head_dim), gen, dtype)
    q_start = torch.zeros(len(chunks) + 1, dtype=torch.int32)
    if chunks:
        q_start[1:] = torch.cumsum(torch.tensor(chunks, dtype=torch.int64), 0).to(torch.int32)
    return PrefillCase(name=name, q=q, k_new=k_new, v_new=v_new, k_pool=base.k_pool, v_pool=base.v_pool,
                       block_tables=base.block_tables, seq_lens=base.seq_lens, q_start=q_start,
                       block_size=block_size, scale=1.0 / math.sqrt(head_dim), histories=histories, chunks=chunks)


_PREFILL_SEEDS = {"prefill": 1006, "prefill_small": 1007}


def make_prefill_case(name: str, *, num_seqs: int | None = None, pool_device="cpu") -> PrefillCase:
    """Named prefill workloads:

    * ``prefill``: bf16; 32 q / 8 kv heads; head_dim 128; b 16; 16 sequences, each a chunk of
      U{512..2048} new tokens after a paged history of U{0..4096} tokens (chunked prefill).
    * ``prefill_small``: the same shape with 4 sequences, chunks U{1..200}, histories U{0..300}.
    """
    gen = torch.Generator().manual_seed(_PREFILL_SEEDS[name])
    if name == "prefill":
        n_seq, chunk_rng, hist_rng = 16, (512, 2048), (0, 4096)
    elif name == "prefill_small":
        n_seq, chunk_rng, hist_rng = 4, (1, 200), (0, 300)
    else:
        raise KeyError(name)
    chunks = torch.randint(chunk_rng[0], chunk_rng[1] + 1, (n_seq,), generator=gen).tolist()
    hists = torch.randint(hist_rng[0], hist_rng[1] + 1, (n_seq,), generator=gen).tolist()
    if num_seqs is not None:
        chunks, hists = chunks[:num_seqs], hists[:num_seqs]
    return build_prefill_case(name=name, histories=hists, chunks=chunks, num_q_heads=32, num_kv_heads=8,
                              head_dim=128, block_size=16, dtype=torch.bfloat16, seed=_PREFILL_SEEDS[name] + 7919,
                              pool_slack=0.05, pool_device=pool_device)
