"""ctypes binding of libpa.so's host block manager (``pa_bm_*``) and of ``pa_copy_blocks``.

:class:`BlockManager` owns one ``pa_block_manager`` handle: the free list and reference counts of a
pool's block ids, the block table and length of every sequence, and the prefix cache. It runs on
the host; the block copies its copy-on-write asks for are run on the GPU by :func:`copy_blocks`.
Every method marshals arguments only: the bookkeeping is the library's C++.
"""

from __future__ import annotations

import ctypes

from . import PaError, _check_tensors, _require, _stream_handle, dtype_code, load_library

PA_ERR_NO_BLOCKS = -4
_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64


class PoolExhausted(PaError):
    """The pool has too few free blocks for the request (nothing was changed)."""


def _bind(lib):
    if getattr(lib, "_pa_bm_bound", False):
        return lib
    sig = {
        "pa_bm_create": ([_I32, _I32], _P),
        "pa_bm_destroy": ([_P], None),
        "pa_bm_num_free": ([_P], _I32),
        "pa_bm_refcount": ([_P, _I32], _I32),
        "pa_bm_num_seqs": ([_P], _I32),
        "pa_bm_add_seq": ([_P, _I64], ctypes.c_int),
        "pa_bm_reserve": ([_P, _I64, _I32, _P, _I32, _P], ctypes.c_int),
        "pa_bm_commit": ([_P, _I64, _I32], ctypes.c_int),
        "pa_bm_fork": ([_P, _I64, _I64], ctypes.c_int),
        "pa_bm_free_seq": ([_P, _I64], ctypes.c_int),
        "pa_bm_truncate": ([_P, _I64, _I32], ctypes.c_int),
        "pa_bm_seq_length": ([_P, _I64], _I32),
        "pa_bm_seq_blocks": ([_P, _I64, _P, _I32], _I32),
        "pa_bm_build_tables": ([_P, _P, _I32, _I32, _I32, _P, _P], ctypes.c_int),
        "pa_bm_prefix_attach": ([_P, _I64, _P, _I32], _I32),
        "pa_bm_prefix_remember": ([_P, _I64, _P, _I32], _I32),
        "pa_bm_prefix_evict": ([_P, _I32], _I32),
        "pa_bm_prefix_entries": ([_P], _I32),
        "pa_copy_blocks": ([_P, _P, _P, _P, _P, _I32, _P], ctypes.c_int),
        "pa_check_copies_host": ([_P, _P, _I32], ctypes.c_int),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    lib._pa_bm_bound = True
    return lib


def _ints(values):
    values = [int(v) for v in values]
    return (_I32 * max(1, len(values)))(*values), len(values)


class BlockManager:
    """Host block manager over ``num_blocks`` blocks of ``block_size`` positions (see include/pa.h)."""

    def __init__(self, num_blocks: int, block_size: int, lib=None):
        self._lib = _bind(lib or load_library())
        self._h = self._lib.pa_bm_create(int(num_blocks), int(block_size))
        if not self._h:
            raise ValueError(f"pa_bm_create({num_blocks}, {block_size}) failed")
        self.num_blocks, self.block_size = int(num_blocks), int(block_size)

    def close(self):
        if self._h:
            self._lib.pa_bm_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def _ok(self, func: str, status: int) -> int:
        if status == PA_ERR_NO_BLOCKS:
            raise PoolExhausted(func, status, self._lib.pa_status_string(status).decode())
        if status < 0:
            raise PaError(func, status, self._lib.pa_status_string(status).decode())
        return status

    @property
    def num_free(self) -> int:
        return self._ok("pa_bm_num_free", self._lib.pa_bm_num_free(self._h))

    @property
    def num_seqs(self) -> int:
        return self._ok("pa_bm_num_seqs", self._lib.pa_bm_num_seqs(self._h))

    @property
    def num_entries(self) -> int:
        return self._ok("pa_bm_prefix_entries", self._lib.pa_bm_prefix_entries(self._h))

    def refcount(self, block: int) -> int:
        return self._ok("pa_bm_refcount", self._lib.pa_bm_refcount(self._h, int(block)))

    def refcounts(self) -> list[int]:
        return [self.refcount(b) for b in range(self.num_blocks)]

    def add_seq(self, seq: int):
        self._ok("pa_bm_add_seq", self._lib.pa_bm_add_seq(self._h, int(seq)))

    def reserve(self, seq: int, new_tokens: int) -> list[tuple[int, int]]:
        """Blocks for the next ``new_tokens`` positions; returns the (source, destination) copies."""
        cap = self.length(seq) // self.block_size + int(new_tokens) // self.block_size + 2
        buf = (_I32 * (2 * cap))()
        n = _I32(0)
        self._ok("pa_bm_reserve",
                 self._lib.pa_bm_reserve(self._h, int(seq), int(new_tokens), buf, cap, ctypes.byref(n)))
        return [(buf[2 * i], buf[2 * i + 1]) for i in range(n.value)]

    def commit(self, seq: int, length: int):
        self._ok("pa_bm_commit", self._lib.pa_bm_commit(self._h, int(seq), int(length)))

    def fork(self, parent: int, child: int):
        self._ok("pa_bm_fork", self._lib.pa_bm_fork(self._h, int(parent), int(child)))

    def free(self, seq: int):
        self._ok("pa_bm_free_seq", self._lib.pa_bm_free_seq(self._h, int(seq)))

    def truncate(self, seq: int, length: int):
        self._ok("pa_bm_truncate", self._lib.pa_bm_truncate(self._h, int(seq), int(length)))

    def length(self, seq: int) -> int:
        return self._ok("pa_bm_seq_length", self._lib.pa_bm_seq_length(self._h, int(seq)))

    def table(self, seq: int) -> list[int]:
        n = self._ok("pa_bm_seq_blocks", self._lib.pa_bm_seq_blocks(self._h, int(seq), None, 0))
        buf = (_I32 * max(1, n))()
        self._ok("pa_bm_seq_blocks", self._lib.pa_bm_seq_blocks(self._h, int(seq), buf, n))
        return list(buf[:n])

    def build_tables(self, seqs, width: int, pad: int = 0):
        """(rows, lengths): int32 table rows padded to ``width`` with ``pad``, and the lengths."""
        seqs = [int(s) for s in seqs]
        ids = (_I64 * max(1, len(seqs)))(*seqs)
        tab = (_I32 * max(1, len(seqs) * int(width)))()
        lens = (_I32 * max(1, len(seqs)))()
        self._ok("pa_bm_build_tables",
                 self._lib.pa_bm_build_tables(self._h, ids, len(seqs), int(width), int(pad), tab, lens))
        w = int(width)
        return [list(tab[i * w:(i + 1) * w]) for i in range(len(seqs))], list(lens[:len(seqs)])

    def attach(self, seq: int, prompt) -> int:
        buf, n = _ints(prompt)
        return self._ok("pa_bm_prefix_attach", self._lib.pa_bm_prefix_attach(self._h, int(seq), buf, n))

    def remember(self, seq: int, tokens) -> int:
        buf, n = _ints(tokens)
        return self._ok("pa_bm_prefix_remember", self._lib.pa_bm_prefix_remember(self._h, int(seq), buf, n))

    def evict(self, blocks_wanted: int) -> int:
        return self._ok("pa_bm_prefix_evict", self._lib.pa_bm_prefix_evict(self._h, int(blocks_wanted)))


def copy_blocks(k_pool, v_pool, pairs, *, scales=None, stream=None):
    """``pa_copy_blocks``: copy block ``pairs[i, 0]`` onto block ``pairs[i, 1]`` in both pools, and for
    8-bit pools (int8 or float8_e4m3fn) the blocks' ``scales [N, Hkv, 2]`` with them (required there,
    absent for float pools). ``pairs`` is an int32 ``[n, 2]`` tensor on the pools' device (or a list of
    pairs, copied there)."""
    import torch

    lib = _bind(load_library())
    if not isinstance(pairs, torch.Tensor):
        pairs = torch.tensor([list(p) for p in pairs], dtype=torch.int32).reshape(-1, 2).to(k_pool.device)
    tensors = dict(k_pool=k_pool, v_pool=v_pool, pairs=pairs)
    if scales is not None:
        tensors["scales"] = scales
    dev = _check_tensors(**tensors)
    _require(pairs.dtype == torch.int32 and pairs.dim() == 2 and pairs.shape[1] == 2, "pairs must be int32 [n, 2]")
    _require(k_pool.shape == v_pool.shape and k_pool.dim() == 4, "pools must be [N, Hkv, b, D] alike")
    from . import PaDims

    n, hkv, bs, d = k_pool.shape
    code = dtype_code(k_pool.dtype)
    if scales is not None:
        _require(scales.dtype == torch.float32 and tuple(scales.shape) == (n, hkv, 2), "scales must be float32 [N, Hkv, 2]")
    dims = PaDims(0, 1, hkv, hkv, d, bs, n, 1, code, code, code, 0, 0)
    st = lib.pa_copy_blocks(ctypes.byref(dims), k_pool.data_ptr(), v_pool.data_ptr(),
                            scales.data_ptr() if scales is not None else None, pairs.data_ptr(),
                            int(pairs.shape[0]), _stream_handle(stream, dev))
    if st:
        raise PaError("pa_copy_blocks", st, lib.pa_status_string(st).decode())
