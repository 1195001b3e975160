"""paged_kv_cache_69_amd: a paged-KV-cache decode step for AMD MI355X (gfx950).

This module is a thin ctypes binding over ``libpa.so``, whose C ABI is declared
in ``include/pa.h``. It only marshals arguments: every step of the path runs in
the library's HIP kernels, and PyTorch supplies device memory and streams. If
the library is missing, every call raises. There is no fallback path.

Entry points, with the same names as the C ABI:

* :func:`write_kv`: the KV-append scatter (``pa_write_kv``).
* :func:`decode`: single-pass paged decode attention (``pa_decode``).
* :func:`decode_partitioned`: split-context decode plus its merge pass
  (``pa_decode_partitioned``).
* :func:`workspace_bytes`: workspace size for :func:`decode_partitioned`.
* :func:`decode_partitioned_noalloc`: the same with the library's fixed device scratch instead of a
  workspace, for callers that cannot allocate (``pa_decode_partitioned_noalloc``).
* :func:`write_kv_decode`: append + decode in one launch (``pa_write_kv_decode``,
  ``pa_write_kv_decode_partitioned``).
* :func:`decode_cascade`: decode with a shared prefix attended once (``pa_decode_cascade``).
* :func:`write_kv_int8`, :func:`decode_int8`, :func:`decode_partitioned_int8`: the int8 KV cache, and
  the same three for FP8 (E4M3) pools. 8-bit pools carry one ``scales [N, Hkv, 2]`` float32 tensor,
  the (K, V) scale pair of every (block, kv head).
* :func:`write_kv_varlen`, :func:`prefill`: paged (chunked) prefill over packed chunks
  (``pa_write_kv_varlen``, ``pa_prefill``).
* :mod:`.blocks`: the host block manager (``pa_bm_*``: free list, reference counts, tables with
  copy-on-write, prefix cache) and :func:`copy_blocks` (``pa_copy_blocks``).
"""

from __future__ import annotations

import ctypes
import os

from ._build import LIB_PATH

PA_F32, PA_BF16, PA_INT8, PA_FP8_E4M3 = 0, 1, 2, 3
NOALLOC_SCRATCH_BYTES = 32 << 20  # PA_NOALLOC_SCRATCH_BYTES
VARIANT_AUTO, VARIANT_VALU, VARIANT_MFMA = 0, 1, 2
SPLIT_AUTO, SPLIT_ONE_PER_WAVE, SPLIT_TWO_PER_WAVE, SPLIT_BALANCED = 0, 1, 2, 3  # pa_split_schedule
EXPORTS = (
    "pa_write_kv",
    "pa_decode",
    "pa_decode_partitioned_workspace_bytes",
    "pa_decode_partitioned",
    "pa_decode_partitioned_schedule",
    "pa_decode_partitioned_noalloc",
    "pa_decode_cascade_workspace_bytes",
    "pa_decode_cascade",
    "pa_write_kv_decode_cascade",
    "pa_write_kv_decode",
    "pa_write_kv_decode_partitioned",
    "pa_write_kv_int8",
    "pa_decode_int8",
    "pa_decode_partitioned_int8",
    "pa_write_kv_fp8",
    "pa_decode_fp8",
    "pa_decode_partitioned_fp8",
    "pa_write_kv_varlen",
    "pa_prefill",
    "pa_check_prefill_host",
    "pa_copy_blocks",
    "pa_check_copies_host",
    "pa_bm_create",
    "pa_bm_destroy",
    "pa_bm_num_free",
    "pa_bm_refcount",
    "pa_bm_num_seqs",
    "pa_bm_add_seq",
    "pa_bm_reserve",
    "pa_bm_commit",
    "pa_bm_fork",
    "pa_bm_free_seq",
    "pa_bm_truncate",
    "pa_bm_seq_length",
    "pa_bm_seq_blocks",
    "pa_bm_build_tables",
    "pa_bm_prefix_attach",
    "pa_bm_prefix_remember",
    "pa_bm_prefix_evict",
    "pa_bm_prefix_entries",
    "pa_check_inputs_host",
    "pa_status_string",
    "pa_abi_version",
)
ABI_VERSION = 2

_DIM_FIELDS = ("num_seqs", "q_tokens", "num_q_heads", "num_kv_heads", "head_dim", "block_size",
               "num_blocks", "max_blocks_per_seq", "q_dtype", "kv_dtype", "out_dtype", "variant", "split_schedule")


class PaDims(ctypes.Structure):
    """Mirror of ``pa_dims`` in include/pa.h."""

    _fields_ = [(name, ctypes.c_int32) for name in _DIM_FIELDS]


class PaError(RuntimeError):
    """A libpa entry point returned a non-zero status."""

    def __init__(self, func: str, status: int, text: str):
        super().__init__(f"{func} failed: {text} (status {status})")
        self.status = status


_lib = None
_P = ctypes.c_void_p
_I32 = ctypes.c_int32


def load_library(path: str | None = None) -> ctypes.CDLL:
    """Load libpa.so (once) and declare its signatures. Raises if it has not been built."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    path = path or LIB_PATH
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it first (python -m paged_kv_cache_69_amd._build, "
                           "or __graft_entry__.build())")
    # torch first: its HIP runtime (libamdhip64.so.7, the same soname as ROCm's) is then the one
    # libpa.so binds to. Loaded the other way round, the process would hold two HIP runtimes and the
    # streams and device pointers torch hands over would belong to the other one.
    import torch  # noqa: F401

    lib = ctypes.CDLL(path)
    dims_p = ctypes.POINTER(PaDims)
    lib.pa_write_kv.argtypes = [dims_p, _P, _P, _P, _P, _P, _P, _P]
    lib.pa_write_kv.restype = ctypes.c_int
    lib.pa_decode.argtypes = [dims_p, _P, _P, _P, _P, _P, ctypes.c_float, _P, _P]
    lib.pa_decode.restype = ctypes.c_int
    lib.pa_decode_partitioned_workspace_bytes.argtypes = [dims_p, _I32, _I32]
    lib.pa_decode_partitioned_workspace_bytes.restype = ctypes.c_size_t
    lib.pa_decode_partitioned_schedule.argtypes = [dims_p, _I32, _I32]
    lib.pa_decode_partitioned_schedule.restype = ctypes.c_int
    lib.pa_decode_partitioned.argtypes = [dims_p, _P, _P, _P, _P, _P, ctypes.c_float, _P, _I32, _I32, _P,
                                          ctypes.c_size_t, _P]
    lib.pa_decode_partitioned.restype = ctypes.c_int
    lib.pa_decode_partitioned_noalloc.argtypes = [dims_p, _P, _P, _P, _P, _P, ctypes.c_float, _P, _I32, _I32, _P]
    lib.pa_decode_partitioned_noalloc.restype = ctypes.c_int
    lib.pa_decode_cascade_workspace_bytes.argtypes = [dims_p, _I32, _I32, _I32]
    lib.pa_decode_cascade_workspace_bytes.restype = ctypes.c_size_t
    lib.pa_decode_cascade.argtypes = [dims_p, _P, _P, _P, _P, _P, ctypes.c_float, _P, _I32, _I32, _I32, _P,
                                      ctypes.c_size_t, _P]
    lib.pa_decode_cascade.restype = ctypes.c_int
    lib.pa_write_kv_decode_cascade.argtypes = [dims_p, _P, _P, _P, _P, _P, _P, _P, ctypes.c_float, _P, _I32, _I32,
                                               _I32, _P, ctypes.c_size_t, _P]
    lib.pa_write_kv_decode_cascade.restype = ctypes.c_int
    lib.pa_write_kv_decode.argtypes = [dims_p, _P, _P, _P, _P, _P, _P, _P, ctypes.c_float, _P, _P]
    lib.pa_write_kv_decode.restype = ctypes.c_int
    lib.pa_write_kv_decode_partitioned.argtypes = [dims_p, _P, _P, _P, _P, _P, _P, _P, ctypes.c_float, _P, _I32,
                                                   _I32, _P, ctypes.c_size_t, _P]
    lib.pa_write_kv_decode_partitioned.restype = ctypes.c_int
    lib.pa_write_kv_int8.argtypes = [dims_p, _P, _P, _P, _P, _P, _P, _P, _P]
    lib.pa_write_kv_int8.restype = ctypes.c_int
    lib.pa_decode_int8.argtypes = [dims_p, _P, _P, _P, _P, _P, _P, ctypes.c_float, _P, _P]
    lib.pa_decode_int8.restype = ctypes.c_int
    lib.pa_decode_partitioned_int8.argtypes = [dims_p, _P, _P, _P, _P, _P, _P, ctypes.c_float, _P, _I32, _I32,
                                               _P, ctypes.c_size_t, _P]
    lib.pa_decode_partitioned_int8.restype = ctypes.c_int
    for suffix in ("write_kv", "decode", "decode_partitioned"):  # the FP8 entry points mirror the int8 ones
        src, dst = getattr(lib, f"pa_{suffix}_int8"), getattr(lib, f"pa_{suffix}_fp8")
        dst.argtypes, dst.restype = src.argtypes, src.restype
    lib.pa_write_kv_varlen.argtypes = [dims_p, _P, _P, _P, _P, _P, _P, _P, _P]
    lib.pa_write_kv_varlen.restype = ctypes.c_int
    lib.pa_prefill.argtypes = [dims_p, _P, _P, _P, _P, _P, _P, ctypes.c_float, _P, _P]
    lib.pa_prefill.restype = ctypes.c_int
    lib.pa_check_prefill_host.argtypes = [dims_p, _P, _P, _P]
    lib.pa_check_prefill_host.restype = ctypes.c_int
    lib.pa_check_inputs_host.argtypes = [dims_p, _P, _P, _P]
    lib.pa_check_inputs_host.restype = ctypes.c_int
    lib.pa_status_string.argtypes = [ctypes.c_int]
    lib.pa_status_string.restype = ctypes.c_char_p
    lib.pa_abi_version.argtypes = []
    lib.pa_abi_version.restype = ctypes.c_int
    if lib.pa_abi_version() != ABI_VERSION:
        raise RuntimeError(f"libpa.so ABI {lib.pa_abi_version()} != binding ABI {ABI_VERSION}; rebuild")
    if path == LIB_PATH:
        _lib = lib
    return lib


def _check(lib, func: str, status: int):
    if status != 0:
        raise PaError(func, status, lib.pa_status_string(status).decode())


def dtype_code(dtype) -> int:
    import torch

    if dtype == torch.float32:
        return PA_F32
    if dtype == torch.bfloat16:
        return PA_BF16
    if dtype == torch.int8:
        return PA_INT8
    if dtype == torch.float8_e4m3fn:
        return PA_FP8_E4M3
    raise TypeError(f"unsupported dtype {dtype}; use float32 or bfloat16 (int8 for quantised pools)")


def _stream_handle(stream, device):
    import torch

    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


def _require(cond: bool, msg: str):
    if not cond:
        raise ValueError(msg)


def _check_tensors(**tensors):
    devs = {t.device for t in tensors.values()}
    _require(len(devs) == 1, f"all tensors must share one device, got {devs}")
    dev = next(iter(devs))
    _require(dev.type == "cuda", "tensors must live on the GPU")
    for name, t in tensors.items():
        _require(t.is_contiguous(), f"{name} must be contiguous")
    return dev


def make_dims(q, k_pool, block_tables, *, out_dtype=None, variant: int = VARIANT_AUTO,
              split_schedule: int = SPLIT_AUTO) -> PaDims:
    """Dims for q ``[B, T, Hq, D]``, pools ``[N, Hkv, b, D]`` and tables ``[B, MB]``."""
    _require(q.dim() == 4 and k_pool.dim() == 4 and block_tables.dim() == 2, "bad tensor ranks")
    b, t, hq, d = q.shape
    n, hkv, bs, d2 = k_pool.shape
    _require(d == d2, "head_dim of q and pools differ")
    _require(block_tables.shape[0] == b, "block_tables rows != num_seqs")
    return PaDims(b, t, hq, hkv, d, bs, n, block_tables.shape[1], dtype_code(q.dtype), dtype_code(k_pool.dtype),
                  dtype_code(out_dtype if out_dtype is not None else q.dtype), int(variant), int(split_schedule))


def write_kv(k_new, v_new, k_pool, v_pool, block_tables, positions, *, stream=None):
    """``pa_write_kv``: scatter ``k_new``/``v_new [B, T, Hkv, D]`` into the pools at ``positions [B, T]``."""
    import torch

    lib = load_library()
    dev = _check_tensors(k_new=k_new, v_new=v_new, k_pool=k_pool, v_pool=v_pool, block_tables=block_tables,
                         positions=positions)
    _require(block_tables.dtype == torch.int32 and positions.dtype == torch.int32, "tables/positions must be int32")
    _require(k_new.shape == v_new.shape and k_pool.shape == v_pool.shape, "K/V shapes differ")
    bsz, t, hkv, d = k_new.shape
    _require(positions.shape == (bsz, t), "positions must be [B, T]")
    _require(k_pool.shape[1] == hkv and k_pool.shape[3] == d, "pool and new rows disagree")
    code = dtype_code(k_pool.dtype)
    _require(dtype_code(k_new.dtype) == code, "new rows and pools must share a dtype")
    dims = PaDims(bsz, t, hkv, hkv, d, k_pool.shape[2], k_pool.shape[0], block_tables.shape[1], code, code, code, 0, 0)
    st = lib.pa_write_kv(ctypes.byref(dims), k_new.data_ptr(), v_new.data_ptr(), k_pool.data_ptr(),
                         v_pool.data_ptr(), block_tables.data_ptr(), positions.data_ptr(),
                         _stream_handle(stream, dev))
    _check(lib, "pa_write_kv", st)


def decode(q, k_pool, v_pool, block_tables, seq_lens, scale: float, out=None, *, out_dtype=None,
           variant: int = VARIANT_AUTO, stream=None):
    """``pa_decode``: returns ``out [B, T, Hq, D]`` (fp32 unless ``out``/``out_dtype`` says otherwise)."""
    import torch

    lib = load_library()
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype or torch.float32, device=q.device)
    dev = _check_tensors(q=q, k_pool=k_pool, v_pool=v_pool, block_tables=block_tables, seq_lens=seq_lens, out=out)
    _require(block_tables.dtype == torch.int32 and seq_lens.dtype == torch.int32, "tables/seq_lens must be int32")
    _require(out.shape == q.shape and k_pool.shape == v_pool.shape, "shape mismatch")
    dims = make_dims(q, k_pool, block_tables, out_dtype=out.dtype, variant=variant)
    st = lib.pa_decode(ctypes.byref(dims), q.data_ptr(), k_pool.data_ptr(), v_pool.data_ptr(),
                       block_tables.data_ptr(), seq_lens.data_ptr(), float(scale), out.data_ptr(),
                       _stream_handle(stream, dev))
    _check(lib, "pa_decode", st)
    return out


def workspace_bytes(q, k_pool, block_tables, max_seq_len: int, partition_tokens: int,
                    *, variant: int = VARIANT_AUTO, split_schedule: int = SPLIT_AUTO) -> int:
    """``pa_decode_partitioned_workspace_bytes`` for these tensors (twice the slots when
    ``split_schedule`` asks for balanced ranges)."""
    lib = load_library()
    dims = make_dims(q, k_pool, block_tables, variant=variant, split_schedule=split_schedule)
    n = lib.pa_decode_partitioned_workspace_bytes(ctypes.byref(dims), int(max_seq_len), int(partition_tokens))
    if n == 0:
        raise PaError("pa_decode_partitioned_workspace_bytes", -1, "invalid argument")
    return int(n)


def split_schedule(q, k_pool, block_tables, max_seq_len: int, partition_tokens: int, *,
                   force: int = SPLIT_AUTO) -> int:
    """``pa_decode_partitioned_schedule``: the split schedule (1 one partition per wave, 2 two, 3 balanced
    ranges) a split call with these tensors runs on the matrix-core kernels (``force`` is
    ``pa_dims.split_schedule``)."""
    lib = load_library()
    dims = make_dims(q, k_pool, block_tables, split_schedule=force)
    n = lib.pa_decode_partitioned_schedule(ctypes.byref(dims), int(max_seq_len), int(partition_tokens))
    if n < 0:
        raise PaError("pa_decode_partitioned_schedule", n, "invalid argument" if n == -1 else "unsupported")
    return int(n)


def decode_partitioned(q, k_pool, v_pool, block_tables, seq_lens, scale: float, max_seq_len: int,
                       partition_tokens: int, out=None, workspace=None, *, out_dtype=None,
                       variant: int = VARIANT_AUTO, split_schedule: int = SPLIT_AUTO, stream=None):
    """``pa_decode_partitioned``: split-context decode + merge. ``workspace`` is a uint8 device tensor
    of at least :func:`workspace_bytes` bytes (allocated here if omitted); ``split_schedule`` is
    ``pa_dims.split_schedule`` (0: the library's choice)."""
    import torch

    lib = load_library()
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype or torch.float32, device=q.device)
    need = workspace_bytes(q, k_pool, block_tables, max_seq_len, partition_tokens, variant=variant,
                           split_schedule=split_schedule)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    dev = _check_tensors(q=q, k_pool=k_pool, v_pool=v_pool, block_tables=block_tables, seq_lens=seq_lens, out=out,
                         workspace=workspace)
    _require(block_tables.dtype == torch.int32 and seq_lens.dtype == torch.int32, "tables/seq_lens must be int32")
    _require(out.shape == q.shape and k_pool.shape == v_pool.shape, "shape mismatch")
    dims = make_dims(q, k_pool, block_tables, out_dtype=out.dtype, variant=variant, split_schedule=split_schedule)
    st = lib.pa_decode_partitioned(ctypes.byref(dims), q.data_ptr(), k_pool.data_ptr(), v_pool.data_ptr(),
                                   block_tables.data_ptr(), seq_lens.data_ptr(), float(scale), out.data_ptr(),
                                   int(max_seq_len), int(partition_tokens), workspace.data_ptr(),
                                   workspace.numel() * workspace.element_size(), _stream_handle(stream, dev))
    _check(lib, "pa_decode_partitioned", st)
    return out


def decode_partitioned_noalloc(q, k_pool, v_pool, block_tables, seq_lens, scale: float, max_seq_len: int,
                               partition_tokens: int, out, *, variant: int = VARIANT_AUTO,
                               split_schedule: int = SPLIT_AUTO, stream=None):
    """``pa_decode_partitioned_noalloc``: split-context decode + merge with the partials in the library's
    fixed device scratch (no workspace, no allocation). ``out`` must be given: nothing is allocated here
    either. Calls that overlap on one GPU race on the scratch."""
    import torch

    lib = load_library()
    dev = _check_tensors(q=q, k_pool=k_pool, v_pool=v_pool, block_tables=block_tables, seq_lens=seq_lens, out=out)
    _require(block_tables.dtype == torch.int32 and seq_lens.dtype == torch.int32, "tables/seq_lens must be int32")
    _require(out.shape == q.shape and k_pool.shape == v_pool.shape, "shape mismatch")
    dims = make_dims(q, k_pool, block_tables, out_dtype=out.dtype, variant=variant, split_schedule=split_schedule)
    st = lib.pa_decode_partitioned_noalloc(ctypes.byref(dims), q.data_ptr(), k_pool.data_ptr(), v_pool.data_ptr(),
                                           block_tables.data_ptr(), seq_lens.data_ptr(), float(scale), out.data_ptr(),
                                           int(max_seq_len), int(partition_tokens), _stream_handle(stream, dev))
    _check(lib, "pa_decode_partitioned_noalloc", st)
    return out


# ----------------------------------------------------------------------------- cascade over a shared prefix

def cascade_workspace_bytes(q, k_pool, block_tables, prefix_tokens: int, max_seq_len: int,
                            partition_tokens: int) -> int:
    """``pa_decode_cascade_workspace_bytes`` for these tensors."""
    lib = load_library()
    dims = make_dims(q, k_pool, block_tables)
    n = lib.pa_decode_cascade_workspace_bytes(ctypes.byref(dims), int(prefix_tokens), int(max_seq_len),
                                              int(partition_tokens))
    if n == 0:
        raise PaError("pa_decode_cascade_workspace_bytes", -1, "invalid argument")
    return int(n)


def decode_cascade(q, k_pool, v_pool, block_tables, seq_lens, scale: float, prefix_tokens: int, max_seq_len: int,
                   partition_tokens: int, out=None, workspace=None, *, out_dtype=None, stream=None):
    """``pa_decode_cascade``: decode where every sequence shares its first ``prefix_tokens`` positions
    (the same physical blocks); the prefix is attended once per kv head for all sequences."""
    import torch

    lib = load_library()
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype or torch.float32, device=q.device)
    need = cascade_workspace_bytes(q, k_pool, block_tables, prefix_tokens, max_seq_len, partition_tokens)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    dev = _check_tensors(q=q, k_pool=k_pool, v_pool=v_pool, block_tables=block_tables, seq_lens=seq_lens, out=out,
                         workspace=workspace)
    _require(block_tables.dtype == torch.int32 and seq_lens.dtype == torch.int32, "tables/seq_lens must be int32")
    _require(out.shape == q.shape and k_pool.shape == v_pool.shape, "shape mismatch")
    dims = make_dims(q, k_pool, block_tables, out_dtype=out.dtype)
    st = lib.pa_decode_cascade(ctypes.byref(dims), q.data_ptr(), k_pool.data_ptr(), v_pool.data_ptr(),
                               block_tables.data_ptr(), seq_lens.data_ptr(), float(scale), out.data_ptr(),
                               int(prefix_tokens), int(max_seq_len), int(partition_tokens), workspace.data_ptr(),
                               workspace.numel() * workspace.element_size(), _stream_handle(stream, dev))
    _check(lib, "pa_decode_cascade", st)
    return out


def write_kv_decode_cascade(q, k_new, v_new, k_pool, v_pool, block_tables, seq_lens, scale: float, prefix_tokens: int,
                            max_seq_len: int, partition_tokens: int, out=None, workspace=None, *, out_dtype=None,
                            stream=None):
    """``pa_write_kv_decode_cascade``: the step's KV append and the cascade decode in the same launches."""
    import torch

    lib = load_library()
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype or torch.float32, device=q.device)
    need = cascade_workspace_bytes(q, k_pool, block_tables, prefix_tokens, max_seq_len, partition_tokens)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    dev = _check_tensors(q=q, k_new=k_new, v_new=v_new, k_pool=k_pool, v_pool=v_pool, block_tables=block_tables,
                         seq_lens=seq_lens, out=out, workspace=workspace)
    _require(block_tables.dtype == torch.int32 and seq_lens.dtype == torch.int32, "tables/seq_lens must be int32")
    _require(out.shape == q.shape and k_pool.shape == v_pool.shape and k_new.shape == v_new.shape, "shape mismatch")
    dims = make_dims(q, k_pool, block_tables, out_dtype=out.dtype)
    st = lib.pa_write_kv_decode_cascade(ctypes.byref(dims), q.data_ptr(), k_new.data_ptr(), v_new.data_ptr(),
                                        k_pool.data_ptr(), v_pool.data_ptr(), block_tables.data_ptr(),
                                        seq_lens.data_ptr(), float(scale), out.data_ptr(), int(prefix_tokens),
                                        int(max_seq_len), int(partition_tokens), workspace.data_ptr(),
                                        workspace.numel() * workspace.element_size(), _stream_handle(stream, dev))
    _check(lib, "pa_write_kv_decode_cascade", st)
    return out


# ----------------------------------------------------------------------------- fused append + decode

def write_kv_decode(q, k_new, v_new, k_pool, v_pool, block_tables, seq_lens, scale: float, out=None, *,
                    max_seq_len: int | None = None, partition_tokens: int | None = None, workspace=None,
                    out_dtype=None, variant: int = VARIANT_AUTO, split_schedule: int = SPLIT_AUTO, stream=None):
    """``pa_write_kv_decode`` (or ``pa_write_kv_decode_partitioned`` when ``partition_tokens`` is
    given): append ``k_new``/``v_new [B, T, Hkv, D]`` at each sequence's last T positions and decode,
    in one launch. Returns ``out``."""
    import torch

    lib = load_library()
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype or torch.float32, device=q.device)
    tensors = dict(q=q, k_new=k_new, v_new=v_new, k_pool=k_pool, v_pool=v_pool, block_tables=block_tables,
                   seq_lens=seq_lens, out=out)
    split = partition_tokens is not None
    if split:
        need = workspace_bytes(q, k_pool, block_tables, max_seq_len, partition_tokens, variant=variant,
                               split_schedule=split_schedule)
        if workspace is None:
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
        tensors["workspace"] = workspace
    dev = _check_tensors(**tensors)
    _require(block_tables.dtype == torch.int32 and seq_lens.dtype == torch.int32, "tables/seq_lens must be int32")
    _require(out.shape == q.shape and k_pool.shape == v_pool.shape and k_new.shape == v_new.shape, "shape mismatch")
    _require(k_new.dtype == q.dtype and k_pool.dtype == q.dtype, "q, new rows and pools must share a dtype")
    dims = make_dims(q, k_pool, block_tables, out_dtype=out.dtype, variant=variant, split_schedule=split_schedule)
    args = [ctypes.byref(dims), q.data_ptr(), k_new.data_ptr(), v_new.data_ptr(), k_pool.data_ptr(),
            v_pool.data_ptr(), block_tables.data_ptr(), seq_lens.data_ptr(), float(scale), out.data_ptr()]
    if split:
        st = lib.pa_write_kv_decode_partitioned(*args, int(max_seq_len), int(partition_tokens), workspace.data_ptr(),
                                                workspace.numel() * workspace.element_size(),
                                                _stream_handle(stream, dev))
        _check(lib, "pa_write_kv_decode_partitioned", st)
    else:
        st = lib.pa_write_kv_decode(*args, _stream_handle(stream, dev))
        _check(lib, "pa_write_kv_decode", st)
    return out


# ----------------------------------------------------------------------------- 8-bit pools (int8, FP8)

def _q8_format(k_pool, fmt: str):
    import torch

    if fmt == "int8":
        _require(k_pool.dtype == torch.int8, "int8 entry points take int8 pools")
        return PA_INT8
    _require(k_pool.dtype in (torch.float8_e4m3fn, torch.uint8), "fp8 entry points take float8_e4m3fn (or uint8) pools")
    return PA_FP8_E4M3


def _check_scales(k_pool, scales):
    import torch

    want = tuple(k_pool.shape[:2]) + (2,)
    _require(tuple(scales.shape) == want, "scales must be [N, Hkv, 2] (K scale, V scale)")
    _require(scales.dtype == torch.float32, "scales must be float32")


def _write_kv_q8(fmt, k_new, v_new, k_pool, v_pool, scales, block_tables, positions, stream):
    import torch

    lib = load_library()
    kv_code = _q8_format(k_pool, fmt)
    dev = _check_tensors(k_new=k_new, v_new=v_new, k_pool=k_pool, v_pool=v_pool, scales=scales,
                         block_tables=block_tables, positions=positions)
    _check_scales(k_pool, scales)
    _require(block_tables.dtype == torch.int32 and positions.dtype == torch.int32, "tables/positions must be int32")
    _require(k_new.shape == v_new.shape and k_pool.shape == v_pool.shape, "K/V shapes differ")
    bsz, t, hkv, d = k_new.shape
    _require(positions.shape == (bsz, t), "positions must be [B, T]")
    _require(k_pool.shape[1] == hkv and k_pool.shape[3] == d, "pool and new rows disagree")
    code = dtype_code(k_new.dtype)
    dims = PaDims(bsz, t, hkv, hkv, d, k_pool.shape[2], k_pool.shape[0], block_tables.shape[1], code, kv_code,
                  code, 0, 0)
    func = "pa_write_kv_int8" if fmt == "int8" else "pa_write_kv_fp8"
    st = getattr(lib, func)(ctypes.byref(dims), k_new.data_ptr(), v_new.data_ptr(), k_pool.data_ptr(),
                            v_pool.data_ptr(), scales.data_ptr(), block_tables.data_ptr(), positions.data_ptr(),
                            _stream_handle(stream, dev))
    _check(lib, func, st)


def _decode_q8(fmt, q, k_pool, v_pool, scales, block_tables, seq_lens, scale, out, out_dtype, stream, split=None,
               split_schedule=SPLIT_AUTO):
    import torch

    lib = load_library()
    kv_code = _q8_format(k_pool, fmt)
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype or torch.float32, device=q.device)
    tensors = dict(q=q, k_pool=k_pool, v_pool=v_pool, scales=scales, block_tables=block_tables, seq_lens=seq_lens,
                   out=out)
    if split is not None:
        max_seq_len, partition_tokens, workspace = split
        if workspace is None:
            need = workspace_bytes(q, k_pool.view(torch.int8), block_tables, max_seq_len, partition_tokens,
                                   split_schedule=split_schedule)
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
        tensors["workspace"] = workspace
    dev = _check_tensors(**tensors)
    _check_scales(k_pool, scales)
    _require(block_tables.dtype == torch.int32 and seq_lens.dtype == torch.int32, "tables/seq_lens must be int32")
    _require(out.shape == q.shape and k_pool.shape == v_pool.shape, "shape mismatch")
    dims = make_dims(q, k_pool.view(torch.int8), block_tables, out_dtype=out.dtype, split_schedule=split_schedule)
    dims.kv_dtype = kv_code
    args = [ctypes.byref(dims), q.data_ptr(), k_pool.data_ptr(), v_pool.data_ptr(), scales.data_ptr(),
            block_tables.data_ptr(), seq_lens.data_ptr(), float(scale), out.data_ptr()]
    if split is None:
        func = "pa_decode_int8" if fmt == "int8" else "pa_decode_fp8"
        st = getattr(lib, func)(*args, _stream_handle(stream, dev))
    else:
        func = "pa_decode_partitioned_int8" if fmt == "int8" else "pa_decode_partitioned_fp8"
        st = getattr(lib, func)(*args, int(max_seq_len), int(partition_tokens), workspace.data_ptr(),
                                workspace.numel() * workspace.element_size(), _stream_handle(stream, dev))
    _check(lib, func, st)
    return out


def write_kv_int8(k_new, v_new, k_pool, v_pool, scales, block_tables, positions, *, stream=None):
    """``pa_write_kv_int8``: append ``k_new``/``v_new [B, T, Hkv, D]`` (bf16 or fp32) into int8 pools
    ``[N, Hkv, b, D]`` with per-(block, kv head) scale pairs ``scales [N, Hkv, 2]`` (updated in place)."""
    _write_kv_q8("int8", k_new, v_new, k_pool, v_pool, scales, block_tables, positions, stream)


def decode_int8(q, k_pool, v_pool, scales, block_tables, seq_lens, scale: float, out=None, *, out_dtype=None,
                stream=None):
    """``pa_decode_int8``: decode over int8 pools; returns ``out [B, T, Hq, D]`` (fp32 by default)."""
    return _decode_q8("int8", q, k_pool, v_pool, scales, block_tables, seq_lens, scale, out, out_dtype, stream)


def decode_partitioned_int8(q, k_pool, v_pool, scales, block_tables, seq_lens, scale: float, max_seq_len: int,
                            partition_tokens: int, out=None, workspace=None, *, out_dtype=None,
                            split_schedule: int = SPLIT_AUTO, stream=None):
    """``pa_decode_partitioned_int8``: split-context decode + merge over int8 pools."""
    return _decode_q8("int8", q, k_pool, v_pool, scales, block_tables, seq_lens, scale, out, out_dtype, stream,
                      (max_seq_len, partition_tokens, workspace), split_schedule)


def write_kv_fp8(k_new, v_new, k_pool, v_pool, scales, block_tables, positions, *, stream=None):
    """``pa_write_kv_fp8``: append into E4M3 pools (``torch.float8_e4m3fn`` or their uint8 bits)."""
    _write_kv_q8("fp8", k_new, v_new, k_pool, v_pool, scales, block_tables, positions, stream)


def decode_fp8(q, k_pool, v_pool, scales, block_tables, seq_lens, scale: float, out=None, *, out_dtype=None,
               stream=None):
    """``pa_decode_fp8``: decode over E4M3 pools; returns ``out [B, T, Hq, D]`` (fp32 by default)."""
    return _decode_q8("fp8", q, k_pool, v_pool, scales, block_tables, seq_lens, scale, out, out_dtype, stream)


def decode_partitioned_fp8(q, k_pool, v_pool, scales, block_tables, seq_lens, scale: float, max_seq_len: int,
                           partition_tokens: int, out=None, workspace=None, *, out_dtype=None,
                           split_schedule: int = SPLIT_AUTO, stream=None):
    """``pa_decode_partitioned_fp8``: split-context decode + merge over E4M3 pools."""
    return _decode_q8("fp8", q, k_pool, v_pool, scales, block_tables, seq_lens, scale, out, out_dtype, stream,
                      (max_seq_len, partition_tokens, workspace), split_schedule)


# ----------------------------------------------------------------------------- paged prefill

def _prefill_dims(q_rows, k_pool, block_tables, max_chunk: int, num_q_heads: int, code_q, code_out) -> PaDims:
    n, hkv, bs, d = k_pool.shape
    return PaDims(block_tables.shape[0], int(max_chunk), num_q_heads, hkv, d, bs, n, block_tables.shape[1], code_q,
                  dtype_code(k_pool.dtype), code_out, 0, 0)


def write_kv_varlen(k_new, v_new, k_pool, v_pool, block_tables, seq_lens, q_start, max_chunk: int, *, stream=None):
    """``pa_write_kv_varlen``: store packed chunk rows ``k_new``/``v_new [Q, Hkv, D]`` at positions
    ``L_i - n_i .. L_i - 1`` (``n_i = q_start[i+1] - q_start[i]``, at most ``max_chunk``)."""
    import torch

    lib = load_library()
    dev = _check_tensors(k_new=k_new, v_new=v_new, k_pool=k_pool, v_pool=v_pool, block_tables=block_tables,
                         seq_lens=seq_lens, q_start=q_start)
    _require(all(t.dtype == torch.int32 for t in (block_tables, seq_lens, q_start)), "index arrays must be int32")
    _require(k_new.shape == v_new.shape and k_pool.shape == v_pool.shape, "K/V shapes differ")
    _require(k_new.dim() == 3 and k_new.shape[1:] == (k_pool.shape[1], k_pool.shape[3]), "new rows must be [Q, Hkv, D]")
    _require(q_start.shape == (block_tables.shape[0] + 1,) and seq_lens.shape == (block_tables.shape[0],),
             "q_start must be [B + 1] and seq_lens [B]")
    code = dtype_code(k_pool.dtype)
    _require(dtype_code(k_new.dtype) == code, "new rows and pools must share a dtype")
    dims = _prefill_dims(k_new, k_pool, block_tables, max(1, int(max_chunk)), k_pool.shape[1], code, code)
    st = lib.pa_write_kv_varlen(ctypes.byref(dims), k_new.data_ptr(), v_new.data_ptr(), k_pool.data_ptr(),
                                v_pool.data_ptr(), block_tables.data_ptr(), seq_lens.data_ptr(), q_start.data_ptr(),
                                _stream_handle(stream, dev))
    _check(lib, "pa_write_kv_varlen", st)


def prefill(q, k_pool, v_pool, block_tables, seq_lens, q_start, scale: float, max_chunk: int, out=None, *,
            out_dtype=None, stream=None):
    """``pa_prefill``: causal attention of packed chunk rows ``q [Q, Hq, D]`` over their sequences'
    paged history and chunk; returns ``out [Q, Hq, D]`` (fp32 unless ``out``/``out_dtype`` says otherwise)."""
    import torch

    lib = load_library()
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype or torch.float32, device=q.device)
    dev = _check_tensors(q=q, k_pool=k_pool, v_pool=v_pool, block_tables=block_tables, seq_lens=seq_lens,
                         q_start=q_start, out=out)
    _require(all(t.dtype == torch.int32 for t in (block_tables, seq_lens, q_start)), "index arrays must be int32")
    _require(q.dim() == 3 and out.shape == q.shape and k_pool.shape == v_pool.shape, "shape mismatch")
    _require(q.shape[2] == k_pool.shape[3], "head_dim of q and pools differ")
    _require(q_start.shape == (block_tables.shape[0] + 1,) and seq_lens.shape == (block_tables.shape[0],),
             "q_start must be [B + 1] and seq_lens [B]")
    dims = _prefill_dims(q, k_pool, block_tables, max(1, int(max_chunk)), q.shape[1], dtype_code(q.dtype),
                         dtype_code(out.dtype))
    st = lib.pa_prefill(ctypes.byref(dims), q.data_ptr(), k_pool.data_ptr(), v_pool.data_ptr(),
                        block_tables.data_ptr(), seq_lens.data_ptr(), q_start.data_ptr(), float(scale),
                        out.data_ptr(), _stream_handle(stream, dev))
    _check(lib, "pa_prefill", st)
    return out
