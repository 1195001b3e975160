"""The C-ABI library loads on a CPU-only host, exports every symbol include/pa.h
declares, and rejects bad arguments before touching the GPU."""

from __future__ import annotations

import ctypes
import os
import re

import pytest

import paged_kv_cache_69_amd as pa

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "pa.h")


def _declared_functions():
    text = open(HEADER, encoding="utf-8").read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pa_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(pa.LIB_PATH):
        pytest.fail("libpa.so is not built: run __graft_entry__.build() first")
    return pa.load_library()


def test_header_declares_the_abi():
    assert _declared_functions() == sorted(pa.EXPORTS)


def test_every_declared_symbol_is_exported(lib):
    for name in _declared_functions():
        assert hasattr(lib, name), name


def test_pa_dims_layout_matches_header():
    text = open(HEADER, encoding="utf-8").read()
    body = re.search(r"typedef struct \{(.*?)\} pa_dims;", text, flags=re.S).group(1)
    fields = re.findall(r"int32_t\s+(\w+);", re.sub(r"/\*.*?\*/", "", body))
    assert tuple(fields) == tuple(name for name, _ in pa.PaDims._fields_)
    assert ctypes.sizeof(pa.PaDims) == 4 * len(fields)


def test_status_strings_and_version(lib):
    assert lib.pa_abi_version() == pa.ABI_VERSION
    assert lib.pa_status_string(0) == b"ok"
    assert lib.pa_status_string(-1) == b"invalid argument"
    assert lib.pa_status_string(-2) == b"unsupported shape or dtype"
    assert lib.pa_status_string(-3) == b"kernel launch failed"
    assert lib.pa_status_string(12345) == b"unknown status"


def _dims(**kw):
    base = dict(num_seqs=4, q_tokens=1, num_q_heads=32, num_kv_heads=8, head_dim=128, block_size=16,
                num_blocks=100, max_blocks_per_seq=8, q_dtype=pa.PA_BF16, kv_dtype=pa.PA_BF16,
                out_dtype=pa.PA_F32, variant=0, split_schedule=0)
    base.update(kw)
    return pa.PaDims(*[base[n] for n, _ in pa.PaDims._fields_])


FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: every case below fails validation first


@pytest.mark.parametrize("kw,status", [
    (dict(num_q_heads=30), -1),          # Hq % Hkv != 0
    (dict(q_tokens=0), -1),
    (dict(head_dim=0), -1),
    (dict(kv_dtype=7), -1),
    (dict(variant=9), -1),
    (dict(q_dtype=pa.PA_F32), -2),       # q and KV dtypes differ
    (dict(head_dim=96), -2),             # no kernel for this head_dim
    (dict(block_size=64), -2),
    (dict(split_schedule=4), -1),
    (dict(split_schedule=-1), -1),
])
def test_decode_rejects_bad_dims(lib, kw, status):
    d = _dims(**kw)
    st = lib.pa_decode(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, 0.1, FAKE, None)
    assert st == status


def test_null_pointers_rejected(lib):
    d = _dims()
    assert lib.pa_decode(None, FAKE, FAKE, FAKE, FAKE, FAKE, 0.1, FAKE, None) == -1
    assert lib.pa_decode(ctypes.byref(d), None, FAKE, FAKE, FAKE, FAKE, 0.1, FAKE, None) == -1
    assert lib.pa_write_kv(ctypes.byref(d), FAKE, None, FAKE, FAKE, FAKE, FAKE, None) == -1
    assert lib.pa_decode(ctypes.byref(d), ctypes.c_void_p(0x1004), FAKE, FAKE, FAKE, FAKE, 0.1, FAKE, None) == -1
    assert lib.pa_decode(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, float("nan"), FAKE, None) == -1


def test_empty_batch_is_a_no_op(lib):
    d = _dims(num_seqs=0)
    assert lib.pa_decode(ctypes.byref(d), None, None, None, None, None, 0.1, None, None) == 0
    assert lib.pa_write_kv(ctypes.byref(d), None, None, None, None, None, None, None) == 0


def test_partitioned_workspace_arithmetic(lib):
    """rows = 16 * 32 = 512; P = ceil(32768 / 512) = 64 partitions: 2P + 2 slots and 16 int32 slot counts when
    the call runs balanced ranges (asked for, or chosen: 16 * 8 * 64 > 2048 partitions), one slot per
    partition otherwise; 32 query rows per kv head allow no balanced ranges: one slot per partition."""
    align = lambda x: (x + 255) // 256 * 256  # noqa: E731
    for sched, slots, counts in ((0, 130, align(16 * 4)), (1, 64, 0), (2, 64, 0), (3, 130, align(16 * 4))):
        d = _dims(num_seqs=16, q_tokens=1, num_q_heads=32, head_dim=128, split_schedule=sched)
        want = align(512 * slots * 2 * 4) + align(512 * slots * 128 * 4) + counts
        assert lib.pa_decode_partitioned_workspace_bytes(ctypes.byref(d), 32768, 512) == want
    d32 = _dims(num_seqs=16, q_tokens=4, num_q_heads=64, head_dim=128, split_schedule=3)
    rows32 = 16 * 4 * 64
    want32 = align(rows32 * 64 * 2 * 4) + align(rows32 * 64 * 128 * 4)
    assert lib.pa_decode_partitioned_workspace_bytes(ctypes.byref(d32), 32768, 512) == want32
    d = _dims(num_seqs=16, q_tokens=1, num_q_heads=32, head_dim=128)
    # a small split (16 * 8 * 16 = 2048 partitions, one resident round) keeps one slot per partition
    assert lib.pa_decode_partitioned_workspace_bytes(ctypes.byref(d), 16 * 512, 512) == \
        align(512 * 16 * 2 * 4) + align(512 * 16 * 128 * 4)
    assert lib.pa_decode_partitioned_workspace_bytes(ctypes.byref(d), 0, 512) == 0
    assert lib.pa_decode_partitioned_workspace_bytes(None, 10, 512) == 0


def test_partitioned_schedule_choice(lib):
    """PA_SPLIT_AUTO, once B * Hkv * ceil(max_seq_len / partition_tokens) > 2048: balanced ranges where the
    dims allow them, else two partitions per wave (bf16 pools, <= 16 rows per kv head); one otherwise."""
    d = _dims(num_seqs=16, q_tokens=1, num_q_heads=32, head_dim=128)
    assert d.num_kv_heads == 8
    f = lambda dd, msl, pt: lib.pa_decode_partitioned_schedule(ctypes.byref(dd), msl, pt)  # noqa: E731
    assert f(d, 32768, 512) == pa.SPLIT_BALANCED      # 16 * 8 * 64 = 8192 partitions
    assert f(d, 16 * 512, 512) == pa.SPLIT_ONE_PER_WAVE  # 16 * 8 * 16 = 2048: one round already
    assert f(d, 16 * 512 + 1, 512) == pa.SPLIT_BALANCED
    d_b8 = _dims(num_seqs=16, q_tokens=1, num_q_heads=32, head_dim=128, block_size=8)  # b = 8: no balanced
    assert f(d_b8, 32768, 512) == pa.SPLIT_TWO_PER_WAVE
    assert f(d, 0, 512) == -1 and f(d, 100, 0) == -1
    assert lib.pa_decode_partitioned_schedule(None, 100, 512) == -1
    d32 = _dims(num_seqs=16, q_tokens=4, num_q_heads=64, head_dim=128)  # 32 rows per kv head
    assert f(d32, 32768, 512) == pa.SPLIT_ONE_PER_WAVE
    for code in (pa.PA_INT8, pa.PA_FP8_E4M3):  # 8-bit pools: balanced, else one partition per wave
        d8 = _dims(num_seqs=16, q_tokens=1, num_q_heads=32, head_dim=128, kv_dtype=code)
        assert f(d8, 32768, 512) == pa.SPLIT_BALANCED
        assert f(_dims(num_seqs=16, q_tokens=1, num_q_heads=32, head_dim=128, kv_dtype=code, block_size=8),
                 32768, 512) == pa.SPLIT_ONE_PER_WAVE
    big_b = _dims(num_seqs=1100, q_tokens=1, num_q_heads=32, head_dim=128, split_schedule=3)  # too many to stage
    assert f(big_b, 4096, 512) == -2
    # q rows staged in 48 KiB of LDS: 48 sequences of 4 rows (256 bytes each) fit, 49 do not, and the
    # automatic choice then takes two partitions per wave
    assert f(_dims(num_seqs=48, q_tokens=1, num_q_heads=32, head_dim=128, split_schedule=3), 32768, 512) == 3
    assert f(_dims(num_seqs=49, q_tokens=1, num_q_heads=32, head_dim=128, split_schedule=3), 32768, 512) == -2
    assert f(_dims(num_seqs=49, q_tokens=1, num_q_heads=32, head_dim=128), 32768, 512) == pa.SPLIT_TWO_PER_WAVE
    d_b8 = _dims(num_seqs=16, q_tokens=1, num_q_heads=32, head_dim=128, block_size=8, split_schedule=3)
    assert f(d_b8, 32768, 512) == -2


def test_partitioned_schedule_override(lib, monkeypatch):
    """pa_dims.split_schedule forces a schedule; two per wave falls back to one where it does not exist; a
    forced balanced schedule the dims do not allow is PA_ERR_UNSUPPORTED; no environment variable changes
    anything."""
    f = lambda d: lib.pa_decode_partitioned_schedule(ctypes.byref(d), 32768, 512)  # noqa: E731
    base = dict(num_seqs=16, q_tokens=1, num_q_heads=32, head_dim=128)
    assert f(_dims(**base, split_schedule=1)) == 1
    assert f(_dims(**base, split_schedule=2)) == 2
    assert f(_dims(**base, split_schedule=3)) == 3
    assert f(_dims(num_seqs=1, q_tokens=1, num_q_heads=32, head_dim=128, split_schedule=3)) == 3
    monkeypatch.setenv("PA_SPLIT_WAVE_PARTS", "1")  # the variable of an earlier version: no effect
    assert f(_dims(**base, split_schedule=0)) == 3
    for code in (pa.PA_INT8, pa.PA_FP8_E4M3):
        assert f(_dims(**base, kv_dtype=code, split_schedule=2)) == 1
    assert f(_dims(num_seqs=16, q_tokens=4, num_q_heads=64, head_dim=128, split_schedule=2)) == 1
    assert f(_dims(num_seqs=16, q_tokens=4, num_q_heads=64, head_dim=128, split_schedule=3)) == -2
    assert f(_dims(split_schedule=5)) == -1


def test_fused_cascade_refuses_missing_rows(lib):
    d = _dims()
    ws = ctypes.c_void_p(0x100000)
    call = lambda kn, vn, n=10**9: lib.pa_write_kv_decode_cascade(  # noqa: E731
        ctypes.byref(d), FAKE, kn, vn, FAKE, FAKE, FAKE, FAKE, 0.1, FAKE, 32, 1000, 512, ws, n, None)
    assert call(None, FAKE) == -1 and call(FAKE, None) == -1
    assert call(ctypes.c_void_p(0x1008), FAKE) == -1  # k_new not 16-byte aligned
    d0 = _dims(num_seqs=0)  # an empty batch is a no-op
    assert lib.pa_write_kv_decode_cascade(ctypes.byref(d0), None, None, None, None, None, None, None, 0.1, None, 0, 1,
                                          16, None, 0, None) == 0


def test_partitioned_rejects_bad_partitions(lib):
    d = _dims()
    ws = ctypes.c_void_p(0x100000)
    need = lib.pa_decode_partitioned_workspace_bytes(ctypes.byref(d), 1000, 512)
    call = lambda pt, nbytes, w=ws: lib.pa_decode_partitioned(  # noqa: E731
        ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, 0.1, FAKE, 1000, pt, w, nbytes, None)
    assert call(24, 10**9) == -1        # not a multiple of 16
    assert call(512, need - 1) == -1    # workspace too small
    assert call(512, need, ctypes.c_void_p(0x100010)) == -1  # workspace not 256-byte aligned
    assert call(0, 10**9) == -1


def test_write_kv_rejects_unaligned_rows(lib):
    d = _dims(head_dim=6, kv_dtype=pa.PA_BF16)  # 12-byte rows cannot be copied in 16-byte chunks
    assert lib.pa_write_kv(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == -2


# ----------------------------------------------------------------------------- PA_CHECK preconditions

def _np_ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def _check_case():
    """b = 4, N = 10 blocks, MB = 3, two sequences of lengths 6 and 9 (2 and 3 blocks), T = 2."""
    import numpy as np

    d = _dims(num_seqs=2, q_tokens=2, num_q_heads=4, num_kv_heads=2, head_dim=64, block_size=4, num_blocks=10,
              max_blocks_per_seq=3, q_dtype=pa.PA_F32, kv_dtype=pa.PA_F32)
    tables = np.array([[5, 1, 2**31 - 1], [7, 0, 9]], dtype=np.int32)
    lens = np.array([6, 9], dtype=np.int32)
    pos = np.array([[4, 5], [7, 8]], dtype=np.int32)
    return d, tables, lens, pos


def test_check_inputs_accepts_valid(lib):
    d, tables, lens, pos = _check_case()
    assert lib.pa_check_inputs_host(ctypes.byref(d), _np_ptr(tables), _np_ptr(lens), _np_ptr(pos)) == 0
    assert lib.pa_check_inputs_host(ctypes.byref(d), _np_ptr(tables), None, None) == 0


@pytest.mark.parametrize("what", ["len_below_T", "len_past_table", "entry_negative", "entry_past_pool",
                                  "pos_negative", "pos_past_table", "slot_twice", "pos_block_invalid"])
def test_check_inputs_rejects(lib, what):
    d, tables, lens, pos = _check_case()
    if what == "len_below_T":
        lens[0] = 1
    elif what == "len_past_table":
        lens[1] = 13              # MB * b = 12
    elif what == "entry_negative":
        tables[1, 2] = -1         # used: ceil(9 / 4) = 3 entries
    elif what == "entry_past_pool":
        tables[0, 1] = 10
    elif what == "pos_negative":
        pos[0, 0] = -1
    elif what == "pos_past_table":
        pos[1, 1] = 12
    elif what == "slot_twice":
        tables[1, 1] = 5          # sequence 1 position 7 -> block 5 offset 3; make it collide below
        pos[0, 1] = 7 - 4         # sequence 0 position 3 -> block 5 offset 3
        lens[1] = 6
    elif what == "pos_block_invalid":
        pos[0, 1] = 9             # block index 2 of sequence 0 is padding
    assert lib.pa_check_inputs_host(ctypes.byref(d), _np_ptr(tables), _np_ptr(lens), _np_ptr(pos)) == -1


def test_check_inputs_padding_past_length_is_ignored(lib):
    d, tables, lens, pos = _check_case()
    tables[0, 2] = -5             # sequence 0 uses 2 entries only
    assert lib.pa_check_inputs_host(ctypes.byref(d), _np_ptr(tables), _np_ptr(lens), None) == 0


def test_library_binds_to_torchs_hip_runtime():
    """Loading libpa.so in a fresh process before anything imported torch still leaves one HIP runtime
    in the process: the binding imports torch first, so libpa.so binds to torch's copy."""
    import subprocess
    import sys

    code = ("import paged_kv_cache_69_amd as pa; pa.load_library(); "
            "maps = open('/proc/self/maps').read().splitlines(); "
            "print(len({l.split()[-1] for l in maps if l.split()[-1].endswith('libamdhip64.so.7') "
            "or 'libamdhip64.so' in l.split()[-1].rsplit('/', 1)[-1]}))")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, cwd=root, timeout=300)
    assert out.returncode == 0, out.stderr
    assert out.stdout.strip() == "1"


def test_timeline_entry_points_only_in_the_timeline_build():
    """libpa.so exports no timeline entry point (the records exist only in the measurement build); the
    timeline build, when present, exports the two that include/pa_timeline.h declares and the whole
    decode ABI besides."""
    import re
    import subprocess

    from paged_kv_cache_69_amd._build import LIB_PATH, TIMELINE_LIB_PATH

    def exported(path):
        out = subprocess.run(["nm", "-D", "--defined-only", path], capture_output=True, text=True, check=True).stdout
        return {ln.split()[-1] for ln in out.splitlines() if ln.strip()}

    assert not any(s.startswith("pa_timeline") for s in exported(LIB_PATH))
    if not os.path.exists(TIMELINE_LIB_PATH):
        pytest.skip("timeline build not present (python -m paged_kv_cache_69_amd._build --timeline)")
    header = open(os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "pa_timeline.h")).read()
    declared = set(re.findall(r"\b(pa_timeline_[a-z]+)\s*\(", re.sub(r"/\*.*?\*/", "", header, flags=re.S)))
    assert declared == {"pa_timeline_read", "pa_timeline_clear"}
    syms = exported(TIMELINE_LIB_PATH)
    assert declared <= syms
    assert {s for s in exported(LIB_PATH) if s.startswith("pa_")} <= syms
