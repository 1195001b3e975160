"""Test-side helpers: conversions between torch tensors and the oracle's numpy arrays,
and the tail-slot poisoning that proves the kernels never read past a sequence."""

from __future__ import annotations

import numpy as np
import torch

import oracle


def to_f64(t: torch.Tensor) -> np.ndarray:
    """Exact widening of fp32/bf16 CPU tensors to float64 numpy."""
    return t.detach().to("cpu").to(torch.float64).numpy()


def to_f32_view(t: torch.Tensor) -> np.ndarray:
    """Values of an fp32 or bf16 tensor as float32 numpy, exactly; big pools stay half the size of float64."""
    return t.detach().to("cpu").to(torch.float32).numpy()


def bits(t: torch.Tensor) -> np.ndarray:
    """Raw bit pattern of a tensor as unsigned numpy integers."""
    t = t.detach().to("cpu").contiguous()
    size = t.element_size()
    signed = {1: torch.int8, 2: torch.int16, 4: torch.int32, 8: torch.int64}[size]
    unsigned = {1: np.uint8, 2: np.uint16, 4: np.uint32, 8: np.uint64}[size]
    return t.view(signed).numpy().view(unsigned)


def from_bits(arr: np.ndarray, dtype: torch.dtype) -> torch.Tensor:
    signed = {1: np.int8, 2: np.int16, 4: np.int32, 8: np.int64}[arr.dtype.itemsize]
    tdt = {1: torch.int8, 2: torch.int16, 4: torch.int32, 8: torch.int64}[arr.dtype.itemsize]
    return torch.from_numpy(np.ascontiguousarray(arr).view(signed)).view(tdt).view(dtype)


def poison_case(case, *, slots_to_write=True):
    """NaN-fill every slot of a sequence's blocks at or beyond position L (the tail of the
    last block). If ``slots_to_write``, also NaN-fill the slots the step's KV write will
    fill. The slots are located with the oracle's own scatter. Modifies ``case`` in place."""
    b = case.block_size
    n_seq, n_tok = case.positions.shape
    hkv, d = case.k_pool.shape[1], case.k_pool.shape[3]
    kp, vp = bits(case.k_pool), bits(case.v_pool)
    for i in range(n_seq):
        seq_len = int(case.seq_lens[i])
        nblk = oracle.blocks_needed(seq_len, b)
        start = seq_len - n_tok if slots_to_write else seq_len
        pos = np.arange(max(start, 0), nblk * b, dtype=np.int64)
        if pos.size == 0:
            continue
        nan_rows = bits(torch.full((1, pos.size, hkv, d), float("nan"), dtype=case.k_pool.dtype))
        kp, vp = oracle.write_kv(kp, vp, nan_rows, nan_rows, case.block_tables[i:i + 1].numpy(),
                                 pos[None, :], b)
    case.k_pool = from_bits(kp, case.k_pool.dtype).reshape(case.k_pool.shape)
    case.v_pool = from_bits(vp, case.v_pool.dtype).reshape(case.v_pool.shape)
    return case


def oracle_after_write(case):
    """The oracle's pools after the step's KV write, as numpy bit arrays."""
    return oracle.write_kv(bits(case.k_pool), bits(case.v_pool), bits(case.k_new), bits(case.v_new),
                           case.block_tables.numpy(), case.positions.numpy(), case.block_size)


def assert_attention_close(got, ref, *, kv_dtype, out_dtype, what=""):
    """The parity bar for attention outputs.

    * fp32 inputs: for every output row, max_d |got - ref| <= 1e-5 * max_d |ref| (1e-5 relative).
    * bf16 inputs (fp32 accumulation): |got - ref| <= 2e-3 elementwise, against the oracle run on
      the same bf16-rounded inputs.
    * bf16 outputs also get half a bf16 ulp of |ref| on top, the rounding of the stored result.
    """
    if isinstance(got, torch.Tensor):
        got = got.detach().cpu().double().numpy()
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    err = np.abs(got - ref)
    if out_dtype == torch.bfloat16:
        ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(ref), 1e-30))) - 7)
        extra = 0.5 * ulp
    else:
        extra = 0.0
    if kv_dtype == torch.float32:
        bound = 1e-5 * np.abs(ref).max(axis=-1, keepdims=True) + extra
    else:
        bound = 2e-3 + extra
    bad = err > bound
    assert not bad.any(), (f"{what}: {int(bad.sum())} elements out of tolerance; max err {err.max():.3e}; "
                           f"worst at {np.unravel_index(np.argmax(err - bound), err.shape)}")
    return float(err.max())
