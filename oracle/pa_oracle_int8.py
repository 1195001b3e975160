"""Float64 CPU oracle for the int8 KV cache with one scale per (block, kv head).

TEST INFRASTRUCTURE ONLY (see the package docstring): no product code imports it.

[P2] "Модуль 09: PagedAttention: пейджинг KV-кэша", §6 (block-wise KV
quantisation), defines the format. For every block and kv head, the scale is
the largest magnitude among that head's values in the block, divided by 127.
A value is stored as its quotient by the scale, rounded and clipped to
[-127, 127], and read back as code times scale. The error per element is then
at most the range over 254. The page notes the benefit of per-block scales: a
new token can only change its own block's scale, never the whole sequence's.

Readings taken where the page leaves a step open:

* The codes are decided in float32, as in the page's own listing: the scale is
  the float32 quotient amax / 127, and each code is the float32 quotient
  x / scale, rounded half to even (numpy's and IEEE's default rounding), then
  clipped.
* A head whose values in the block are all zero gets scale 0 and codes 0.
* Appending new rows to a block that already holds m valid rows (m > 0):
  the new scale is the larger of the old scale and (largest new magnitude) /
  127. When it grows, the m old codes are re-quantised: code' =
  clip(round((code * old_scale) / new_scale)), each product and quotient in
  float32. The new rows are then quantised with the new scale. A block whose
  first new row lands at offset 0 holds no valid rows, so its old scale is
  ignored.
* Decode attention over such a pool is ordinary attention over the
  dequantised values code * scale, widened to float64.
"""

from __future__ import annotations

import numpy as np

from .pa_oracle import decode, decode_row, physical_slot

__all__ = ["quantize_block", "dequantize_pool", "append_int8", "decode_int8", "decode_row_int8"]

_F32 = np.float32


def quantize_block(x):
    """Codes and scale of one (block, kv head): ``x`` is ``[n, D]`` (any float dtype).

    Returns ``(codes int8 [n, D], scale float32)``: scale = max|x| / 127 and
    code = clip(round_half_even(x / scale), -127, 127), both in float32.
    """
    xf = np.asarray(x, dtype=_F32)
    amax = _F32(np.max(np.abs(xf))) if xf.size else _F32(0)
    scale = _F32(amax / _F32(127))
    if scale == 0:
        return np.zeros(xf.shape, dtype=np.int8), scale
    codes = np.clip(np.rint(xf / scale), -127, 127).astype(np.int8)
    return codes, scale


def dequantize_pool(codes, scales):
    """``codes [N, Hkv, b, D]`` int8 and ``scales [N, Hkv]`` float32 -> float64 code * scale."""
    return np.asarray(codes, dtype=np.float64) * np.asarray(scales, dtype=np.float64)[:, :, None, None]


def _requantize(codes, old_scale, new_scale):
    prod = np.asarray(codes, dtype=_F32) * _F32(old_scale)
    return np.clip(np.rint(prod / _F32(new_scale)), -127, 127).astype(np.int8)


def append_int8(k_codes, k_scales, v_codes, v_scales, k_new, v_new, block_tables, positions, block_size):
    """KV append into int8 pools; returns new ``(k_codes, k_scales, v_codes, v_scales)``.

    For every sequence i, the new rows of ``k_new[i, :, h]`` / ``v_new[i, :, h]``
    (``[B, T, Hkv, D]``) go to the slots of ``positions[i, :]`` (consecutive, as
    in a decode step), block by block, with the re-scaling rule of the module
    docstring. Pools are ``[N, Hkv, b, D]`` int8, scales ``[N, Hkv]`` float32.
    """
    out = []
    for codes, scales, new in ((k_codes, k_scales, k_new), (v_codes, v_scales, v_new)):
        c = np.array(codes, dtype=np.int8, copy=True)
        s = np.array(scales, dtype=_F32, copy=True)
        newf = np.asarray(new, dtype=_F32)
        n_seq, n_tok = positions.shape
        for i in range(n_seq):
            by_block = {}
            for t in range(n_tok):
                blk, off = physical_slot(block_tables[i], int(positions[i, t]), block_size)
                by_block.setdefault(blk, []).append((off, t))
            for blk, items in by_block.items():
                first = min(off for off, _ in items)
                for h in range(c.shape[1]):
                    rows = np.stack([newf[i, t, h] for _, t in items])
                    cand = _F32(_F32(np.max(np.abs(rows))) / _F32(127))
                    if first > 0:
                        old = s[blk, h]
                        new_scale = max(old, cand)
                        if new_scale > old:
                            c[blk, h, :first] = _requantize(c[blk, h, :first], old, new_scale)
                    else:
                        new_scale = cand
                    for off, t in items:
                        if new_scale == 0:
                            c[blk, h, off] = 0
                        else:
                            c[blk, h, off] = np.clip(np.rint(newf[i, t, h] / _F32(new_scale)), -127, 127)
                    s[blk, h] = new_scale
        out += [c, s]
    return tuple(out)


def decode_int8(q, k_codes, k_scales, v_codes, v_scales, block_tables, seq_lens, scale, block_size):
    """Decode attention over int8 pools: :func:`oracle.decode` on the dequantised values."""
    return decode(q, dequantize_pool(k_codes, k_scales), dequantize_pool(v_codes, v_scales), block_tables,
                  seq_lens, scale, block_size)


def decode_row_int8(q, k_codes, k_scales, v_codes, v_scales, block_tables, seq_lens, scale, block_size, i, t, h):
    """One output row of :func:`decode_int8` (dequantises only the blocks that row reads)."""
    kd = _LazyDequant(k_codes, k_scales)
    vd = _LazyDequant(v_codes, v_scales)
    return decode_row(q, kd, vd, block_tables, seq_lens, scale, block_size, i, t, h)


class _LazyDequant:
    """Pool view that dequantises the rows an index expression asks for (big pools, few rows)."""

    def __init__(self, codes, scales):
        self.codes, self.scales = codes, scales
        self.shape = codes.shape

    def __getitem__(self, idx):
        blocks, head, offsets, sl = idx
        return (np.asarray(self.codes[blocks, head, offsets, sl], dtype=np.float64)
                * np.asarray(self.scales[blocks, head], dtype=np.float64)[..., None])
