"""Float64 CPU oracle for the FP8 (E4M3) KV cache with one scale per (block, kv head).

TEST INFRASTRUCTURE ONLY (see the package docstring): no product code imports it.

[P2] "Модуль 09: PagedAttention: пейджинг KV-кэша", §6, names FP8 E4M3 beside
int8 as the per-block, per-head KV format that halves the cache at no visible
quality cost, and [P1] "Attention that reads through the table" lists FP8 KV
caches among what production paged kernels add. The pages give int8's scale
rule (largest magnitude over the code range) and leave FP8's to the reader.

Readings taken:

* E4M3 is the OCP 8-bit format with 1 sign, 4 exponent (bias 7) and 3 mantissa
  bits, no infinities, NaN at S.1111.111, largest finite 448 = 1.75 * 2^8,
  subnormals m * 2^-9.
* Per (block, kv head): scale = max|x| / 448 in float32, the int8 rule with
  E4M3's largest finite value in place of 127; code = E4M3(x / scale), the
  quotient in float32, rounded to the nearest E4M3 value with ties to the even
  code (mantissa LSB 0), saturated at +-448. A sign is kept on codes that round
  to zero (-0 is 0x80).
* Appending to a partly filled block follows the int8 oracle: the scale grows to
  the larger of the old scale and the new rows' max / 448; when it grows, old
  codes are re-encoded from (value(code) * old_scale) / new_scale in float32.
* Decode is ordinary attention over the dequantised values value(code) * scale.
"""

from __future__ import annotations

import numpy as np

from .pa_oracle import decode, decode_row

__all__ = ["E4M3_MAX", "e4m3_values", "encode_e4m3", "quantize_block_fp8", "dequantize_pool_fp8",
           "append_fp8", "decode_fp8", "decode_row_fp8"]

E4M3_MAX = 448.0
_F32 = np.float32


def e4m3_values() -> np.ndarray:
    """float64 value of each of the 256 codes (NaN for 0x7F and 0xFF), from the bit fields."""
    out = np.empty(256, dtype=np.float64)
    for code in range(256):
        sign = -1.0 if code & 0x80 else 1.0
        e, m = (code >> 3) & 0xF, code & 0x7
        if e == 0xF and m == 0x7:
            out[code] = np.nan
        elif e == 0:
            out[code] = sign * m * 2.0 ** -9
        else:
            out[code] = sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return out


_VALUES = e4m3_values()
_POS = _VALUES[:127]  # codes 0 .. 126: the non-negative finite values, increasing


def encode_e4m3(y) -> np.ndarray:
    """Codes (uint8) of float32 values ``y``: nearest E4M3 value, ties to the even code, saturated at
    +-448 (brute force over the 127 non-negative values; the sign is the input's)."""
    y = np.asarray(y, dtype=_F32)
    a = np.minimum(np.abs(y.astype(np.float64)), E4M3_MAX)
    hi = np.searchsorted(_POS, a, side="left").clip(0, 126)  # first value >= a
    lo = np.maximum(hi - 1, 0)
    d_lo, d_hi = a - _POS[lo], _POS[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    return np.where(np.signbit(y), code | 0x80, code).astype(np.uint8)


def quantize_block_fp8(x):
    """Codes and scale of one (block, kv head): ``x`` is ``[n, D]``.
    Returns ``(codes uint8 [n, D], scale float32)``."""
    xf = np.asarray(x, dtype=_F32)
    amax = _F32(np.max(np.abs(xf))) if xf.size else _F32(0)
    scale = _F32(amax / _F32(E4M3_MAX))
    if scale == 0:
        return np.zeros(xf.shape, dtype=np.uint8), scale
    return encode_e4m3(xf / scale), scale


def dequantize_pool_fp8(codes, scales):
    """``codes [N, Hkv, b, D]`` uint8 and ``scales [N, Hkv]`` float32 -> float64 value(code) * scale."""
    return _VALUES[np.asarray(codes, dtype=np.uint8)] * np.asarray(scales, dtype=np.float64)[:, :, None, None]


def _reencode(codes, old_scale, new_scale):
    prod = _VALUES[np.asarray(codes, dtype=np.uint8)].astype(_F32) * _F32(old_scale)
    return encode_e4m3(prod / _F32(new_scale))


def append_fp8(k_codes, k_scales, v_codes, v_scales, k_new, v_new, block_tables, positions, block_size):
    """KV append into FP8 pools; returns new ``(k_codes, k_scales, v_codes, v_scales)``.
    Shapes as in the int8 oracle: pools ``[N, Hkv, b, D]`` uint8, scales ``[N, Hkv]`` float32, new rows
    ``[B, T, Hkv, D]``, positions ``[B, T]``."""
    from .pa_oracle import physical_slot

    out = []
    for codes, scales, new in ((k_codes, k_scales, k_new), (v_codes, v_scales, v_new)):
        c = np.array(codes, dtype=np.uint8, copy=True)
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
                    cand = _F32(_F32(np.max(np.abs(rows))) / _F32(E4M3_MAX))
                    if first > 0:
                        old = s[blk, h]
                        new_scale = max(old, cand)
                        if new_scale > old:
                            c[blk, h, :first] = _reencode(c[blk, h, :first], old, new_scale)
                    else:
                        new_scale = cand
                    for off, t in items:
                        if new_scale == 0:
                            c[blk, h, off] = 0
                        else:
                            c[blk, h, off] = encode_e4m3(newf[i, t, h] / _F32(new_scale))
                    s[blk, h] = new_scale
        out += [c, s]
    return tuple(out)


def decode_fp8(q, k_codes, k_scales, v_codes, v_scales, block_tables, seq_lens, scale, block_size):
    """Decode attention over FP8 pools: :func:`oracle.decode` on the dequantised values."""
    return decode(q, dequantize_pool_fp8(k_codes, k_scales), dequantize_pool_fp8(v_codes, v_scales), block_tables,
                  seq_lens, scale, block_size)


def decode_row_fp8(q, k_codes, k_scales, v_codes, v_scales, block_tables, seq_lens, scale, block_size, i, t, h):
    """One output row of :func:`decode_fp8` (dequantises only the blocks that row reads)."""
    return decode_row(q, _LazyDequantFp8(k_codes, k_scales), _LazyDequantFp8(v_codes, v_scales), block_tables,
                      seq_lens, scale, block_size, i, t, h)


class _LazyDequantFp8:
    """Pool view that dequantises only the rows an index expression (blocks, head, offsets, slice)
    asks for: value(code) times the scale of that row's own (block, kv head)."""

    def __init__(self, codes, scales):
        self.codes, self.scales, self.shape = codes, scales, codes.shape

    def __getitem__(self, idx):
        blocks, head, offsets, sl = idx
        values = _VALUES[np.asarray(self.codes[blocks, head, offsets, sl], dtype=np.uint8)]
        return values * np.asarray(self.scales[blocks, head], dtype=np.float64)[..., None]
