"""Pins of the FP8 (E4M3) KV oracle against torch's float8_e4m3fn dtype (a library definition of the
OCP format: every code's value, and its float32 -> E4M3 cast, round to nearest even), closed forms of
the format (largest finite 448, smallest normal 2^-6, smallest subnormal 2^-9, ties to even), error
bounds of the per-block quantiser, the append rules, and planted mistakes."""

from __future__ import annotations

import importlib

import numpy as np
import pytest
import torch

import oracle
from oracle import pa_oracle_fp8 as F

FP8 = torch.float8_e4m3fn


def _torch_values():
    return torch.arange(256, dtype=torch.int32).to(torch.uint8).view(FP8).to(torch.float64).numpy()


def _torch_encode(y):
    return torch.from_numpy(np.asarray(y, dtype=np.float32)).to(FP8).view(torch.uint8).numpy()


def test_code_values_match_torch():
    mine, ref = F.e4m3_values(), _torch_values()
    assert np.array_equal(np.isnan(mine), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(mine[ok], ref[ok])
    assert np.array_equal(np.isnan(mine).nonzero()[0], [0x7F, 0xFF])


def test_format_closed_forms():
    enc = lambda v: int(F.encode_e4m3(np.float32(v)))  # noqa: E731
    assert enc(448.0) == 0x7E and enc(-448.0) == 0xFE
    assert enc(2.0 ** -6) == 0x08 and enc(2.0 ** -9) == 0x01
    assert enc(1.0) == 0x38 and enc(-2.0) == 0xC0
    # ties go to the even code: 1 + 1/16 sits halfway between 1 (0x38) and 1.125 (0x39)
    assert enc(1.0 + 1 / 16) == 0x38 and enc(1.125 + 1 / 16) == 0x3A
    assert enc(2.0 ** -10) == 0x00 and enc(3 * 2.0 ** -10) == 0x02  # subnormal ties
    assert enc(1000.0) == 0x7E  # saturated
    assert enc(-0.0) == 0x80 and enc(-(2.0 ** -12)) == 0x80  # the sign survives a round to zero


def test_encoder_matches_torch_cast():
    rng = np.random.default_rng(5)
    mags = np.exp(rng.uniform(np.log(2.0 ** -12), np.log(448.0), 20000))
    ys = (mags * rng.choice([-1.0, 1.0], mags.size)).astype(np.float32)
    vals = F.e4m3_values()[:127]
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)  # exact ties
    ys = np.concatenate([ys, mids, -mids, vals.astype(np.float32)])
    assert np.array_equal(F.encode_e4m3(ys), _torch_encode(ys))


def test_quantiser_error_bounds():
    rng = np.random.default_rng(6)
    for scale_pow in (-8, 0, 3):
        x = (rng.standard_normal((16, 128)) * 2.0 ** scale_pow).astype(np.float32)
        codes, s = F.quantize_block_fp8(x)
        back = F.e4m3_values()[codes] * float(s)
        err = np.abs(back - x)
        amax = np.abs(x).max()
        assert np.abs(back).max() == pytest.approx(amax, rel=1e-6)  # the extreme maps to +-448
        assert (np.abs(F.e4m3_values()[codes]) <= 448).all()
        normal = np.abs(x) >= 2.0 ** -6 * float(s)
        assert (err[normal] <= 2.0 ** -4 * np.abs(x[normal]) * (1 + 1e-6)).all()  # half an ulp of 3 bits
        assert (err[~normal] <= 2.0 ** -10 * float(s) * (1 + 1e-6)).all()


def test_zero_block():
    codes, s = F.quantize_block_fp8(np.zeros((4, 8), np.float32))
    assert s == 0 and not codes.any()


def _block_case(rng, b=16, hkv=2, d=8, first_len=5, new=3, big=20.0):
    n_blocks = 3
    kc = np.zeros((n_blocks, hkv, b, d), np.uint8)
    ks = np.zeros((n_blocks, hkv), np.float32)
    old = rng.standard_normal((first_len, hkv, d)).astype(np.float32)
    for h in range(hkv):
        c, s = F.quantize_block_fp8(old[:, h])
        kc[1, h, :first_len], ks[1, h] = c, s
    rows = (rng.standard_normal((1, new, hkv, d)) * big).astype(np.float32)
    pos = np.arange(first_len, first_len + new)[None]
    tables = np.array([[1, 2]])
    return kc, ks, rows, pos, tables, old


def test_append_rescale_and_untouched():
    rng = np.random.default_rng(7)
    kc, ks, rows, pos, tables, old = _block_case(rng)
    c2, s2, _, _ = F.append_fp8(kc, ks, kc, ks, rows, rows, tables, pos, 16)
    for h in range(2):
        assert s2[1, h] == np.float32(np.float32(np.abs(rows[0, :, h]).max()) / np.float32(448))
        back = F.e4m3_values()[c2[1, h, :5]] * float(s2[1, h])
        # two roundings: the first quantisation, then the re-encoding with the larger scale, each at
        # most half an ulp (2^-4 relative) in the normal range, 2^-10 scale below it
        bound = (2.0 ** -4 + 2.0 ** -4 * (1 + 2.0 ** -4)) * np.abs(old[:, h]) + 2.0 ** -9 * float(s2[1, h])
        assert (np.abs(back - old[:, h]) <= bound * (1 + 1e-6)).all()
    assert np.array_equal(c2[0], kc[0]) and np.array_equal(c2[2], kc[2])


def test_append_in_max_first_order_equals_whole_block():
    rng = np.random.default_rng(8)
    x = rng.standard_normal((16, 2, 8)).astype(np.float32)
    x[0] = np.sign(x[0]) * 9.0  # the first row holds each head's largest magnitude
    kc = np.zeros((2, 2, 16, 8), np.uint8)
    ks = np.zeros((2, 2), np.float32)
    tables = np.array([[1]])
    for t in range(16):
        kc, ks, _, _ = F.append_fp8(kc, ks, kc, ks, x[None, t:t + 1], x[None, t:t + 1], tables, np.array([[t]]), 16)
    for h in range(2):
        codes, s = F.quantize_block_fp8(x[:, h])
        assert ks[1, h] == s and np.array_equal(kc[1, h], codes)


def test_decode_fp8_is_decode_of_the_torch_dequantised_pool():
    """Codes read through torch's float8_e4m3fn dtype, times power-of-two scales, are exact float
    pools; fp8 decode must equal the pinned float decode on them."""
    rng = np.random.default_rng(9)
    n, hkv, b, d = 6, 2, 4, 8
    kc = rng.integers(0, 256, (n, hkv, b, d)).astype(np.uint8)
    vc = rng.integers(0, 256, (n, hkv, b, d)).astype(np.uint8)
    kc[(kc & 0x7F) == 0x7F] = 0x38  # no NaN codes
    vc[(vc & 0x7F) == 0x7F] = 0x38
    ks = (2.0 ** rng.integers(-8, -4, (n, hkv))).astype(np.float32)
    vs = (2.0 ** rng.integers(-3, 0, (n, hkv))).astype(np.float32)
    kf = torch.from_numpy(kc).view(FP8).to(torch.float64).numpy() * ks[:, :, None, None]
    vf = torch.from_numpy(vc).view(FP8).to(torch.float64).numpy() * vs[:, :, None, None]
    q = rng.standard_normal((2, 1, 4, d))
    tables = np.array([[0, 3, 5], [1, 2, 4]])
    lens = np.array([11, 7])
    got = F.decode_fp8(q, kc, ks, vc, vs, tables, lens, 0.3, b)
    assert np.array_equal(got, oracle.decode(q, kf, vf, tables, lens, 0.3, b))


def test_decode_row_fp8_equals_decode_fp8_row_by_row():
    """Every output row of the one-row oracle equals the same row of the whole-batch oracle (itself
    pinned above to the float decode of torch's dequantisation). Scales differ per (block, kv head),
    and two query tokens per sequence read two kv heads across several blocks, so a row that took
    another head's or another block's scale would differ."""
    rng = np.random.default_rng(21)
    n, hkv, b, d, T = 7, 2, 4, 8, 2
    kc = rng.integers(0, 256, (n, hkv, b, d)).astype(np.uint8)
    vc = rng.integers(0, 256, (n, hkv, b, d)).astype(np.uint8)
    kc[(kc & 0x7F) == 0x7F] = 0x30
    vc[(vc & 0x7F) == 0x7F] = 0x30
    ks = rng.uniform(0.01, 0.05, (n, hkv)).astype(np.float32)
    vs = rng.uniform(0.5, 2.0, (n, hkv)).astype(np.float32)
    q = rng.standard_normal((2, T, 4, d))
    tables = np.array([[6, 0, 3, 5], [1, 2, 4, 0]])
    lens = np.array([14, 9])
    whole = F.decode_fp8(q, kc, ks, vc, vs, tables, lens, 0.4, b)
    for i in range(2):
        for t in range(T):
            for h in range(4):
                row = F.decode_row_fp8(q, kc, ks, vc, vs, tables, lens, 0.4, b, i, t, h)
                np.testing.assert_allclose(row, whole[i, t, h], rtol=0, atol=1e-13)


def _pins_fail(mod) -> bool:
    tests = [test_format_closed_forms, test_encoder_matches_torch_cast, test_quantiser_error_bounds,
             test_append_rescale_and_untouched, test_append_in_max_first_order_equals_whole_block,
             test_decode_fp8_is_decode_of_the_torch_dequantised_pool, test_code_values_match_torch,
             test_decode_row_fp8_equals_decode_fp8_row_by_row]
    global F
    saved = F
    F = mod
    try:
        for t in tests:
            try:
                t()
            except (AssertionError, Exception):
                return True
        return False
    finally:
        F = saved


def test_planted_mistakes_are_caught():
    assert not _pins_fail(F)

    def fresh():
        spec = importlib.util.find_spec("oracle.pa_oracle_fp8")
        mod = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(mod)
        return mod

    mutants = {}
    m = fresh()  # int8's constant in the scale
    m.E4M3_MAX = 127.0
    mutants["scale-over-127"] = m

    m = fresh()  # ties away from zero
    vals = m.e4m3_values()[:127]
    def enc_away(y):
        y = np.asarray(y, dtype=np.float32)
        a = np.minimum(np.abs(y.astype(np.float64)), 448.0)
        hi = np.searchsorted(vals, a, side="left").clip(0, 126)
        lo = np.maximum(hi - 1, 0)
        code = np.where(vals[hi] - a <= a - vals[lo], hi, lo).astype(np.uint8)
        return np.where(np.signbit(y), code | 0x80, code).astype(np.uint8)
    m.encode_e4m3 = enc_away
    mutants["ties-away"] = m

    m = fresh()  # exponent bias 8 (values halved)
    orig = m.e4m3_values
    m.e4m3_values = lambda: orig() / 2
    m._VALUES = m.e4m3_values()
    m._POS = m._VALUES[:127]
    mutants["bias-8"] = m

    m = fresh()  # old codes keep their bits when the scale grows
    m._reencode = lambda codes, old, new: np.array(codes, dtype=np.uint8)
    mutants["no-reencode"] = m

    m = fresh()  # sign dropped
    orig_enc = m.encode_e4m3
    m.encode_e4m3 = lambda y: orig_enc(np.abs(np.asarray(y, dtype=np.float32)))
    mutants["no-sign"] = m

    m = fresh()  # the one-row oracle reads the scale of the neighbouring kv head
    class OtherHead(m._LazyDequantFp8):
        def __getitem__(self, idx):
            blocks, head, offsets, sl = idx
            values = m._VALUES[np.asarray(self.codes[blocks, head, offsets, sl], dtype=np.uint8)]
            other = (head + 1) % self.scales.shape[1]
            return values * np.asarray(self.scales[blocks, other], dtype=np.float64)[..., None]
    m._LazyDequantFp8 = OtherHead
    mutants["row-scale-other-head"] = m

    m = fresh()  # the one-row oracle reads every position's scale from the row's first block
    class FirstBlock(m._LazyDequantFp8):
        def __getitem__(self, idx):
            blocks, head, offsets, sl = idx
            values = m._VALUES[np.asarray(self.codes[blocks, head, offsets, sl], dtype=np.uint8)]
            first = np.full_like(np.asarray(blocks), np.asarray(blocks).reshape(-1)[0])
            return values * np.asarray(self.scales[first, head], dtype=np.float64)[..., None]
    m._LazyDequantFp8 = FirstBlock
    mutants["row-scale-first-block"] = m

    for name, mod in mutants.items():
        assert _pins_fail(mod), f"planted mistake '{name}' was not caught by the pins"
