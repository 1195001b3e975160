"""Pins of the int8 KV oracle ([P2] "Модуль 09: PagedAttention", §6) against what the page and
arithmetic fix: the page's error bound and its own worked test, closed forms, exact cases, the
rounding rule, and invariants of the append rule. None of these re-derives a code the way the
oracle does."""

from __future__ import annotations

import numpy as np
import pytest

import oracle
import oracle.pa_oracle_int8

# The module under test; the planted-mistake test swaps in mutated copies.
Q = oracle.pa_oracle_int8

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def test_error_bound_range_over_254():
    """§6: per element, |code * scale - x| <= max|x| / 254 (up to float32 rounding of the scale)."""
    rng = np.random.default_rng(0)
    for amp in (1e-3, 1.0, 4.0, 300.0):
        x = (rng.standard_normal((16, 128)) * amp).astype(np.float32)
        codes, scale = Q.quantize_block(x)
        err = np.abs(codes.astype(np.float64) * float(scale) - x.astype(np.float64))
        amax = float(np.abs(x).max())
        assert err.max() <= amax / 254 * (1 + 1e-6)


def test_pages_worked_check_16x8x128():
    """§6's own check: a 16-position block of 8 heads x 128 values ~ N(0, 2^2), one scale per head,
    reconstructs with max |err| < 0.1."""
    rng = np.random.default_rng(3)
    block = rng.normal(scale=2.0, size=(16, 8, 128)).astype(np.float32)
    worst = 0.0
    for h in range(8):
        codes, scale = Q.quantize_block(block[:, h, :])
        worst = max(worst, float(np.abs(codes * np.float64(scale) - block[:, h, :]).max()))
    assert worst < 0.1


def test_scale_is_max_over_127_and_extreme_maps_to_127():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((16, 128)).astype(np.float32)
    x[3, 7] = -9.0  # the largest magnitude, negative
    codes, scale = Q.quantize_block(x)
    assert scale == np.float32(np.float32(9.0) / np.float32(127))
    assert codes[3, 7] == -127
    assert codes.min() >= -127 and codes.max() <= 127 and codes.dtype == np.int8


def test_exact_multiples_round_trip():
    """Values that are integer multiples k * s of a power-of-two scale s, with max |k| = 127, are
    stored as k exactly."""
    rng = np.random.default_rng(2)
    k = rng.integers(-127, 128, size=(16, 128))
    k[0, 0] = 127
    s = 2.0 ** -5
    codes, scale = Q.quantize_block((k * s).astype(np.float32))
    assert scale == np.float32(s)
    assert np.array_equal(codes.astype(np.int64), k)


def test_rounding_is_half_to_even():
    """With scale 1 (max |x| = 127): 2.5 -> 2, 3.5 -> 4, -2.5 -> -2, 0.5 -> 0."""
    x = np.array([[127.0, 2.5, 3.5, -2.5, 0.5, 1.5]], dtype=np.float32)
    codes, scale = Q.quantize_block(x)
    assert scale == 1.0
    assert codes.tolist() == [[127, 2, 4, -2, 0, 2]]


def test_zero_block():
    codes, scale = Q.quantize_block(np.zeros((16, 128), dtype=np.float32))
    assert scale == 0 and not codes.any()


def _pool(n_blocks=6, hkv=2, b=16, d=128, seed=0):
    rng = np.random.default_rng(seed)
    codes = rng.integers(-127, 128, size=(n_blocks, hkv, b, d)).astype(np.int8)
    scales = rng.uniform(0.01, 0.05, size=(n_blocks, hkv)).astype(np.float32)
    return codes, scales


def test_append_in_max_first_order_equals_whole_block_quantisation():
    """If a block's first row already holds its largest magnitude, appending the b rows one by one
    never raises the scale, so the block ends exactly as quantising all b rows at once."""
    rng = np.random.default_rng(4)
    b, d, hkv = 16, 128, 2
    rows = rng.standard_normal((b, hkv, d)).astype(np.float32)
    rows[0, :, 5] = 50.0
    kc, ks = _pool(1, hkv, b, d)
    vc, vs = kc.copy(), ks.copy()
    tables = np.array([[0]], dtype=np.int32)
    for p in range(b):
        new = rows[p][None, None]
        kc, ks, vc, vs = Q.append_int8(kc, ks, vc, vs, new, new, tables, np.array([[p]], dtype=np.int32), b)
    for h in range(hkv):
        codes, scale = Q.quantize_block(rows[:, h, :])
        assert ks[0, h] == scale and np.array_equal(kc[0, h], codes)
        assert vs[0, h] == scale and np.array_equal(vc[0, h], codes)


def test_append_rescale_bounds_and_untouched_slots():
    """A new row larger than the block's range raises the scale to its max / 127; the re-quantised old
    rows stay within half a new step of their old values; slots past the new row, other kv heads' data
    of other blocks, and other blocks are untouched."""
    rng = np.random.default_rng(5)
    b, d, hkv = 16, 128, 2
    kc, ks = _pool(4, hkv, b, d, seed=6)
    vc, vs = _pool(4, hkv, b, d, seed=7)
    tables = np.array([[2, 0]], dtype=np.int32)
    pos = np.array([[16 + 9]], dtype=np.int32)           # block 0, offset 9: rows 0..8 are valid
    new_k = (rng.standard_normal((1, 1, hkv, d)) * 10).astype(np.float32)
    new_v = (rng.standard_normal((1, 1, hkv, d)) * 1e-3).astype(np.float32)  # smaller: V scale stays
    kc2, ks2, vc2, vs2 = Q.append_int8(kc, ks, vc, vs, new_k, new_v, tables, pos, b)
    for h in range(hkv):
        cand = np.float32(np.float32(np.abs(new_k[0, 0, h]).max()) / np.float32(127))
        assert ks2[0, h] == max(ks[0, h], cand) > ks[0, h]
        old = kc[0, h, :9].astype(np.float64) * np.float64(ks[0, h])
        new = kc2[0, h, :9].astype(np.float64) * np.float64(ks2[0, h])
        assert np.abs(new - old).max() <= float(ks2[0, h]) / 2 * (1 + 1e-5)
        assert np.abs(kc2[0, h, 9] * np.float64(ks2[0, h]) - new_k[0, 0, h]).max() <= float(ks2[0, h]) / 2 * (1 + 1e-5)
        assert vs2[0, h] == vs[0, h] and np.array_equal(vc2[0, h, :9], vc[0, h, :9])
    assert np.array_equal(kc2[0, :, 10:], kc[0, :, 10:]) and np.array_equal(vc2[0, :, 10:], vc[0, :, 10:])
    for blk in (1, 2, 3):
        assert np.array_equal(kc2[blk], kc[blk]) and np.array_equal(ks2[blk], ks[blk])


def test_append_to_fresh_block_ignores_stale_scale():
    """Offset 0: the block holds no valid rows, so a stale scale (even a huge one) has no effect."""
    rng = np.random.default_rng(8)
    b, d, hkv = 16, 128, 2
    kc, ks = _pool(3, hkv, b, d, seed=9)
    new = rng.standard_normal((1, 1, hkv, d)).astype(np.float32)
    tables = np.array([[1, 2]], dtype=np.int32)
    pos = np.array([[16]], dtype=np.int32)                # block 2, offset 0
    a = Q.append_int8(kc, ks, kc, ks, new, new, tables, pos, b)
    ks_big = ks.copy()
    ks_big[2] = 1e30
    c = Q.append_int8(kc, ks_big, kc, ks_big, new, new, tables, pos, b)
    for x, y in zip(a, c):
        assert np.array_equal(x, y)
    for h in range(hkv):
        codes, scale = Q.quantize_block(new[0, 0, h][None])
        assert a[1][2, h] == scale and np.array_equal(a[0][2, h, 0], codes[0])


def test_multi_token_append_spanning_two_blocks():
    """T = 4 rows at positions 14..17 (b = 16): two rows close block 0 (rescaling its 14 old rows if
    needed), two open block 1 (fresh). Each block's scale covers exactly its own new rows."""
    rng = np.random.default_rng(10)
    b, d, hkv = 16, 128, 1
    kc, ks = _pool(2, hkv, b, d, seed=11)
    new = (rng.standard_normal((1, 4, hkv, d)) * 5).astype(np.float32)
    tables = np.array([[0, 1]], dtype=np.int32)
    pos = np.array([[14, 15, 16, 17]], dtype=np.int32)
    k2, s2, _, _ = Q.append_int8(kc, ks, kc, ks, new, new, tables, pos, b)
    c0 = np.float32(np.float32(np.abs(new[0, :2]).max()) / np.float32(127))
    c1 = np.float32(np.float32(np.abs(new[0, 2:]).max()) / np.float32(127))
    assert s2[0, 0] == max(ks[0, 0], c0)
    assert s2[1, 0] == c1
    assert np.array_equal(k2[1, 0, 2:], kc[1, 0, 2:])


def test_decode_int8_is_decode_of_dequantised_pool():
    """With codes from exact multiples of power-of-two scales, the int8 pools hold exactly the values
    of a float pool; int8 decode then equals float decode of that pool (pinned in test_oracle.py)."""
    rng = np.random.default_rng(12)
    n, hkv, b, d = 5, 2, 16, 64
    codes = rng.integers(-127, 128, size=(n, hkv, b, d)).astype(np.int8)
    scales = (2.0 ** -rng.integers(3, 8, size=(n, hkv))).astype(np.float32)
    vals = codes.astype(np.float64) * scales[:, :, None, None]
    q = rng.standard_normal((2, 1, 4, d))
    tables = np.array([[0, 3, 4], [1, 2, 0]], dtype=np.int32)
    lens = np.array([40, 20], dtype=np.int32)
    got = Q.decode_int8(q, codes, scales, codes, scales, tables, lens, 0.125, b)
    want = oracle.decode(q, vals, vals, tables, lens, 0.125, b)
    assert np.array_equal(got, want)
    np.testing.assert_allclose(Q.dequantize_pool(codes, scales), vals, rtol=0, atol=0)
    row = Q.decode_row_int8(q, codes, scales, codes, scales, tables, lens, 0.125, b, 1, 0, 3)
    np.testing.assert_allclose(row, want[1, 0, 3], rtol=0, atol=1e-14)


def test_planted_mistakes_are_caught():
    """Plausible mistakes planted in copies of the int8 oracle each fail at least one pin above."""
    import importlib

    global Q
    pins = [f for name, f in sorted(globals().items())
            if name.startswith("test_") and name != "test_planted_mistakes_are_caught"]

    def fresh():
        spec = importlib.util.find_spec("oracle.pa_oracle_int8")
        mod = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(mod)
        return mod

    def failures(mod):
        global Q
        Q = mod
        bad = []
        try:
            for f in pins:
                try:
                    f()
                except AssertionError:
                    bad.append(f.__name__)
        finally:
            Q = oracle.pa_oracle_int8
        return bad

    assert failures(oracle.pa_oracle_int8) == []
    F32 = np.float32
    mutants = {}

    m = fresh()  # divides by 128 instead of 127
    def q128(x):
        xf = np.asarray(x, dtype=F32)
        s = F32(F32(np.abs(xf).max()) / F32(128))
        return (np.clip(np.rint(xf / s), -127, 127).astype(np.int8) if s else np.zeros(xf.shape, np.int8)), s
    m.quantize_block = q128
    mutants["scale-over-128"] = m

    m = fresh()  # rounds half away from zero
    def qaway(x):
        xf = np.asarray(x, dtype=F32)
        s = F32(F32(np.abs(xf).max()) / F32(127))
        if not s:
            return np.zeros(xf.shape, np.int8), s
        y = xf / s
        return np.clip(np.sign(y) * np.floor(np.abs(y) + F32(0.5)), -127, 127).astype(np.int8), s
    m.quantize_block = qaway
    mutants["round-half-away"] = m

    m = fresh()  # old rows keep their codes when the scale grows
    m._requantize = lambda codes, old, new: np.array(codes, dtype=np.int8)
    mutants["no-requantise"] = m

    m = fresh()  # a fresh block still takes max(old, new)
    orig = m.append_int8
    def sticky(kc, ks, vc, vs, kn, vn, tables, pos, b):
        big = lambda s: np.maximum(s, F32(0))  # noqa: E731
        out = orig(kc, ks, vc, vs, kn, vn, tables, pos, b)
        k2, s2, v2, sv2 = [np.array(a, copy=True) for a in out]
        for i in range(pos.shape[0]):
            for t in range(pos.shape[1]):
                blk = int(tables[i][int(pos[i, t]) // b])
                if int(pos[i, t]) % b == 0:
                    s2[blk] = np.maximum(s2[blk], big(ks[blk]))
        return k2, s2, v2, sv2
    m.append_int8 = sticky
    mutants["fresh-block-keeps-old-scale"] = m

    m = fresh()  # one scale for all kv heads of a block (max over heads)
    orig2 = m.append_int8
    def head_shared(kc, ks, vc, vs, kn, vn, tables, pos, b):
        k2, s2, v2, sv2 = orig2(kc, ks, vc, vs, kn, vn, tables, pos, b)
        s2 = np.repeat(s2.max(axis=1, keepdims=True), s2.shape[1], axis=1)
        return k2, s2, v2, sv2
    m.append_int8 = head_shared
    mutants["scale-shared-by-heads"] = m

    m = fresh()  # dequantised with the scale of the wrong kv head
    m.dequantize_pool = lambda codes, scales: (np.asarray(codes, np.float64)
                                               * np.asarray(scales, np.float64)[:, ::-1, None, None])
    mutants["dequant-head-swapped"] = m

    for name, mod in mutants.items():
        assert failures(mod), f"planted mistake '{name}' was not caught by the pins"
