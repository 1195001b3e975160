"""The matrix-core kernel's reference restart on 8-bit pools and on the cascade's prefix items, and int8
pools with large-magnitude queries, on the GPU.

A wave's first tile sets each row's reference max; a later score more than 2^64 above it restarts the
wave's range with the raised reference ([P5] "Chapter 7 Paged KV Cache and Memory Management", section
4.2: the output does not depend on the reference, only the rescale when the running max jumps does).
N(0, 1) data never gets there, so these cases build scores that climb by tens of base-2 units per tile:
K codes point along head_dim 0 only, and the per-(block, kv head) K scales (8-bit pools) or the K values
(the bf16 prefix) grow along the sequence. Every case is compared with the float64 oracle.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from tests.helpers import assert_attention_close, bits, oracle_after_write, to_f32_view
from workloads import build_case, fp8_pools, int8_pools

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _np_codes(t, fmt):
    return t.cpu().view(torch.uint8).numpy().view(np.int8 if fmt == "int8" else np.uint8)


def _oracle_8bit(case, fmt, kc, vc, sc):
    s = sc.cpu().numpy()
    dec = oracle.decode_int8 if fmt == "int8" else oracle.decode_fp8
    return dec(case.q.float().numpy(), _np_codes(kc, fmt), np.ascontiguousarray(s[..., 0]), _np_codes(vc, fmt),
               np.ascontiguousarray(s[..., 1]), case.block_tables.numpy(), case.seq_lens.numpy(), case.scale,
               case.block_size)


def _decode_8bit(pa, fmt, case, kc, vc, sc, pt):
    q, tab, lens = (getattr(case, k).to(DEV) for k in ("q", "block_tables", "seq_lens"))
    if pt:
        f = pa.decode_partitioned_int8 if fmt == "int8" else pa.decode_partitioned_fp8
        out = f(q, kc, vc, sc, tab, lens, case.scale, case.max_seq_len, pt)
    else:
        out = (pa.decode_int8 if fmt == "int8" else pa.decode_fp8)(q, kc, vc, sc, tab, lens, case.scale)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("fmt", ["int8", "fp8"])
@pytest.mark.parametrize("hq,t", [(32, 1), (64, 4)])
def test_8bit_reference_restarts(gpu_lib, fmt, hq, t):
    """K codes are the largest code along head_dim 0 (127, or E4M3 128.0) and zero elsewhere; block j of a
    sequence gets K scale 0.05 * j (int8) or 0.05 * 127 / 128 * j (FP8), so every K row's value is 6.35 j
    and a score climbs by about 5 base-2 units per 16-position block: a restart every dozen or so tiles,
    several inside each 512-position partition. Single pass, 512- and 64-position partitions; 16 and 32
    query rows per kv head (FP8 split waves of 16 rows run four per SIMD)."""
    lengths = [t + 30, 400, 1100, 1700]
    case = build_case(lengths=lengths, num_q_heads=hq, num_kv_heads=8, head_dim=128, block_size=16, q_tokens=t,
                      dtype=torch.bfloat16, seed=8100 + hq + t, pool_slack=0.1)
    case.q[..., 0] = (6.0 + 0.1 * case.q[..., 0].float()).to(torch.bfloat16)
    kc, vc, sc = (int8_pools if fmt == "int8" else fp8_pools)(case, seed=hq + t)
    kc.view(torch.uint8).zero_()
    if fmt == "int8":
        kc[..., 0] = 127
    else:
        kc[..., 0] = torch.tensor(128.0, dtype=torch.float8_e4m3fn)  # E4M3 code 0x70, exactly 128
    for i, L in enumerate(lengths):
        for j in range(-(-L // 16)):
            blk = int(case.block_tables[i, j])
            sc[blk, :, 0] = 0.05 * j * (1.0 if fmt == "int8" else 127.0 / 128.0)
    ref = _oracle_8bit(case, fmt, kc, vc, sc)
    g = [x.to(DEV) for x in (kc, vc, sc)]
    for pt in (None, 512, 64):
        print(f"[case] {fmt} restarts hq={hq} T={t} pt={pt}", flush=True)
        out = _decode_8bit(gpu_lib, fmt, case, *g, pt)
        assert_attention_close(out.cpu(), ref, kv_dtype=torch.int8, out_dtype=torch.float32, what=f"{fmt} pt={pt}")


@pytest.mark.parametrize("fmt", ["int8", "fp8"])
def test_8bit_large_magnitude_queries(gpu_lib, fmt):
    """q ~ N(0, 30^2) with outliers: single elements of +-5e3, +-4e4 and +-1e5 (above fp16's 65504, so
    the int8 path scales those rows by a power of two before its fp16 conversion) in some rows. Scores
    reach thousands of base-2 units, so those rows' softmax is one-hot; every row still meets the oracle."""
    case = build_case(lengths=[9, 100, 333, 700], num_q_heads=32, num_kv_heads=8, head_dim=128, block_size=16,
                      dtype=torch.bfloat16, seed=8200, pool_slack=0.1)
    gen = torch.Generator().manual_seed(8201)
    q = torch.randn(case.q.shape, generator=gen) * 30.0
    q[0, 0, 3, 7] = 5e3
    q[1, 0, 10, 100] = -4e4
    q[2, 0, 17, 0] = 1e5
    q[3, 0, 31, 127] = -1e5
    q[3, 0, 30, 5] = 1e5
    q[3, 0, 30, 6] = -7.0e4
    case.q = q.to(torch.bfloat16)
    kc, vc, sc = (int8_pools if fmt == "int8" else fp8_pools)(case, seed=55)
    ref = _oracle_8bit(case, fmt, kc, vc, sc)
    g = [x.to(DEV) for x in (kc, vc, sc)]
    for pt in (None, 128):
        print(f"[case] {fmt} large q pt={pt}", flush=True)
        out = _decode_8bit(gpu_lib, fmt, case, *g, pt)
        assert_attention_close(out.cpu(), ref, kv_dtype=torch.int8, out_dtype=torch.float32, what=f"{fmt} large q")


def test_cascade_prefix_items_restart(gpu_lib):
    """128 sequences share a 4096-position prefix, so the prefix items take 256-position chunks (16
    tiles). K points along head_dim 0 with values 16 * ((p / 16) mod 16): within every 256 positions
    the scores climb by about 12 base-2 units per tile, and the prefix waves (which start at different
    tiles of a chunk) restart several times per chunk. Suffixes are ordinary N(0, 1) rows."""
    b, prefix = 16, 4096
    gen = torch.Generator().manual_seed(8300)
    lengths = (prefix + torch.randint(1, 200, (128,), generator=gen)).tolist()
    case = build_case(lengths=lengths, num_q_heads=32, num_kv_heads=8, head_dim=128, block_size=b,
                      dtype=torch.bfloat16, seed=8301, shared_prefix_blocks=prefix // b, pool_slack=0.05)
    for j in range(prefix // b):
        blk = int(case.block_tables[0, j])
        case.k_pool[blk] = 0.0
        case.k_pool[blk, :, :, 0] = float(16 * (j % 16))
    case.q[..., 0] = (6.0 + 0.1 * case.q[..., 0].float()).to(torch.bfloat16)
    kp, vp = oracle_after_write(case)
    as_t = lambda x: torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).reshape(case.k_pool.shape)  # noqa
    ref = oracle.decode(to_f32_view(case.q), to_f32_view(as_t(kp)), to_f32_view(as_t(vp)), case.block_tables.numpy(),
                        case.seq_lens.numpy(), case.scale, b)
    g = {k: getattr(case, k).to(DEV, copy=True) for k in ("q", "k_new", "v_new", "k_pool", "v_pool", "block_tables",
                                                         "seq_lens", "positions")}
    print("[case] cascade prefix restarts", flush=True)
    out = gpu_lib.write_kv_decode_cascade(g["q"], g["k_new"], g["v_new"], g["k_pool"], g["v_pool"], g["block_tables"],
                                          g["seq_lens"], case.scale, prefix, case.max_seq_len, 256)
    torch.cuda.synchronize()
    assert np.array_equal(bits(g["k_pool"]), kp) and np.array_equal(bits(g["v_pool"]), vp)
    assert_attention_close(out.cpu(), ref, kv_dtype=torch.bfloat16, out_dtype=torch.float32, what="cascade restarts")
