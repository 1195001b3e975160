"""Fused append + decode over 8-bit pools (pa_write_kv_decode_int8 / _fp8), on the GPU.

One launch appends the step's rows into int8 or FP8 (E4M3) pools with per-(block, kv head) scales and
attends. It must equal pa_write_kv_int8 (or _fp8) followed by pa_decode_int8 (or _fp8) bit for bit: the
codes, the scales and the output. The separate calls are themselves checked against the oracle in
test_gpu_int8.py / test_gpu_fp8.py; here the fused output also meets the oracle run on the oracle's own
append. Nothing expected comes from the GPU.
"""

from __future__ import annotations

import pytest
import torch

import oracle
from tests.helpers import assert_attention_close
from workloads import build_case, fp8_pools, int8_pools, make_case

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _bits(t):
    t = t.detach().cpu().contiguous()
    return t.view(torch.int32) if t.dtype == torch.float32 else t.view(torch.uint8)


def _run_both(pa, kind, case, pools):
    """(separate, fused): each a tuple of (k codes, k scales, v codes, v scales, out) on the GPU."""
    res = []
    for fused in (False, True):
        kc, ks, vc, vs = (x.to(DEV, copy=True) for x in pools)
        q, kn, vn, tab, lens, pos = (x.to(DEV) for x in (case.q, case.k_new, case.v_new, case.block_tables,
                                                         case.seq_lens, case.positions))
        if fused:
            f = pa.write_kv_decode_int8 if kind == "int8" else pa.write_kv_decode_fp8
            out = f(q, kn, vn, kc, vc, ks, vs, tab, lens, case.scale)
        else:
            w = pa.write_kv_int8 if kind == "int8" else pa.write_kv_fp8
            d = pa.decode_int8 if kind == "int8" else pa.decode_fp8
            w(kn, vn, kc, vc, ks, vs, tab, pos)
            out = d(q, kc, vc, ks, vs, tab, lens, case.scale)
        torch.cuda.synchronize()
        res.append((kc, ks, vc, vs, out))
    return res


def _assert_same(sep, fused, what):
    for name, a, b in zip(("k codes", "k scales", "v codes", "v scales", "out"), sep, fused):
        assert torch.equal(_bits(a), _bits(b)), f"{what}: {name} differ"


@pytest.mark.parametrize("kind", ["int8", "fp8"])
@pytest.mark.parametrize("hq,hkv,t", [(32, 8, 1), (8, 2, 2), (16, 4, 3), (16, 2, 4), (64, 8, 4)])
def test_fused_8bit_append_decode_bitwise(gpu_lib, kind, hq, hkv, t):
    """New rows at offset 0 of a fresh block, in the middle of a block and (T > 1) across two blocks;
    every other sequence's new K rows (and the others' V rows) are 20x larger, so their block's scale
    grows and its old codes are re-quantised. Pools, scales and output equal the separate calls'."""
    b = 16
    lengths = sorted({max(t, x) for x in (1, 2, b - 1, b, b + 1, b + 2, 2 * b + 2, 3 * b, 47, 70, 100, 257)})
    case = build_case(lengths=lengths, num_q_heads=hq, num_kv_heads=hkv, head_dim=128, block_size=b, q_tokens=t,
                      dtype=torch.bfloat16, seed=8300 + hq + t, pool_slack=0.3)
    case.k_new[::2] *= 20
    case.v_new[1::2] *= 20
    pools = (int8_pools if kind == "int8" else fp8_pools)(case, seed=hq * 3 + t)
    print(f"[case] fused {kind} hq={hq} hkv={hkv} T={t}", flush=True)
    sep, fused = _run_both(gpu_lib, kind, case, pools)
    _assert_same(sep, fused, f"{kind} T={t}")
    # and the fused output meets the oracle on the oracle's own append
    kc, ks, vc, vs = [(x.view(torch.uint8) if x.dtype == torch.float8_e4m3fn else x).cpu().numpy() for x in pools]
    app = oracle.append_int8 if kind == "int8" else oracle.append_fp8
    dec = oracle.decode_int8 if kind == "int8" else oracle.decode_fp8
    kc2, ks2, vc2, vs2 = app(kc, ks, vc, vs, case.k_new.float().numpy(), case.v_new.float().numpy(),
                             case.block_tables.numpy(), case.positions.numpy(), b)
    ref = dec(case.q.float().numpy(), kc2, ks2, vc2, vs2, case.block_tables.numpy(), case.seq_lens.numpy(),
              case.scale, b)
    assert_attention_close(fused[4].cpu(), ref, kv_dtype=torch.int8, out_dtype=torch.float32, what=f"fused {kind}")


@pytest.mark.parametrize("kind", ["int8", "fp8"])
def test_fused_8bit_full_size_bitwise(gpu_lib, kind):
    """The batch64 workload with 8-bit pools, all 64 sequences: fused equals separate bit for bit."""
    case = make_case("batch64")
    pools = (int8_pools if kind == "int8" else fp8_pools)(case, seed=17)
    print(f"[case] fused {kind} full batch64", flush=True)
    sep, fused = _run_both(gpu_lib, kind, case, pools)
    _assert_same(sep, fused, f"{kind} batch64")


def test_fused_8bit_refuses_unsupported(gpu_lib):
    """b = 32 pools (a tile is half a block) have no fused 8-bit path: PA_ERR_UNSUPPORTED, nothing written."""
    case = build_case(lengths=[5, 40], num_q_heads=8, num_kv_heads=2, head_dim=128, block_size=32,
                      dtype=torch.bfloat16, seed=5)
    kc, ks, vc, vs = (x.to(DEV) for x in int8_pools(case, seed=3))
    before = kc.clone()
    q, kn, vn, tab, lens = (x.to(DEV) for x in (case.q, case.k_new, case.v_new, case.block_tables, case.seq_lens))
    with pytest.raises(gpu_lib.PaError) as err:
        gpu_lib.write_kv_decode_int8(q, kn, vn, kc, vc, ks, vs, tab, lens, case.scale)
    assert err.value.status == -2
    torch.cuda.synchronize()
    assert torch.equal(kc, before)
