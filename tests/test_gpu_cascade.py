"""Parity of pa_decode_cascade (a shared prefix attended once for all sequences) against the float64
oracle, on the GPU. The cascade is exact ([P5] section 4.2): the bar is the same as pa_decode's."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from tests.helpers import assert_attention_close, bits, oracle_after_write, poison_case, to_f32_view
from workloads import build_case, make_case

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _gpu(case):
    return {k: getattr(case, k).to(DEV, copy=True) for k in ("q", "k_new", "v_new", "k_pool", "v_pool",
                                                          "block_tables", "seq_lens", "positions")}


def _oracle(case, kp, vp):
    def as_t(a, like):
        return torch.from_numpy(a.view(np.int16)).view(like.dtype).reshape(like.shape)
    return oracle.decode(to_f32_view(case.q), to_f32_view(as_t(kp, case.k_pool)), to_f32_view(as_t(vp, case.v_pool)),
                         case.block_tables.numpy(), case.seq_lens.numpy(), case.scale, case.block_size)


def _step(pa, case, prefix_tokens, pt):
    g = _gpu(case)
    pa.write_kv(g["k_new"], g["v_new"], g["k_pool"], g["v_pool"], g["block_tables"], g["positions"])
    out = pa.decode_cascade(g["q"], g["k_pool"], g["v_pool"], g["block_tables"], g["seq_lens"], case.scale,
                            prefix_tokens, case.max_seq_len, pt)
    torch.cuda.synchronize()
    return g, out


def _fused_step(pa, case, prefix_tokens, pt):
    """pa_write_kv_decode_cascade on fresh copies of the inputs."""
    f = _gpu(case)
    out = pa.write_kv_decode_cascade(f["q"], f["k_new"], f["v_new"], f["k_pool"], f["v_pool"], f["block_tables"],
                                     f["seq_lens"], case.scale, prefix_tokens, case.max_seq_len, pt)
    torch.cuda.synchronize()
    return f, out


def _same_step(g, out, f, fout):
    assert torch.equal(g["k_pool"].view(torch.int16), f["k_pool"].view(torch.int16)), "fused append: K pool differs"
    assert torch.equal(g["v_pool"].view(torch.int16), f["v_pool"].view(torch.int16)), "fused append: V pool differs"
    assert torch.equal(out, fout), "fused append: output differs"


@pytest.mark.parametrize("b", [4, 8, 16, 32])
@pytest.mark.parametrize("hq,hkv,t", [(4, 4, 1), (32, 8, 1), (8, 2, 4), (64, 8, 4), (12, 4, 3)])
def test_cascade_shapes(gpu_lib, b, hq, hkv, t):
    """Shared prefixes of 1-6 blocks, suffixes from T to a few hundred positions (tails at tile and block
    boundaries), partitions that cut the prefix and that hold it whole."""
    for n_pref, pts in ((max(1, 16 // b), (16, 32)), (max(2, 96 // b), (32, 48 if 48 % b == 0 else 64, 128))):
        prefix = n_pref * b
        suffixes = [t, t + 1, 15, 16, 17, 33, b + 3, 100, 257]
        lengths = [prefix + max(t, s) for s in suffixes]
        case = build_case(lengths=lengths, num_q_heads=hq, num_kv_heads=hkv, head_dim=128, block_size=b, q_tokens=t,
                          dtype=torch.bfloat16, seed=1200 + b + hq + t + n_pref, shared_prefix_blocks=n_pref,
                          pool_slack=0.2)
        poison_case(case)
        kp, vp = oracle_after_write(case)
        ref = _oracle(case, kp, vp)
        for pt in [x for x in pts if x % b == 0]:
            print(f"[case] cascade b={b} hq={hq} hkv={hkv} T={t} prefix={prefix} pt={pt}", flush=True)
            g, out = _step(gpu_lib, case, prefix, pt)
            assert np.array_equal(bits(g["k_pool"]), kp) and np.array_equal(bits(g["v_pool"]), vp)
            assert_attention_close(out.cpu(), ref, kv_dtype=torch.bfloat16, out_dtype=torch.float32,
                                   what=f"cascade prefix={prefix} pt={pt}")
            _same_step(g, out, *_fused_step(gpu_lib, case, prefix, pt))


def test_cascade_without_prefix_is_the_split_path_bitwise(gpu_lib):
    """prefix_tokens = 0: no prefix items, and the call is pa_decode_partitioned bit for bit."""
    case = make_case("prefix", num_seqs=6)
    g = _gpu(case)
    a = gpu_lib.decode_cascade(g["q"], g["k_pool"], g["v_pool"], g["block_tables"], g["seq_lens"], case.scale, 0,
                               case.max_seq_len, 512)
    b = gpu_lib.decode_partitioned(g["q"], g["k_pool"], g["v_pool"], g["block_tables"], g["seq_lens"], case.scale,
                                   case.max_seq_len, 512, variant=2)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


@pytest.mark.parametrize("pt", [256, 512, 1024])
def test_cascade_prefix_workload_subset(gpu_lib, pt):
    """The prefix workload's shape (2048 shared tokens, 32/8 heads) on its first 8 sequences, whole."""
    case = make_case("prefix", num_seqs=8)
    poison_case(case)
    kp, vp = oracle_after_write(case)
    g, out = _step(gpu_lib, case, 2048, pt)
    assert_attention_close(out.cpu(), _oracle(case, kp, vp), kv_dtype=torch.bfloat16, out_dtype=torch.float32,
                           what=f"prefix pt={pt}")


def test_cascade_fused_append_full_size_bitwise(gpu_lib):
    """All 128 sequences of the prefix workload: the fused append + cascade equals pa_write_kv followed by
    pa_decode_cascade bit for bit (pools and out), in the launch configuration the benchmark times."""
    case = make_case("prefix", pool_device=DEV)
    print("[case] cascade fused full", flush=True)
    g, out = _step(gpu_lib, case, 2048, 256)
    f, fout = _fused_step(gpu_lib, case, 2048, 256)
    _same_step(g, out, f, fout)


def test_cascade_full_size_sampled(gpu_lib):
    """All 128 sequences of the prefix workload; sampled rows against the oracle row by row."""
    case = make_case("prefix", pool_device=DEV)
    g, out = _step(gpu_lib, case, 2048, 512)
    kp, vp = oracle_after_write(case)
    kpool = torch.from_numpy(kp.view(np.int16)).view(torch.bfloat16).reshape(case.k_pool.shape).float().numpy()
    vpool = torch.from_numpy(vp.view(np.int16)).view(torch.bfloat16).reshape(case.v_pool.shape).float().numpy()
    q = case.q.float().numpy()
    tables, lens = case.block_tables.numpy(), case.seq_lens.numpy()
    rng = np.random.default_rng(77)
    b, t, hq, _ = case.q.shape
    rows = sorted({(0, 0, h) for h in range(hq)} | {(b - 1, 0, h) for h in range(hq)}
                  | {(int(rng.integers(b)), 0, int(rng.integers(hq))) for _ in range(64)})
    ref = np.stack([oracle.decode_row(q, kpool, vpool, tables, lens, case.scale, case.block_size, i, tt, h)
                    for i, tt, h in rows])
    got = out.cpu().double().numpy()
    err = assert_attention_close(np.stack([got[i, tt, h] for i, tt, h in rows]), ref, kv_dtype=torch.bfloat16,
                                 out_dtype=torch.float32, what="prefix full")
    print(f"[result] cascade full prefix: {len(rows)} rows, max |err| = {err:.2e}", flush=True)


def test_cascade_pa_check_rejects_unshared_prefix(gpu_lib, monkeypatch):
    """PA_CHECK=1: a sequence whose first blocks are not the shared ones is refused before any launch."""
    case = make_case("prefix", num_seqs=4)
    g = _gpu(case)
    monkeypatch.setenv("PA_CHECK", "1")
    ok = gpu_lib.decode_cascade(g["q"], g["k_pool"], g["v_pool"], g["block_tables"], g["seq_lens"], case.scale, 2048,
                                case.max_seq_len, 512)
    torch.cuda.synchronize()
    assert torch.isfinite(ok).all()
    bad = g["block_tables"].clone()
    bad[2, 5], bad[2, 130] = bad[2, 130].item(), bad[2, 5].item()  # a private block swapped into the prefix
    with pytest.raises(gpu_lib.PaError) as err:
        gpu_lib.decode_cascade(g["q"], g["k_pool"], g["v_pool"], bad, g["seq_lens"], case.scale, 2048,
                               case.max_seq_len, 512)
    assert err.value.status == -1
