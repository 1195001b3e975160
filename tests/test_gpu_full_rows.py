"""Every output row of the full-size workloads against the float64 oracle, in the launch configuration the
benchmark times, on the GPU.

batch64: one fused append + single-pass call (pa_write_kv_decode). long: one fused append + split call
with 512-token partitions (pa_write_kv_decode_partitioned). prefix: one fused append + cascade call with
the 2048-token shared prefix and 256-token suffix partitions (pa_write_kv_decode_cascade). The 8-bit
workloads: the append call, then single pass (batch64) or 512-token partitions (long). The pools after
the step are compared bit for bit with the oracle's append, then every (sequence, token, head) row of the
output with the oracle's decode of those pools: 2e-3 absolute, the bf16 bar.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from tests.helpers import assert_attention_close, bits, oracle_after_write, to_f32_view
from workloads import fp8_pools, int8_pools, make_case

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _gpu(case):
    return {k: getattr(case, k).to(DEV, copy=True) for k in ("q", "k_new", "v_new", "k_pool", "v_pool", "block_tables",
                                                    "seq_lens", "positions")}


def _as_pool(case, x):
    return torch.from_numpy(x.view(np.int16)).view(case.k_pool.dtype).reshape(case.k_pool.shape)


@pytest.mark.parametrize("name", ["batch64", "long", "prefix"])
def test_every_row_bf16_workloads(gpu_lib, name):
    case = make_case(name, pool_device=DEV)
    g = _gpu(case)
    print(f"[case] every row {name} B={case.q.shape[0]} pool={tuple(case.k_pool.shape)}", flush=True)
    if name == "batch64":
        out = gpu_lib.write_kv_decode(g["q"], g["k_new"], g["v_new"], g["k_pool"], g["v_pool"], g["block_tables"],
                                      g["seq_lens"], case.scale)
    elif name == "long":
        out = gpu_lib.write_kv_decode(g["q"], g["k_new"], g["v_new"], g["k_pool"], g["v_pool"], g["block_tables"],
                                      g["seq_lens"], case.scale, max_seq_len=case.max_seq_len, partition_tokens=512)
    else:
        out = gpu_lib.write_kv_decode_cascade(g["q"], g["k_new"], g["v_new"], g["k_pool"], g["v_pool"],
                                              g["block_tables"], g["seq_lens"], case.scale, 2048, case.max_seq_len, 256)
    torch.cuda.synchronize()
    kp, vp = oracle_after_write(case)
    assert np.array_equal(bits(g["k_pool"]), kp) and np.array_equal(bits(g["v_pool"]), vp)
    del g
    ref = oracle.decode(to_f32_view(case.q), to_f32_view(_as_pool(case, kp)), to_f32_view(_as_pool(case, vp)),
                        case.block_tables.numpy(), case.seq_lens.numpy(), case.scale, case.block_size)
    err = assert_attention_close(out.cpu(), ref, kv_dtype=torch.bfloat16, out_dtype=torch.float32, what=name)
    print(f"[result] {name}: all {ref.shape[0] * ref.shape[1] * ref.shape[2]} rows, max |err| = {err:.2e}", flush=True)


@pytest.mark.parametrize("fmt", ["int8", "fp8"])
@pytest.mark.parametrize("name,pt", [("batch64", None), ("long", 512)])
def test_every_row_8bit_workloads(gpu_lib, fmt, name, pt):
    case = make_case(name, pool_device=DEV)
    pools = (int8_pools if fmt == "int8" else fp8_pools)(case, seed=23)
    print(f"[case] every row {name}_{fmt}", flush=True)
    kc, vc, sc = (x.to(DEV, copy=True) for x in pools)
    q, kn, vn, tab, lens, pos = (getattr(case, k).to(DEV) for k in ("q", "k_new", "v_new", "block_tables", "seq_lens",
                                                                   "positions"))
    (gpu_lib.write_kv_int8 if fmt == "int8" else gpu_lib.write_kv_fp8)(kn, vn, kc, vc, sc, tab, pos)
    if pt:
        out = (gpu_lib.decode_partitioned_int8 if fmt == "int8" else gpu_lib.decode_partitioned_fp8)(
            q, kc, vc, sc, tab, lens, case.scale, case.max_seq_len, pt)
    else:
        out = (gpu_lib.decode_int8 if fmt == "int8" else gpu_lib.decode_fp8)(q, kc, vc, sc, tab, lens, case.scale)
    torch.cuda.synchronize()

    def np_codes(t):
        return t.cpu().view(torch.uint8).numpy().view(np.int8 if fmt == "int8" else np.uint8)

    s0 = pools[2].cpu().numpy()
    ref_pools = (oracle.append_int8 if fmt == "int8" else oracle.append_fp8)(
        np_codes(pools[0]), np.ascontiguousarray(s0[..., 0]), np_codes(pools[1]), np.ascontiguousarray(s0[..., 1]),
        case.k_new.float().numpy(), case.v_new.float().numpy(), case.block_tables.numpy(), case.positions.numpy(),
        case.block_size)
    s1 = sc.cpu().numpy()
    assert np.array_equal(np_codes(kc), ref_pools[0]) and np.array_equal(np_codes(vc), ref_pools[2])
    assert np.array_equal(s1[..., 0].view(np.int32), ref_pools[1].view(np.int32))
    assert np.array_equal(s1[..., 1].view(np.int32), ref_pools[3].view(np.int32))
    del kc, vc, sc, pools
    ref = (oracle.decode_int8 if fmt == "int8" else oracle.decode_fp8)(
        case.q.float().numpy(), *ref_pools, case.block_tables.numpy(), case.seq_lens.numpy(), case.scale,
        case.block_size)
    err = assert_attention_close(out.cpu(), ref, kv_dtype=torch.int8, out_dtype=torch.float32, what=f"{name}_{fmt}")
    print(f"[result] {name}_{fmt}: all rows, max |err| = {err:.2e}", flush=True)
