"""pa_decode_partitioned_noalloc through the C ABI, on the GPU: the partials live in the library's fixed
device scratch, and the output must be the same bits as pa_decode_partitioned with a caller workspace
(the same kernels) on a schedule that gives the same bits on every call, on two calls in a row, the
second with a smaller input, and meet the float64 oracle; the library's own choice (balanced ranges for
the larger input, whose last bits may vary from call to call) meets the oracle too. Sizes past the
fixed scratch are refused with PA_ERR_TOO_LARGE before any launch."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from tests.helpers import assert_attention_close, oracle_after_write, poison_case, to_f32_view
from workloads import build_case, make_case

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _prepared(case):
    poison_case(case)
    g = {k: getattr(case, k).to(DEV, copy=True) for k in ("q", "k_new", "v_new", "k_pool", "v_pool", "block_tables",
                                                         "seq_lens", "positions")}
    return g


def _oracle(case):
    kp, vp = oracle_after_write(case)
    back = lambda x: torch.from_numpy(x.view(np.int16)).view(case.k_pool.dtype).reshape(case.k_pool.shape)  # noqa
    return oracle.decode(to_f32_view(case.q), to_f32_view(back(kp)), to_f32_view(back(vp)), case.block_tables.numpy(),
                         case.seq_lens.numpy(), case.scale, case.block_size)


def test_noalloc_matches_workspace_call_twice(gpu_lib):
    big = make_case("long", num_seqs=6)  # lengths from the long workload's distribution, 512-position partitions
    small = build_case(lengths=[1, 17, 300, 40], num_q_heads=32, num_kv_heads=8, head_dim=128, block_size=16,
                       dtype=torch.bfloat16, seed=4242)
    for case, pt in ((big, 512), (small, 64)):
        print(f"[case] noalloc B={case.q.shape[0]} max_len={case.max_seq_len} pt={pt}", flush=True)
        need = gpu_lib.workspace_bytes(case.q, case.k_pool, case.block_tables, case.max_seq_len, pt)
        assert need <= gpu_lib.NOALLOC_SCRATCH_BYTES
        g = _prepared(case)
        gpu_lib.write_kv(g["k_new"], g["v_new"], g["k_pool"], g["v_pool"], g["block_tables"], g["positions"])
        want = _oracle(case)
        for sched in (2, 0):  # two partitions per wave (same bits on every call), then the library's choice
            ref_out = gpu_lib.decode_partitioned(g["q"], g["k_pool"], g["v_pool"], g["block_tables"], g["seq_lens"],
                                                 case.scale, case.max_seq_len, pt, split_schedule=sched)
            out = torch.empty_like(ref_out)
            gpu_lib.decode_partitioned_noalloc(g["q"], g["k_pool"], g["v_pool"], g["block_tables"], g["seq_lens"],
                                               case.scale, case.max_seq_len, pt, out, split_schedule=sched)
            torch.cuda.synchronize()
            if sched == 2:
                assert torch.equal(out, ref_out), "the scratch-backed call gave other bits than the workspace call"
            assert_attention_close(out.cpu(), want, kv_dtype=torch.bfloat16, out_dtype=torch.float32,
                                   what=f"noalloc pt={pt} schedule={sched}")
            assert_attention_close(ref_out.cpu(), want, kv_dtype=torch.bfloat16, out_dtype=torch.float32,
                                   what=f"workspace pt={pt} schedule={sched}")


def test_noalloc_refuses_sizes_past_the_scratch(gpu_lib):
    case = build_case(lengths=[20, 30], num_q_heads=32, num_kv_heads=8, head_dim=128, block_size=16,
                      dtype=torch.bfloat16, seed=4343)
    g = _prepared(case)
    out = torch.zeros(case.q.shape, dtype=torch.float32, device=DEV)
    huge = 1 << 30  # a max_seq_len whose partials need far more than 32 MiB
    assert gpu_lib.workspace_bytes(case.q, case.k_pool, case.block_tables, huge, 16) > gpu_lib.NOALLOC_SCRATCH_BYTES
    print("[case] noalloc too large", flush=True)
    with pytest.raises(gpu_lib.PaError) as err:
        gpu_lib.decode_partitioned_noalloc(g["q"], g["k_pool"], g["v_pool"], g["block_tables"], g["seq_lens"],
                                           case.scale, huge, 16, out)
    assert err.value.status == -5
    torch.cuda.synchronize()
    assert not out.any()  # nothing ran
