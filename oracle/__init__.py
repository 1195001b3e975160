"""Float64 CPU oracle for the paged-KV decode step.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import, call or run anything in this
package. The product path (``paged_kv_cache_69_amd`` and its HIP library) never
imports it, and this package imports nothing from the product path.

Every function restates what the pages define, in float64 numpy, with no
blocking, fusion or online recurrence. The pages are:

* [P1] "25. Paged attention and prefix caching" (inference.shantanugoel.com)
* [P2] "Модуль 09: PagedAttention: пейджинг KV-кэша" (hermes-agent.ru,
  LLM Inference Systems course)
* [P4] "PagedAttention and the KV Cache" (kanthi.in, Writing Kernel with AI)
* [P5] "Chapter 7 Paged KV Cache and Memory Management" (zero-to-sglang)

Parity pins: every function here is pinned by a ``-m "not gpu"`` test in
``tests/test_oracle.py``, ``tests/test_oracle_int8.py``,
``tests/test_oracle_prefill.py``, ``tests/test_oracle_blocks.py`` or
``tests/test_oracle_fp8.py``, which checks it
against something other than itself:
the pages' worked examples, a library routine, closed forms, invariants or
brute force. No function is "parity unpinned".
"""

from .pa_oracle_int8 import (  # noqa: F401
    append_int8,
    decode_int8,
    decode_row_int8,
    dequantize_pool,
    quantize_block,
)
from .pa_oracle_fp8 import (  # noqa: F401
    append_fp8,
    decode_fp8,
    decode_row_fp8,
    dequantize_pool_fp8,
    e4m3_values,
    encode_e4m3,
    quantize_block_fp8,
)
from .pa_oracle_blocks import BlockLedger, PoolExhausted  # noqa: F401
from .pa_oracle_prefill import chunk_positions, prefill, prefill_row, write_kv_varlen  # noqa: F401
from .pa_oracle import (  # noqa: F401
    attend_rows,
    blocks_needed,
    decode,
    decode_row,
    gather_positions,
    physical_slot,
    tail_waste,
    visible_length,
    write_kv,
)
