"""Seeded synthetic inputs for the paged decode step.

The oracle and the HIP path both read these inputs. This module holds none of
the attention arithmetic. It draws lengths, hands out physical blocks, writes
block tables, and fills pools and queries with N(0, 1) values.
"""

from .configs import (  # noqa: F401
    CONFIG_NAMES,
    Case,
    PrefillCase,
    build_case,
    build_prefill_case,
    fp8_pools,
    int8_pools,
    make_case,
    make_prefill_case,
)
