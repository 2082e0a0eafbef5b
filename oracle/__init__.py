"""CPU fp64 oracle for the W4A16 GEMM -- test infrastructure only.

Importable only from ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py``. The product library never uses it.
"""
from .w4a16_ref import (  # noqa: F401
    GROUP,
    bf16_to_f64,
    f32_to_bf16_rne,
    pack_int4,
    unpack_int4,
    dequant,
    gemm,
    gemm_entries,
    splitk_group_ranges,
    gemm_splitk_partials,
    splitk_reduce_bf16,
    group_starts,
    gemm_grouped,
    gemm_batched,
    gate,
)
