"""CPU oracle for the weight-only low-bit matmul.  TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  It shares no code with the HIP library
and never calls it.
"""
from .qref import (  # noqa: F401
    INT4_ASYM, INT2_ASYM, Q4_0, Q8_0, Q4K, BITS, IMPLICIT_ZERO, Q4K_SUPER, Q4K_SUB,
    unpack_codes, pack_codes, dequant_f64, dequant_f32, dequant_f16, qgemm_ref,
    q4k_subblock_params,
    rel_error, within_tolerance, TOLERANCE, loop_block_ref,
    fold_zero_point_ref,
)
