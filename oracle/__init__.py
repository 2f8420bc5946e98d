"""CPU oracle for the PATCH hybrid dense / 2:4 tile GEMM.

TEST INFRASTRUCTURE ONLY: only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package.  It shares no code with the library.
"""
from .patch_oracle import (DENSE, SPARSE24, LEGAL_CODES, TOL, MaskError, Packed, ShapeError,  # noqa: F401
                           bf16_to_f64, check_shape, classify, compress, decompress, gemm_brute,
                           gemm_ref, mask_of, masked_weight, measured_sparsity, rel_error,
                           tile_slots, unpack_bits, within_tolerance)
from . import sample_oracle  # noqa: F401,E402
