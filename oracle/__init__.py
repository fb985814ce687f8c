"""CPU oracle for the bitmap sparse-weight SpMM (test infrastructure only).

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this package; the GPU library never does.
"""
from .tca_bme import *  # noqa: F401,F403
from .tca_bme import (Encoded, Geometry, VAL_F16, VAL_I4, abs_bound, compare, decode, decode_i4,  # noqa: F401
                      decode_loop, dense_weight, encode, encode_i4, encode_loop, masked_popcount, popcount,
                      quantize_rows_i4, spmm, spmm_fp64, storage_bytes)
