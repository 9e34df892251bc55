"""CPU oracle (test infrastructure only; see qmm_oracle.py)."""
from .qmm_oracle import *  # noqa: F401,F403
from .qmm_oracle import (TYPE_Q4_0, TYPE_Q8_0, QK, BLOCK_BYTES, half_bits_to_double,  # noqa: F401
                         row_bytes, block_scales_and_codes, dequantize, matmul, matmul_sampled,
                         within_tolerance, quantize, quantize_codes, pack_blocks)
