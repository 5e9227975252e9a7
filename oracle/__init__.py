"""CPU oracle (fp64 dequantise-then-matmul).  Test infrastructure only: see
``oracle/qgemv_oracle.py`` for what may use it."""
from .qgemv_oracle import *  # noqa: F401,F403
from .qgemv_oracle import (GROUP, code_offset, unpack_uniform, pack_uniform, unpack_mixed,  # noqa: F401
                           row_word_offsets, dequant_uniform, trellis_states, trellis_dequant,
                           hadamard128, rotate, matmul, gemv_uniform, gemv_uniform_rows, gemv_mixed,
                           gemv_trellis, silu, mlp, normwise_rel_err)
