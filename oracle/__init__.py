"""CPU oracle for the AWQ W4A16 hot path -- test infrastructure only.

Importable by the tests, by ``__graft_entry__.smoke`` and by the
``cpu_baseline`` leg of ``bench.py``; never by the product package.
"""
from .awq_oracle import *  # noqa: F401,F403
from .awq_oracle import (act_stat, candidate_scale, quantize, quantize_values, dequantize, pack,
                         unpack, unpack_fast, matmul, matmul_rows, output_mse,
                         search_scale, scale_activations, f16_round_down,
                         levels, packed_words_per_row, pack_rows,
                         packed_words, words_per_quarter, tiles_to_rows,
                         tile_params, untile_params, apply_inv_scale, silu, gate_up,
                         gate_up_rows, search_scale_shared, mlp_block_loss, search_scale_mlp,
                         fake_quantize)
