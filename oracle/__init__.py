"""CPU oracle of the one-device MoE layer: the router, dispatch, grouped SwiGLU FFN,
combine, and their backward.

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's CPU
baseline use it; the product path never imports it.  It is numpy only and shares
no code with the HIP library.  Each function cites the passage of the
low_latency_combine page (Ascend CANN API) it follows.

Parity status: every function here is pinned by a CPU test (see tests/test_oracle_pins.py);
none is "parity unpinned".  The readings of silent points (masked-slot handling,
duplicate handling, prefix kind, row order, summation order) are pinned only by
internal consistency, as the pages print no output values.
"""
from .moe import (ERR_ID_DUPLICATE, ERR_ID_RANGE, ERR_MASK_NOT_PREFIX, Route, combine,
                  combine_bwd, decode, dequant_weights_fp8, dispatch, dispatch_bwd, ffn_bwd,
                  ffn_bwd_fp8, ffn_fwd, ffn_fwd_fp8, layer_bwd, layer_bwd_fp8, layer_fwd,
                  layer_fwd_fp8, qdq_cols_fp8, qdq_rows_fp8, qdq_rows_int8, quant_cols_fp8,
                  quant_weights_fp8, route, silu, wgrad_fp8, dispatch_int8, quant_weights_int8,
                  ffn_fwd_int8, layer_fwd_int8, qdq_rows_mx, quant_weights_mx, ffn_fwd_mx,
                  ffn_bwd_mx, layer_fwd_mx, layer_bwd_mx)
from .router import router_bwd, router_fwd, select_topk, softmax
from .numerics import (bf16_to_f32, dequant_e4m3_blocks, dequant_e4m3_rows, dequant_int8_rows,
                       e4m3_decode, e4m3_encode, f32_to_bf16, quant_e4m3_blocks, quant_e4m3_rows,
                       quant_int8_rows, round_bf16, quant_mx_e4m3_rows, dequant_mx_e4m3_rows)
