"""CPU oracle (test infrastructure only): the plain definition of the drafter step that the HIP path is checked
against. Imported only by the tests, the smoke check and the benchmark's CPU-baseline leg."""
from .drafter import (NEG_FILL_F32, Config, Model, SharedKV, attend, bf16_bits, bf16_to_f64, check_head_invariants,
                      config_from, decoder_layer, dense_head_result, dense_head_row, draft_block, head_order, sample_row, drafter_step, gelu_tanh, key_window,
                      masked_head_row, rmsnorm, rope_rotate, round_bf16, topk_desc)

__all__ = ["NEG_FILL_F32", "Config", "Model", "SharedKV", "attend", "bf16_bits", "bf16_to_f64", "check_head_invariants",
           "config_from", "decoder_layer", "dense_head_result", "dense_head_row", "head_order", "sample_row", "draft_block", "drafter_step", "gelu_tanh", "key_window",
           "masked_head_row", "rmsnorm", "rope_rotate", "round_bf16", "topk_desc"]
