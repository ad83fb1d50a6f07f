"""Synthetic workload shapes and seeded input generators (no method arithmetic)."""
from .configs import (ALL, BLOCK_STACK, BLOCK_SWA, DECODE_PAIR, GLOBAL_PREFILL, STACK, SWA_PREFILL, TINY,
                      MixerShape, stack_layer_roles, with_)
from .inputs import (bf16_bits, bf16_round, block_inputs, block_inputs_torch,
                     block_weight_rows, cached_meta_inputs, decode_inputs, prefill_inputs,
                     prefill_inputs_torch, to_device)
