"""CPU oracle for the SVDQuant W4A4 + low-rank linear (test infrastructure only).

Only the test suite, ``__graft_entry__.smoke()`` and the CPU baseline leg of
``bench.py`` may import this package.  The product path never does.
"""
from .svdq_oracle import *  # noqa: F401,F403
from .svdq_oracle import (GROUP, QMAX, SMOOTH_EPS, activation_absmax, bf16_to_f64,
                          f32_to_bf16, f64_to_bf16, f64_to_f32, forward,
                          group_accumulators, linear_output, lora_down_project,
                          lowrank_split, pack_int4, pack_weights,
                          quantize_act_lora_down, quantize_activation_groups,
                          quantize_weight_groups, smooth_activations,
                          smooth_factors, smoothed_weight, storage_order, unpack_int4)
