"""CPU oracle (test infrastructure only; never imported by the product path)."""
from .loopq_oracle import (  # noqa: F401
    GROUP_A, qmax_for_bits, kron_transform, fold_weights, quant_weights, quant_act,
    group_dots, rescale_dots, qdq_linear, transformed_f32, linear, linear_per_token, looped_forward,
    looped_forward_sets, recurrent_adapter, round_bf16, cta_transition, cta_loop_inputs, looped_forward_cta,
    trajectory_hessian, thresholded_rank,
)
