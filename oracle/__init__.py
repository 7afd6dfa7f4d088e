"""fp64 CPU oracle for GPTQ layer quantization (test infrastructure only; see
gptq_oracle's header for who may import it)."""
from .gptq_oracle import *  # noqa: F401,F403
from .gptq_oracle import (hessian, damp, inverse_cholesky_upper, quant_params, quantize, dequantize,
                          gptq_quantize, gptq_quantize_obs, gptq_quantize_naive, obs_step, rtn, layer_loss,
                          layer_loss_direct, pack_codes, unpack_codes, packed_words, n_groups,
                          quantize_layer_from_x, boundary_distance, dequant_from, maxq_of, check_schedule, dequant_matmul,
                          hadamard_matrix, hadamard_rotate, default_rotation_block, weight_incoherence,
                          silu, swiglu, quantize_mlp_stack, obq_greedy, attention, attention_error_bound,
                          round_activations, quantize_transformer_stack)
