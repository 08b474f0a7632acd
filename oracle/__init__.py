"""CPU oracle of the Wukong interaction stack (forward and one layer's backward)
and of WHALE's fusion step --
TEST INFRASTRUCTURE ONLY.

Imported only by the tests, the package's smoke check and the benchmark's
CPU-baseline leg.  It shares no code with the HIP library.
"""
from .wukong_oracle import (LN_EPS, STORAGE_NAMES, brute_force_head, brute_force_layer,  # noqa: F401
                            decode_bf16, fm_interaction, fmb_mlp, layer_norm, lcb, prediction_head,
                            round_bf16, sigmoid, to_f64, wukong_layer, wukong_stack)
from .whale_oracle import (FUSION_STORAGE, brute_force_attention, cross_attention, silu,  # noqa: F401
                           whale_fusion)
from .wukong_backward import (BACKWARD_STORAGE, layer_backward, layer_loss, layer_norm_backward,  # noqa: F401
                              stack_backward, stack_loss)
from .wukong_moe_oracle import wukong_moe_layer  # noqa: F401
