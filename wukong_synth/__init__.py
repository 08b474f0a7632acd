"""Seeded synthetic workloads for the Wukong interaction stack (shapes + draws only)."""
from .configs import (CONFIGS, BY_NAME, LayerShape, WukongConfig, get,  # noqa: F401
                      TINY_F32, LAYER_D160, STACK8_N256, STACK8_N512, SMALLD_N720, UNITS_N2880)
from .gen import (HostFusionWeights, HostLayerWeights, make_fusion_weights, make_head_weights,  # noqa: F401
                  make_input, make_layer_weights, make_expert_weights, make_out_layernorm, make_sequence, make_stack_weights, make_upstream_grad,
                  to_bf16_bits,
                  bf16_bits_to_f32, feature_scales, stream_key)
