"""MI355X-native forward pass of the stacked Wukong feature-interaction layer.

The layer (Wukong paper, section 2.2, as summarised on the xdnf.cn repost of
the Zhihu article): a Factorization Machine Block and a Linear Compress Block
run side by side on each example's n x d embedding matrix, their outputs are
concatenated, the residual is added and a LayerNorm is applied; layers are
stacked; a prediction head (top MLP + logistic function) can follow the
stack, WHALE's fusion step (shared K = V cross-attention, Fusion MLP,
pre-norm shared-gate SwiGLU) combines a layer's output with a sequence, and
a layer's backward pass gives the input and weight gradients for training,
and a mixture-of-experts layer runs several Wukong modules side by side.
The compute runs in hand-written HIP kernels for gfx950 behind the C ABI in
include/wukong.h; this package is the Python binding.
"""
from ._abi import (ABI_VERSION, BF16, F32, KERNEL_NAMES, DeviceFusion, DeviceHead, DeviceLayer,  # noqa: F401
                   FusionSpec, HeadSpec, LayerGrads, LayerSpec, Trace, WukongError, alloc_workspace,
                   fusion_forward, layer_backward, layer_backward_workspace_size, layer_forward_train,
                   layer_saved_size, saved_layout, stack_saved_size, stack_forward_train,
                   stack_backward_workspace_size, stack_backward, MoeSpec, DeviceMoe, moe_forward, moe_workspace_size,
                   fusion_workspace_size, head_forward, head_workspace_size,
                   layer_forward, layer_workspace_size, library_path, load_library, stack_forward,
                   stack_workspace_size, status_string, to_device, workspace_layout, EXPORTED_SYMBOLS,
                   probe_mfma_bf16, layer_forward_noalloc, noalloc_max_workspace)
