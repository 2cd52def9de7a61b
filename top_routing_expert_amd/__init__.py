"""MI355X-native (gfx950) MoE-layer forward token path.

router -> permute (expert-contiguous, rank-major send layout) -> grouped SwiGLU
FFN -> weighted combine, as hand-written HIP kernels behind a C ABI
(`libmoe_mi355x.so`, declared in include/moe.h).  `top_routing_expert_amd.binding`
marshals torch tensors to that ABI; torch provides device memory and streams only.
"""
from . import configs, inputs  # noqa: F401

__all__ = ["configs", "inputs"]
