"""MI355X (gfx950) MoE expert layer: route -> dispatch -> grouped SwiGLU FFN -> combine.

The compute lives in libmoe_mi355x.so (HIP kernels behind the C ABI of
include/moe.h); ``expert_routing_grouped_amd.moe`` is its Python binding.
"""
__all__ = ["moe", "workloads", "tensors", "build"]
