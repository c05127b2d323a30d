"""Intra-expert-sparse MoE decode layer for AMD MI355X (gfx950).

The HIP library libmoe_mi355x.so (include/moe_mi355x.h) holds every kernel;
`binding` marshals torch tensors into its C ABI and `layer.MoELayer` chains
its calls.  Importing this package does not load the library; the first
call does, and fails loudly if it has not been built.
"""
__all__ = ["binding", "build", "layer"]
