"""Sparse Mixture-of-Experts layer (Nemotron 3 MoE and LatentMoE) for MI355X / gfx950: the
forward pass, and the backward pass of the plain bf16 layer.

The layer runs in hand-written HIP kernels behind the C ABI declared in include/moe.h
(libmoe_mi355x.so, built in-tree by ``python -m sparse_moe_layer_05_amd.build``). This package
is its thin Python binding: torch provides device memory and streams.
"""
from .binding import (Backward, Layer, MoeError, alloc_routing, backward_from, bias_update,
                      dispatch, layer_forward, layer_from, lib, route, status_str, to_device,
                      workspace_size)

__all__ = ["Backward", "Layer", "MoeError", "alloc_routing", "backward_from", "bias_update",
           "dispatch", "layer_forward", "layer_from", "lib", "route", "status_str", "to_device",
           "workspace_size"]
