"""Seeded synthetic workloads for the MoE expert-FFN layer.

This package is shared by the GPU path's tests/bench and by the CPU oracle's
tests.  It only draws random numbers and casts them to the storage formats the
layer consumes; it holds none of the layer's arithmetic (no routing, no
permutation, no GEMM, no activation quantisation).
"""
from .configs import CONFIGS, EXTRA_CONFIGS, MoeConfig, config_by_name  # noqa: F401
from .generate import generate_layer, generate_expert, to_numpy_inputs, LayerInputs  # noqa: F401
