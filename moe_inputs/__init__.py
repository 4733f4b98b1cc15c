"""Seeded synthetic inputs for the output-centric MoE decode layer.

This module only *makes* inputs: activations, routing and MXFP8-packed expert
weights.  It holds none of the layer's arithmetic (no dequantisation, no dot
products, no SiLU, no combine), so both the HIP path and the CPU oracle can
consume the same bytes without sharing any of the computation.

Shapes follow the workload described on the warp-decode blog post (Cursor,
"warp decode", sections "The traditional MoE path" and "Eliminating
buffers"): 128 experts, top-8 routing, hidden size 2048.  The intermediate
size 768 and the larger 4096/1536 shape are the stated synthetic configs.
"""
from .gen import (  # noqa: F401
    Layer,
    MX_BLOCK,
    make_layer,
    make_x,
    route_uniform,
    router_logits,
    route_zipf,
    route_adversarial,
    route_contiguous,
    make_routing,
    layer_seed,
    routing_seed,
    SHAPES,
    WORKLOADS,
)
