"""Seeded synthetic workloads for the MXFP4-weight / FP8-activation routed MoE FFN.

This package is the one place that both the CPU oracle (under ``oracle/``) and the
GPU path (``mxfp4_weights_fp8_amd``) take their inputs from. It draws token
activations, router choices and expert weights, and packs the weights into the
storage formats the FFN consumes. It holds no step of the FFN itself.
"""

from .workloads import (  # noqa: F401
    WORKLOADS,
    Workload,
    MoEInputs,
    make_inputs,
    make_routing,
    make_x,
    make_expert_weights,
    make_shared_weights,
    slice_experts,
    scaled,
    routing_stats,
)
