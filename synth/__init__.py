"""Seeded synthetic inputs for the any-precision MoE layer.

Shared by the oracle and by the GPU path's tests and benchmark.  It draws
random tensors and lays them out in the storage format (bit-planes + LUTs,
or fp16 rows); it computes no part of the layer itself.
"""
from .configs import CONFIGS, CONFIG_ORDER, LayerConfig, VALID_BITS, custom, get  # noqa: F401
from .gen import (LayerInputs, MatrixData, make_inputs, planner_inputs,  # noqa: F401
                  pack_planes, plane_bytes)
