"""any_precision_quantized_amd: an MI355X (gfx950) MoE expert-FFN layer over
any-precision (bit-plane + LUT) expert weights.

The compute path is libapmoe.so (hand-written HIP, C ABI in include/apmoe.h);
this package binds it with ctypes and uses PyTorch only for device memory and
streams.
"""
from . import _lib  # noqa: F401
from ._lib import ApmoeError, GATE_UP_SWIGLU, DOWN  # noqa: F401

__all__ = ["ApmoeError", "GATE_UP_SWIGLU", "DOWN"]
