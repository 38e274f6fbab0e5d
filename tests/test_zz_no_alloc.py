"""apmoe_bitplane_lut_gemm_noalloc against apmoe_bitplane_lut_gemm.

The allocation-free entry point keeps the split-K partial sums in the
library's static scratch instead of a caller's workspace; it runs the same
kernels, so its output must equal the workspace entry point's bit for bit.
Two calls in a row on the same GPU, the second with fewer tokens, both on
shapes whose K is split (so the scratch is really used), each stage checked.
"""
import numpy as np
import pytest

import synth
from any_precision_quantized_amd import _lib
from any_precision_quantized_amd import layer as L

from . import gpu_helpers as G

pytestmark = pytest.mark.gpu

# gate/up K = H = 7168 (56 steps, split in two); down K = I = 7168 likewise
CASES = [
    ("gate_up_split", dict(E=2, H=7168, I=256, k=1, bits=(5, 3))),
    ("down_split", dict(E=2, H=128, I=7168, k=1, bits=(5, 3))),
]


def _run(cfg_kw, T, name):
    import torch
    cfg = synth.custom(f"{name}_t{T}", T=T, **cfg_kw)
    inp = G.inputs(cfg)
    layer = L.from_inputs(inp, bits=np.asarray(cfg.bits, np.int8))
    x = torch.from_numpy(np.ascontiguousarray(inp.x).view(np.int16)).cuda().view(torch.float16)
    layer.forward(x)          # routing and grouping through the layer
    torch.cuda.synchronize()
    E, H, I, k = cfg.E, cfg.H, cfg.I, cfg.k
    assert _lib.workspace_bytes(T, k, E, H, I) > 0, "the shape must split K"
    args = (layer.table.desc, layer.bits, E, layer.offsets, layer.sorted_slots, k)
    A_ws = torch.full_like(layer.A, 7.0)
    A_na = torch.full_like(layer.A, -7.0)
    _lib.bitplane_lut_gemm(_lib.GATE_UP_SWIGLU, *args, x, A_ws, T, H, I, layer.mfma_min_tokens, layer.ws)
    _lib.bitplane_lut_gemm_noalloc(_lib.GATE_UP_SWIGLU, *args, x, A_na, T, H, I, layer.mfma_min_tokens)
    Y_ws = torch.full_like(layer.Y, 7.0)
    Y_na = torch.full_like(layer.Y, -7.0)
    _lib.bitplane_lut_gemm(_lib.DOWN, *args, A_ws, Y_ws, T, H, I, layer.mfma_min_tokens, layer.ws)
    _lib.bitplane_lut_gemm_noalloc(_lib.DOWN, *args, A_ws, Y_na, T, H, I, layer.mfma_min_tokens)
    torch.cuda.synchronize()
    assert torch.equal(A_na, A_ws), "gate/up output differs"
    assert torch.equal(Y_na, Y_ws), "down output differs"
    # and the workspace entry point itself matches the oracle on this grouping
    got = dict(A=A_ws.float().cpu().numpy(), Y=Y_ws.cpu().numpy(), offsets=layer.offsets.cpu().numpy(),
               sorted_slots=layer.sorted_slots.cpu().numpy())
    G.check_experts(inp, np.asarray(cfg.bits, np.int8), got)


@pytest.mark.parametrize("name,cfg_kw", CASES)
def test_noalloc_matches_workspace_entry_point(name, cfg_kw):
    for T in (5, 2):          # two calls in a row, the second smaller
        G.say(f"case {name} T {T}")
        _run(cfg_kw, T, name)
