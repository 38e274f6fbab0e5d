"""GPU parity on seeded random layer shapes: expert counts, hidden and
intermediate sizes (multiples of 32, ragged against the 64-row blocks and
128-column steps), top-k, token counts, shared experts and per-expert
bitwidths drawn from a fixed generator, each compared step by step against
the oracle on both expert paths (every group on the GEMV path, then every
group on the tile path)."""
import numpy as np
import pytest

import synth
from oracle import moe

from . import gpu_helpers as G
from .oracle_cache import resolve_bits

pytestmark = pytest.mark.gpu

ALL_GEMV = 1 << 30
ALL_TILE = 1


def random_config(seed):
    rng = np.random.default_rng(1000 + seed)
    E = int(rng.choice([1, 2, 3, 5, 8, 13, 24, 40, 64, 100]))
    k = int(rng.integers(1, min(E, 8) + 1))
    H = 32 * int(rng.integers(1, 33))          # 32 .. 1024
    I = 32 * int(rng.integers(1, 25))          # 32 .. 768
    T = int(rng.integers(1, 97))
    bits = tuple(int(b) for b in rng.choice([3, 4, 5, 6, 16], size=E))
    shared_I = 0
    if rng.random() < 0.3:
        shared_I = I * int(rng.integers(1, 4)) if rng.random() < 0.7 else 32 * int(rng.integers(1, 25))
    return synth.custom(f"rand{seed}", E=E, H=H, I=I, k=k, T=T, bits=bits, shared_I=shared_I)


@pytest.mark.parametrize("seed", range(40))
def test_random_shape(seed):
    cfg = random_config(seed)
    G.say(f"random shape {seed}: E{cfg.E} H{cfg.H} I{cfg.I} k{cfg.k} T{cfg.T} shared_I{cfg.shared_I} bits {cfg.bits}")
    inp = G.inputs(cfg)
    bits = resolve_bits(inp)
    ref = moe.layer(inp, bits=bits)
    for mfma_min in (ALL_GEMV, ALL_TILE):
        _, got = G.run_layer(inp, bits, mfma_min)
        assert G.check_route(inp, got, ref["ids"], ref["gates"], ref["logits"]) == 0
        G.check_grouping(cfg, got)
        G.check_experts(inp, bits, got)
        G.check_out(got, ref)
