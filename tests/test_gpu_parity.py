"""GPU parity of every step of the layer against the oracle, through the C ABI.

Bars: routing ids, counts, offsets, sorted slots and their inverse bit-exact
(ids outside the near-tie guard); gates within 1e-6; A, Y and the layer
output within |y - y_ref| <= 2e-3 * sum|w||x| + 1e-5 per element.
"""
import dataclasses

import numpy as np
import pytest

import synth
from any_precision_quantized_amd import _lib
from oracle import moe

from . import gpu_helpers as G
from .oracle_cache import layer_ref, resolve_bits

pytestmark = pytest.mark.gpu

ALL_GEMV = 1 << 30     # every group on the bit-plane GEMV path
ALL_TILE = 1           # every group on the MFMA tile path

SMALL = {
    "tiny": synth.get("tiny"),
    # ragged: H = 10 words, I = 26 row-groups of 16 (not a multiple of 64), odd T
    "ragged": synth.custom("ragged", E=6, H=320, I=416, k=2, T=37, bits=(3, 4, 5, 6, 16, 4)),
    # k = E and tiny K (3 words)
    "k_eq_e": synth.custom("k_eq_e", E=5, H=96, I=96, k=5, T=7, bits=(6, 3, 16, 5, 4)),
    # one expert, 50 tokens: a single group crossing the tile threshold
    "one_expert": synth.custom("one_expert", E=1, H=128, I=224, k=1, T=50, bits=(5,)),
    # every expert on the fp16 fallback
    "all_fp16": synth.custom("all_fp16", E=4, H=256, I=160, k=2, T=21, bits=(16, 16, 16, 16)),
    # a single token
    "t1": synth.custom("t1", E=8, H=512, I=384, k=2, T=1, bits=(3, 4, 5, 6, 16, 3, 4, 5)),
    # 128 tokens over 3 experts: groups of ~85 (several 64-token tiles, ragged)
    "wide": synth.custom("wide", E=3, H=192, I=288, k=2, T=128, bits=(4, 6, 3)),
    # shared expert of 3x the routed size: three always-on experts in the routed launches
    "shared_fused": synth.custom("shared_fused", E=5, H=192, I=96, k=2, T=40, bits=(3, 4, 5, 6, 16), shared_I=288),
    # two fp16 experts of 70 tokens each: on the GEMV path, token chunks of 32 + 32 + 6
    "fp16_wide": synth.custom("fp16_wide", E=2, H=128, I=192, k=2, T=70, bits=(16, 16)),
    # shared expert whose size is no multiple of I: its own launches on a side stream
    "shared_side": synth.custom("shared_side", E=4, H=160, I=128, k=1, T=33, bits=(6, 3, 4, 5), shared_I=224),
    # groups of 33..64 tokens on 3-, 6- and 4-bit experts (the 64-token GEMV
    # pass), rows not a multiple of 64
    "mid_groups": synth.custom("mid_groups", E=3, H=224, I=352, k=2, T=60, bits=(3, 6, 4)),
    # the same with a long down projection (K = 7168, 56 steps): 64-token
    # passes under a K split
    "mid_groups_ksplit": synth.custom("mid_groups_ksplit", E=2, H=128, I=7168, k=1, T=90, bits=(3, 5)),
    # 40 experts (three 16-expert router tiles) over H = 1024 split in two
    # hidden chunks: partial logits added by the select launch
    "router_tiles": synth.custom("router_tiles", E=40, H=1024, I=128, k=4, T=48,
                                 bits=tuple((5, 3, 6, 4)[e % 4] for e in range(40))),
    # the largest expert count (256): router lanes hold four experts, the item
    # lookups scan four chunks of 64 experts
    "max_experts": synth.custom("max_experts", E=256, H=64, I=96, k=8, T=48,
                                bits=tuple((3, 4, 5, 6, 16)[e % 5] for e in range(256))),
    # 252 routed experts + a shared expert of 4x the routed size as 4 always-on
    # experts: 256 experts in the grouping and the expert launches
    "max_experts_shared": synth.custom("max_experts_shared", E=252, H=64, I=64, k=4, T=40,
                                       bits=tuple((6, 5, 4, 3)[e % 4] for e in range(252)), shared_I=256),
}


@pytest.mark.parametrize("mfma_min", [ALL_GEMV, ALL_TILE, 16, 65])
@pytest.mark.parametrize("name", list(SMALL))
def test_small_layer_every_step(name, mfma_min):
    cfg = SMALL[name]
    G.say(f"case {name} mfma_min {mfma_min}")
    inp = G.inputs(cfg)
    bits = resolve_bits(inp)
    ref = moe.layer(inp, bits=bits)
    _, got = G.run_layer(inp, bits, mfma_min)
    n_amb = G.check_route(inp, got, ref["ids"], ref["gates"], ref["logits"])
    assert n_amb == 0
    G.check_grouping(cfg, got)
    worst = G.check_experts(inp, bits, got)
    ratio = G.check_out(got, ref)
    G.say(f"  worst expert err/bound {worst:.3g}, layer err/bound {ratio:.3g}")


def test_forced_single_expert_skew():
    cfg = synth.custom("skew", E=4, H=128, I=96, k=1, T=100, bits=(3, 6, 4, 16))
    inp = dataclasses.replace(G.inputs(cfg), bias=np.array([-100, -100, 100, -100], dtype=np.float32))
    ref = moe.layer(inp)
    for mfma_min in (ALL_GEMV, ALL_TILE):
        _, got = G.run_layer(inp, inp.bits, mfma_min)
        assert got["counts"].tolist() == [0, 0, 100, 0]
        G.check_route(inp, got, ref["ids"], ref["gates"], ref["logits"])
        G.check_grouping(cfg, got)
        G.check_out(got, ref)


def test_deterministic_bitwise():
    inp = G.inputs(SMALL["ragged"])
    bits = inp.bits
    for mfma_min in (ALL_GEMV, ALL_TILE):
        layer, a = G.run_layer(inp, bits, mfma_min)
        _, b = G.run_layer(inp, bits, mfma_min, layer=layer)
        for key in ("ids", "gates", "sorted_slots", "A", "Y", "out"):
            assert np.array_equal(a[key], b[key]), key


def test_commit_takes_effect_in_stream_order():
    import torch
    from any_precision_quantized_amd import layer as L
    inp = G.inputs(SMALL["tiny"])
    bits1 = np.array(inp.bits)
    bits2 = np.array([6, 6, 3, 3, 16, 5, 4, 3], dtype=np.int8)
    for e in range(8):
        if bits2[e] == 16 and inp.experts[e]["gate"].w16 is None:
            bits2[e] = 4        # tiny has no fp16 copies
    layer = L.from_inputs(inp, bits=bits1)
    x = torch.from_numpy(inp.x.view(np.int16)).cuda().view(torch.float16)
    out1 = layer.forward(x).clone()          # enqueued before the commit
    layer.commit(bits2)
    out2 = layer.forward(x).clone()
    torch.cuda.synchronize()
    r1, r2 = moe.layer(inp, bits=bits1), moe.layer(inp, bits=bits2)
    G.check_out({"out": out1.float().cpu().numpy()}, r1)
    G.check_out({"out": out2.float().cpu().numpy()}, r2)


def test_commit_rejects_invalid_bits():
    import torch
    dev = torch.zeros(4, dtype=torch.int8, device="cuda")
    with pytest.raises(_lib.ApmoeError):
        _lib.commit_bits([3, 4, 7, 6], dev)
    torch.cuda.synchronize()
    assert dev.cpu().tolist() == [0, 0, 0, 0]


# ---------------------------------------------------------------------------
# The published workloads at full size
# ---------------------------------------------------------------------------

FULL = ["tiny", "qwen_decode", "mixtral_decode_t1", "mixtral_decode_t8", "mixtral_decode_t32",
        "e128_decode", "mixtral_prefill"]


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", FULL)
def test_full_size_layer(name):
    """Every output element of the full-size workload against the oracle
    (the Mixtral-shaped prefill included: all 8192 x 4096 outputs), and the
    expert stages in isolation on the hottest and the coldest touched expert
    (A against the oracle on the same grouping, Y against the oracle fed with
    the GPU's own A); at the prefill shape those groups of about 2048 slots
    run on the MFMA tile path."""
    cfg = synth.get(name)
    G.say(f"full-size case {name}")
    inp = G.inputs(cfg)
    bits = resolve_bits(inp)
    ref = layer_ref(inp, bits)
    _, got = G.run_layer(inp, bits)
    n_amb = G.check_route(inp, got, ref["ids"], ref["gates"], ref["logits"])
    G.check_grouping(cfg, got)
    ratio = G.check_out(got, ref)
    touched = [e for e in range(cfg.E) if got["counts"][e] > 0]
    G.say(f"  layer err/bound {ratio:.3g} over all {cfg.T} tokens; checking experts {touched[0]}, {touched[-1]}")
    worst = G.check_experts(inp, bits, got, experts=sorted({touched[0], touched[-1]}))
    G.say(f"  ambiguous routes {n_amb}, expert err/bound {worst:.3g}, "
          f"groups {sorted(got['counts'].tolist(), reverse=True)[:8]}")


# Expert counts that give the grouping launch's per-expert sums groups of 64,
# 32, 16, 8 and 4 lanes (a shared expert's always-on experts take none), and
# a grouping of more slots than its LDS parks (the workspace path).
STATS_CASES = {
    "e24": synth.custom("e24", E=24, H=256, I=128, k=3, T=40, bits=tuple((3, 4, 5, 6)[e % 4] for e in range(24))),
    "park_ws": synth.custom("park_ws", E=8, H=256, I=128, k=2, T=8200, bits=(3, 4, 5, 6, 3, 4, 5, 6)),
}


@pytest.mark.parametrize("name", ["tiny", "qwen_decode", "mixtral_decode_t8", "e128_decode", "mixtral_prefill",
                                  "e24", "router_tiles", "max_experts", "max_experts_shared", "park_ws"])
def test_route_stats(name):
    """Per-expert routing mass and routing-weighted input norm against the
    oracle's statistics over its own routing: as the forward computes them
    (token norms in the router, sums in the grouping launch; the one-kernel
    router at Mixtral T = 8, the two-kernel one elsewhere) and as
    apmoe_route_stats computes them alone."""
    import torch
    cfg = STATS_CASES.get(name) or SMALL.get(name) or synth.get(name)
    G.say(f"route stats {name}")
    inp = G.inputs(cfg)
    bits = resolve_bits(inp)
    ids, gates, logits = moe.route(inp.x, inp.w_router, inp.bias, cfg.logit_scale, cfg.k)
    mass_ref, wnorm_ref = moe.route_stats(inp.x, ids, gates, cfg.E)
    layer, got = G.run_layer(inp, bits)
    if G.check_route(inp, got, ids, gates, logits):
        pytest.skip("a near-tie routed a token differently; its expert's sums legitimately differ")
    # token norms from the router (fp32 sums of H squares)
    norms_ref = np.sqrt((inp.x.astype(np.float64) ** 2).sum(axis=1))
    np.testing.assert_allclose(layer.x_norms[:cfg.T].cpu().numpy(), norms_ref, rtol=1e-5)
    # the sums the forward's grouping launch computed, then the standalone call
    fused = [t.cpu().numpy().copy() for t in layer.route_stats()]
    x = torch.from_numpy(np.ascontiguousarray(inp.x).view(np.int16)).cuda().view(torch.float16)
    alone = [t.cpu().numpy().copy() for t in layer.route_stats(x)]
    for mass, wnorm in (fused, alone):
        # fp32 sums of at most T*k terms
        np.testing.assert_allclose(mass, mass_ref, rtol=1e-5, atol=1e-5)
        np.testing.assert_allclose(wnorm, wnorm_ref, rtol=1e-5, atol=1e-4)
        assert abs(float(mass.sum()) - cfg.T) <= 1e-4 * cfg.T


def test_online_planner_commits_take_effect():
    """An online re-plan under a growing KV footprint is committed in stream
    order: the next forward call runs at the new bitwidths (checked against
    the oracle at those bitwidths)."""
    import torch
    from any_precision_quantized_amd import layer as L
    cfg = SMALL["ragged"]
    inp = G.inputs(cfg)
    bits0 = [6] * cfg.E
    layer = L.from_inputs(inp, bits=bits0)
    levels = [6, 5, 4, 3]
    nbytes = np.array([[synth_bytes(cfg, b) for b in levels]] * cfg.E, dtype=np.uint64)
    harm = np.array([[0.0, 1.0, 3.0, 7.0]] * cfg.E) * (1 + np.arange(cfg.E))[:, None]
    planner_ = L.OnlinePlanner(layer, levels, harm, nbytes, [3] * cfg.E, [5, 4, 3],
                               m_total=int(nbytes[:, 0].sum()), hysteresis=0, bits_now=bits0)
    st, bits, stage, changed = planner_.step(m_kv=int(nbytes[0, 0] - nbytes[0, 2]) * 2)
    assert st == _lib.OK and changed and stage >= 0
    _, got = G.run_layer(inp, bits, layer=layer)
    ref = moe.layer(inp, bits=bits)
    assert np.array_equal(layer.bits.cpu().numpy(), np.asarray(bits, np.int8))
    G.check_out(got, ref)


def synth_bytes(cfg, b):
    """Plane + LUT bytes of one expert's three matrices at b bits."""
    return 3 * (cfg.H * cfg.I * b // 8) + (2 * cfg.I + cfg.H) * (1 << b) * 2


@pytest.mark.parametrize("rows,cols", [(16, 32), (32, 704), (48, 320), (64, 4096)])
def test_pack_planes_layout(rows, cols):
    """Packed word [p][group][step][g][i] is canonical word 4*step + g of row
    16*group + i of plane p (zero past the last word)."""
    import torch
    rng = np.random.default_rng(rows * 7 + cols)
    canon = rng.integers(0, 2**32, size=(6, rows, cols // 32), dtype=np.uint32)
    src = torch.from_numpy(canon.view(np.int32)).cuda()
    dst = torch.full((_lib.packed_plane_words(rows, cols),), -1, dtype=torch.int32, device="cuda")
    _lib.pack_planes(src, rows, cols, dst)
    got = dst.cpu().numpy().view(np.uint32)
    W = cols // 32
    ns = (W + 3) // 4
    padded = np.zeros((6, rows, 4 * ns), dtype=np.uint32)
    padded[:, :, :W] = canon
    expect = padded.reshape(6, rows // 16, 16, ns, 4).transpose(0, 1, 3, 4, 2).reshape(-1)
    assert np.array_equal(got, expect)


GRAPH_CASES = {
    "tiny": SMALL["tiny"],                  # one-kernel router
    "shared_fused": SMALL["shared_fused"],  # always-on fp16 experts: tile path at mfma_min 16
    "ragged": SMALL["ragged"],
    "router_tiles": SMALL["router_tiles"],  # matrix-core logits + select launch
    # one token over two experts, down stage K = 7168 (56 steps): the down GEMV
    # splits K in two and runs its finalize kernel
    "ksplit": synth.custom("ksplit", E=2, H=128, I=7168, k=1, T=1, bits=(5, 3)),
}


@pytest.mark.parametrize("name", list(GRAPH_CASES))
def test_graph_replay_matches_eager(name):
    """The layer step captured as a HIP graph: every replay, with eager work
    and synchronisations between replays, reproduces the eager step bit for
    bit, and the eager step matches the oracle."""
    import torch
    from any_precision_quantized_amd import layer as L
    cfg = GRAPH_CASES[name]
    G.say(f"case {name} graph replay")
    inp = G.inputs(cfg)
    bits = resolve_bits(inp)
    layer = L.from_inputs(inp, bits=bits, mfma_min_tokens=16)
    x = torch.from_numpy(np.ascontiguousarray(inp.x).view(np.int16)).cuda().view(torch.float16)
    keys = ("out", "topk_ids", "topk_w", "sorted_slots", "A", "Y")
    layer.forward(x)
    torch.cuda.synchronize()
    eager = {key: getattr(layer, key).clone() for key in keys}
    G.check_out({"out": eager["out"].float().cpu().numpy()}, moe.layer(inp, bits=bits))
    g = layer.graph(x)
    for rep in range(3):
        for key in keys:                      # eager work the replay has to overwrite
            getattr(layer, key).fill_(-1 if key in ("topk_ids", "sorted_slots") else 7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for key in keys:
            assert torch.equal(getattr(layer, key), eager[key]), (rep, key)
