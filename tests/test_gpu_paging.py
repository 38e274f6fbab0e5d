"""Plane paging on the GPU through the C ABI (apmoe_pager_*).

After every staged and committed change of bitwidths the layer's output is
checked against the oracle at the new bitwidths (the layer bar), the resident
blocks are read back and compared bit for bit with the host copy (the top b
packed planes and the b-bit LUT of every matrix, no other pointer set), and
the resident and host-to-device bytes are compared with the paging oracle.
"""
import numpy as np
import pytest

import synth
from any_precision_quantized_amd import _lib
from any_precision_quantized_amd.layer import MATS, ExpertTable, MoELayer
from any_precision_quantized_amd.paging import PagedExperts, arena_bytes_for
from oracle import moe, paging

from . import gpu_helpers as G
from .oracle_cache import layer_ref, resolve_bits

pytestmark = pytest.mark.gpu

# K of every matrix a multiple of 128, so packed slabs hold no padding and the
# byte counts equal the oracle's; expert 4 has fp16 weights and may run at 16 bits
PAGED = synth.custom("paged", E=6, H=256, I=384, k=2, T=40, bits=(3, 4, 5, 6, 16, 4))
RAGGED = synth.custom("ragged", E=6, H=320, I=416, k=2, T=37, bits=(3, 4, 5, 6, 16, 4))
PLANS = [
    [6, 6, 6, 6, 16, 6],     # promote everything
    [3, 3, 3, 3, 16, 3],     # demote everything (LUTs change, no plane moves)
    [5, 3, 6, 4, 6, 3],      # mixed; expert 4 from the fp16 fallback to 6 bit-planes
    [4, 6, 3, 5, 16, 5],
]


def _paged(cfg, bits0, arena_bytes=None):
    import torch
    inp = G.inputs(cfg)
    pe = PagedExperts(inp.experts, cfg.H, cfg.I,
                      arena_bytes if arena_bytes is not None else arena_bytes_for(cfg.H, cfg.I, cfg.E))
    shared = ExpertTable([inp.shared]) if inp.shared is not None else None
    layer = MoELayer(cfg.E, cfg.H, cfg.I, cfg.k, cfg.T, inp.w_router, inp.bias, cfg.logit_scale, pe.table,
                     bits0, shared, cfg.shared_I)
    pe.attach(layer, bits0)
    torch.cuda.synchronize()
    return inp, pe, layer


def _forward(inp, layer):
    import torch
    x = torch.from_numpy(np.ascontiguousarray(inp.x).view(np.int16)).cuda().view(torch.float16)
    out = layer.forward(x).clone()
    torch.cuda.synchronize()
    return out.float().cpu().numpy()


def _check_resident(pe, layer, bits):
    """Descriptor words of every paged matrix point into the arena at blocks
    that hold exactly the host copy's top b planes and b-bit LUT."""
    import torch
    torch.cuda.synchronize()
    n = layer.n_shared
    desc = layer.table.desc[n:].cpu().numpy().astype(np.uint64)
    dbits = layer.bits[n:].cpu().numpy()
    assert dbits.tolist() == [int(b) for b in bits]
    arena = pe.arena.cpu().numpy()
    base = pe.arena.data_ptr()
    for e, b in enumerate(bits):
        b = int(b)
        for j, name in enumerate(MATS):
            words = desc[e, 6 * j: 6 * j + 6]
            w16 = pe.table.tensors[e][name]["w16"]
            assert int(words[5]) == (0 if w16 is None else w16.data_ptr()), "w16 word left alone"
            if b == 16:
                assert words[:5].tolist() == [0] * 5
                continue
            host = pe.host_planes[3 * e + j].numpy().view(np.uint8)
            slab = host.size // 6
            off = int(words[0]) - base
            assert 0 <= off and off + b * slab <= arena.size and off % 256 == 0
            assert np.array_equal(arena[off:off + b * slab], host[:b * slab]), f"planes of expert {e} {name}"
            for bb in range(3, 7):
                if bb != b:
                    assert int(words[1 + bb - 3]) == 0
            lut = pe.host_luts[4 * (3 * e + j) + b - 3].numpy().view(np.uint8).reshape(-1)
            lo = int(words[1 + b - 3]) - base
            assert 0 <= lo and lo + lut.size <= arena.size and lo % 256 == 0
            assert np.array_equal(arena[lo:lo + lut.size], lut), f"LUT of expert {e} {name}"


@pytest.mark.parametrize("cfg", [PAGED, RAGGED], ids=lambda c: c.name)
def test_paged_layer_follows_every_plan(cfg):
    G.say(f"paged layer {cfg.name}")
    bits0 = list(cfg.bits)
    inp, pe, layer = _paged(cfg, bits0)
    exact = cfg.H % 128 == 0 and cfg.I % 128 == 0
    prev = bits0
    for bits in [bits0] + PLANS:
        if bits is not bits0:
            assert pe.apply(bits) == _lib.OK
        st = pe.stats()
        if exact:
            assert st["resident"] == paging.resident_bytes(cfg.H, cfg.I, bits)
            if bits is not bits0:
                assert st["h2d"] == paging.host_to_device_bytes(cfg.H, cfg.I, prev, bits)
        if bits is PLANS[0]:
            assert st["d2d"] > 0, "blocks packed back to back: a promotion moves them"
            # staged: one host-to-device range per expert and step
            assert st["ranges"] <= sum(max(0, 6 - (0 if b == 16 else b)) for b in prev), st
        _check_resident(pe, layer, bits)
        got = _forward(inp, layer)
        G.check_out({"out": got}, moe.layer(inp, bits=np.asarray(bits, np.int8)))
        G.say(f"  bits {bits}: resident {st['resident']} h2d {st['h2d']} d2d {st['d2d']}")
        prev = bits
    pe.close()


def test_paging_grows_in_place_after_retire():
    """A demotion's tails return to the arena once the stream has passed its
    commit; promoting back then grows every block in place (no device-to-device
    move)."""
    import torch
    cfg = PAGED
    inp, pe, layer = _paged(cfg, [6] * cfg.E)
    assert pe.apply([3] * cfg.E) == _lib.OK
    torch.cuda.synchronize()
    assert pe.apply([6] * cfg.E) == _lib.OK
    st = pe.stats()
    assert st["d2d"] == 0 and st["h2d"] == paging.host_to_device_bytes(cfg.H, cfg.I, [3] * cfg.E, [6] * cfg.E)
    _check_resident(pe, layer, [6] * cfg.E)
    G.check_out({"out": _forward(inp, layer)}, moe.layer(inp, bits=np.full(cfg.E, 6, np.int8)))
    pe.close()


def test_paging_commit_in_stream_order():
    """Copies staged, a forward call enqueued before the commit runs at the
    old bitwidths, one enqueued after it at the new."""
    import torch
    cfg = PAGED
    inp, pe, layer = _paged(cfg, list(cfg.bits))
    old, new = list(cfg.bits), [6, 6, 6, 6, 6, 6]
    x = torch.from_numpy(np.ascontiguousarray(inp.x).view(np.int16)).cuda().view(torch.float16)
    assert pe.stage(new) == _lib.OK
    out1 = layer.forward(x).clone()
    pe.commit(new)
    out2 = layer.forward(x).clone()
    torch.cuda.synchronize()
    G.check_out({"out": out1.float().cpu().numpy()}, moe.layer(inp, bits=np.asarray(old, np.int8)))
    G.check_out({"out": out2.float().cpu().numpy()}, moe.layer(inp, bits=np.asarray(new, np.int8)))
    _check_resident(pe, layer, new)
    pe.close()


def test_paging_enospace_keeps_the_plan():
    """An arena that holds the 3-bit plan but not the 6-bit one: staging the
    promotion fails with nothing changed, and the layer keeps its plan."""
    cfg = PAGED
    small = paging.resident_bytes(cfg.H, cfg.I, [3] * cfg.E) + 64 * 1024
    inp, pe, layer = _paged(cfg, [3] * cfg.E, arena_bytes=small)
    before = pe.stats()
    assert pe.apply([6] * cfg.E) == _lib.ENOSPACE
    after = pe.stats()
    assert after["resident"] == before["resident"] and after["free"] == before["free"]
    _check_resident(pe, layer, [3] * cfg.E)
    G.check_out({"out": _forward(inp, layer)}, moe.layer(inp, bits=np.full(cfg.E, 3, np.int8)))
    pe.close()


def test_paging_copies_into_place_without_room_to_stage():
    """An arena that holds the 3-bit blocks and the moved 6-bit blocks side by
    side but not a staging block as well: the promotion copies each matrix's
    planes and LUT straight into place (three plane ranges per step and three
    LUT ranges per expert), and the result is the same."""
    cfg = PAGED
    routed = [e for e in range(cfg.E)]
    arena = paging.resident_bytes(cfg.H, cfg.I, [3] * cfg.E) + paging.resident_bytes(cfg.H, cfg.I, [6] * cfg.E) \
        + 64 * 1024
    inp, pe, layer = _paged(cfg, [3] * cfg.E, arena_bytes=arena)
    assert pe.apply([6] * cfg.E) == _lib.OK
    st = pe.stats()
    assert st["ranges"] == len(routed) * (3 * 3 + 3), st
    assert st["h2d"] == paging.host_to_device_bytes(cfg.H, cfg.I, [3] * cfg.E, [6] * cfg.E)
    assert st["d2d"] > 0
    _check_resident(pe, layer, [6] * cfg.E)
    G.check_out({"out": _forward(inp, layer)}, moe.layer(inp, bits=np.full(cfg.E, 6, np.int8)))
    # and back down: the 3-bit LUTs only, staged now that the old 3-bit blocks are free again
    assert pe.apply([3] * cfg.E) == _lib.OK
    _check_resident(pe, layer, [3] * cfg.E)
    G.check_out({"out": _forward(inp, layer)}, moe.layer(inp, bits=np.full(cfg.E, 3, np.int8)))
    pe.close()


@pytest.mark.parametrize("seed,room", [(1, "roomy"), (2, "middle"), (3, "tight")])
def test_paging_random_plans(seed, room):
    """Seeded random plans on the ragged layer in three arena sizes (twice the
    6-bit residency; the 3-bit and the 6-bit residency side by side; the 6-bit
    residency alone, plus 256 KB): stages go through the staging block,
    straight into place when it does not fit, or fail with ENOSPACE and change
    nothing.  After every plan the resident blocks equal the host copy and the
    layer equals the oracle at the bitwidths in force."""
    cfg = RAGGED
    rng = np.random.default_rng(seed)
    lo = paging.resident_bytes(cfg.H, cfg.I, [3] * cfg.E)
    hi = paging.resident_bytes(cfg.H, cfg.I, [6] * cfg.E)
    arena = {"roomy": 2 * hi, "middle": lo + hi, "tight": hi}[room] + 256 * 1024
    bits = [int(b) for b in cfg.bits]
    inp, pe, layer = _paged(cfg, bits, arena_bytes=arena)
    G.say(f"paging random plans seed {seed}")
    staged = direct = refused = 0
    for _ in range(10):
        new = [int(rng.choice([3, 4, 5, 6])) for _ in range(cfg.E)]
        if rng.random() < 0.5:
            new[4] = 16                               # the expert with fp16 weights
        rc = pe.apply(new)
        if rc == _lib.ENOSPACE:
            refused += 1
        else:
            assert rc == _lib.OK
            st = pe.stats()
            moved = sum(max(0, (0 if b == 16 else b) - (0 if a == 16 else a)) for a, b in zip(bits, new))
            if moved:   # a promotion: staged ranges are at most one per expert and step
                staged += st["ranges"] <= moved
                direct += st["ranges"] > moved
            bits = new
        _check_resident(pe, layer, bits)
        G.check_out({"out": _forward(inp, layer)}, moe.layer(inp, bits=np.asarray(bits, np.int8)))
    G.say(f"  {room}: staged {staged} direct {direct} refused {refused}")
    # each arena reaches the path it is sized for (the plans are seeded)
    assert {"roomy": staged, "middle": direct, "tight": refused}[room] > 0
    pe.close()


def test_paged_qwen_decode_full_size():
    """The Qwen-shaped decode layer (60 experts, four always-on fp16 experts
    in front of them in the descriptor table) on paged weights, before and
    after demoting the ten lowest-indexed 6-bit experts by one bit."""
    cfg = synth.get("qwen_decode")
    G.say("paged qwen_decode")
    inp0 = G.inputs(cfg)
    bits0 = resolve_bits(inp0)
    inp, pe, layer = _paged(cfg, bits0)
    assert layer.n_shared == 4
    G.check_out({"out": _forward(inp, layer)}, layer_ref(inp, bits0))
    bits1 = np.array(bits0, np.int8)
    six = np.nonzero(bits1 == 6)[0][:10]
    bits1[six] = 5
    assert pe.apply(bits1) == _lib.OK
    _check_resident(pe, layer, bits1)
    G.check_out({"out": _forward(inp, layer)}, layer_ref(inp, bits1))
    G.say(f"  demoted {len(six)} experts; {pe.stats()}")
    pe.close()


def test_online_planner_on_paged_layer_goes_through_the_pager():
    """The online planner on a paged layer: every changed plan is staged by the
    pager and committed with its planes and LUTs, so the next forward runs at
    the new bitwidths on resident blocks (output against the oracle at those
    bitwidths, blocks against the host copy), while the KV footprint grows and
    then shrinks."""
    from any_precision_quantized_amd.layer import OnlinePlanner
    cfg = PAGED
    bits0 = [6, 6, 6, 6, 6, 6]
    inp, pe, layer = _paged(cfg, bits0)
    levels = [6, 5, 4, 3]
    nbytes = np.array([[paging_bytes(cfg, b) for b in levels]] * cfg.E, dtype=np.uint64)
    harm = np.array([[0.0, 1.0, 3.0, 7.0]] * cfg.E) * (1 + np.arange(cfg.E))[:, None]
    planner_ = OnlinePlanner(layer, levels, harm, nbytes, [3] * cfg.E, [5, 4, 3],
                             m_total=int(nbytes[:, 0].sum()), hysteresis=0, bits_now=bits0)
    step = int(nbytes[0, 0] - nbytes[0, 2])
    seen = set()
    for m_kv in (step, 3 * step, 6 * step, 2 * step, 0):
        st, bits, stage, changed = planner_.step(m_kv=m_kv)
        assert st == _lib.OK
        G.say(f"  m_kv {m_kv}: bits {bits.tolist()} stage {stage} changed {changed}")
        out = _forward(inp, layer)
        _check_resident(pe, layer, bits)
        G.check_out({"out": out}, moe.layer(inp, bits=bits))
        seen.add(tuple(bits.tolist()))
    assert len(seen) >= 3, "the sweep should move through several plans"
    pe.close()


def paging_bytes(cfg, b):
    """Plane + LUT bytes of one expert's three matrices at b bits."""
    return 3 * (cfg.H * cfg.I * b // 8) + (2 * cfg.I + cfg.H) * (1 << b) * 2
