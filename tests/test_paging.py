"""Plane paging on the CPU: pins of the paging oracle (hand-worked residency
and copy bytes, a hand-worked first-fit sequence), the native arena allocator
against the oracle's bitmap first-fit on seeded operation sequences, and the
pager's argument checks (no GPU call is reached)."""
import ctypes

import numpy as np
import pytest

from any_precision_quantized_amd import _lib
from oracle import paging


# ---------------------------------------------------------------------------
# Oracle pins
# ---------------------------------------------------------------------------

def test_resident_bytes_hand_example():
    # H = 256, I = 128: every plane of gate, up (128 x 256) and down (256 x 128) is 4096 bytes
    # 3 bits: 3 planes x 3 mats + LUTs of 8 entries: 2048 + 2048 + 4096
    # 6 bits: 6 planes x 3 mats + LUTs of 64 entries: 16384 + 16384 + 32768
    assert paging.resident_bytes(256, 128, [3]) == 36864 + 8192
    assert paging.resident_bytes(256, 128, [6]) == 73728 + 65536
    assert paging.resident_bytes(256, 128, [16]) == 0
    assert paging.resident_bytes(256, 128, [3, 16, 6]) == 45056 + 139264


def test_host_to_device_bytes_hand_example():
    H, I = 256, 128
    # 3 -> 5: planes 3, 4 of each matrix (2 x 4096 x 3) and the 5-bit LUTs (8192 + 8192 + 16384)
    assert paging.host_to_device_bytes(H, I, [3], [5]) == 24576 + 32768
    # 16 -> 4: four planes of each matrix and the 4-bit LUTs (4096 + 4096 + 8192)
    assert paging.host_to_device_bytes(H, I, [16], [4]) == 49152 + 16384
    # 6 -> 3: no plane moves, the 3-bit LUTs do
    assert paging.host_to_device_bytes(H, I, [6], [3]) == 8192
    # 5 -> 16 and no change: nothing
    assert paging.host_to_device_bytes(H, I, [5], [16]) == 0
    assert paging.host_to_device_bytes(H, I, [4, 6], [4, 6]) == 0
    assert paging.host_to_device_bytes(H, I, [3, 16, 6], [5, 4, 6]) == 57344 + 65536


def test_promote_then_demote_restores_residency():
    H, I = 512, 384
    rng = np.random.default_rng(3)
    levels = np.array([3, 4, 5, 6, 16])
    for _ in range(20):
        a, b = rng.choice(levels, 6), rng.choice(levels, 6)
        # residency depends only on the bits; what moves up one way costs at least the plane bytes
        assert paging.resident_bytes(H, I, a) + paging.resident_bytes(H, I, b) == \
            paging.resident_bytes(H, I, np.concatenate([a, b]))
        up = paging.host_to_device_bytes(H, I, a, b)
        gain = sum(max(0, (0 if y == 16 else y) - (0 if x == 16 else x)) for x, y in zip(a, b))
        assert up >= gain * sum(paging.plane_bytes(r, c) for r, c in paging.expert_mats(H, I))


def test_first_fit_hand_sequence():
    a = paging.FirstFit(2048)                  # 8 units of 256 bytes
    assert a.alloc(300) == 0                   # units 0-1
    assert a.alloc(256) == 512                 # unit 2
    assert a.alloc(1000) == 768                # units 3-6
    assert a.alloc(512) is None                # only unit 7 is free
    assert a.stats() == (256, 256, 1)
    assert a.release(512, 256)                 # unit 2 free again
    assert a.alloc(200) == 512                 # first fit takes the hole, not unit 7
    assert a.release(0, 512)
    assert a.stats() == (768, 512, 2)
    assert a.alloc(768) is None                # 768 free bytes, but in two runs
    assert not a.release(0, 512)               # already free
    assert not a.release(256, 512)             # partly free
    assert a.take(1792, 256) and not a.take(1792, 256)
    assert a.take(0, 300) and a.stats() == (0, 0, 0)


# ---------------------------------------------------------------------------
# Native arena against the oracle
# ---------------------------------------------------------------------------

def _apply(arena, ff, op, arg):
    if op == "alloc":
        return arena.alloc(arg), ff.alloc(arg)
    if op == "take":
        off, n = arg
        return arena.take(off, n), ff.take(off, n)
    off, n = arg
    return arena.release(off, n) == _lib.OK, ff.release(off, n)


@pytest.mark.parametrize("seed", range(8))
def test_native_arena_matches_first_fit(seed):
    rng = np.random.default_rng(seed)
    size = 256 * int(rng.integers(16, 96))
    arena, ff = _lib.Arena(size), paging.FirstFit(size)
    live = []
    for step in range(400):
        r = rng.random()
        if r < 0.45 or not live:
            op, arg = "alloc", int(rng.integers(1, size // 6))
        elif r < 0.8:
            i = int(rng.integers(len(live)))
            off, n = live[i]
            if rng.random() < 0.3:       # part of a live range: the tail, as a demotion frees
                cut = 256 * int(rng.integers(0, max(1, n // 256)))
                op, arg = "release", (off + cut, n - cut)
            else:
                op, arg = "release", (off, n)
        elif r < 0.9:
            op, arg = "take", (256 * int(rng.integers(0, size // 256)), int(rng.integers(1, 1024)))
        else:                            # a bad release: free memory or past the end
            op, arg = "release", (256 * int(rng.integers(0, size // 256 + 2)), 256 * int(rng.integers(1, 6)))
        got, want = _apply(arena, ff, op, arg)
        assert got == want, (step, op, arg, got, want)
        assert arena.stats() == ff.stats(), (step, op, arg)
        if op == "alloc" and got is not None:
            live.append((got, 256 * paging.FirstFit.units(arg)))
        elif op == "release" and got:
            off, n = arg
            n = 256 * paging.FirstFit.units(n)
            for j, (o, m) in enumerate(live):
                if o <= off < o + m:
                    live[j] = (o, off - o)
                    if off - o == 0:
                        live.pop(j)
                    break
        elif op == "take" and got:
            live.append((arg[0], 256 * paging.FirstFit.units(arg[1])))


def test_native_arena_argument_errors():
    lib = _lib._lib()
    a = _lib.Arena(4096)
    off = ctypes.c_uint64()
    assert lib.apmoe_arena_alloc(a._h, 0, ctypes.byref(off)) == _lib.EINVAL
    assert lib.apmoe_arena_take(a._h, 100, 256) == _lib.EINVAL        # misaligned
    assert lib.apmoe_arena_release(a._h, 4096, 256) == _lib.EINVAL    # past the end
    assert lib.apmoe_arena_release(a._h, 0, 256) == _lib.EINVAL       # already free
    assert lib.apmoe_arena_alloc(a._h, 8192, ctypes.byref(off)) == _lib.ENOSPACE
    assert lib.apmoe_arena_create(4096, None) == _lib.EINVAL
    assert a.stats() == (4096, 4096, 1)


# ---------------------------------------------------------------------------
# Pager argument checks (rejected before any GPU call)
# ---------------------------------------------------------------------------

def test_pager_create_argument_errors():
    lib = _lib._lib()
    E, H, I = 2, 64, 96
    fake = ctypes.c_void_p(1 << 20)
    hp = (ctypes.c_void_p * (3 * E))(*([1 << 20] * 3 * E))
    hl = (ctypes.c_void_p * (12 * E))(*([1 << 20] * 12 * E))
    out = ctypes.c_void_p()
    big = 1 << 30
    assert lib.apmoe_pager_create(0, H, I, hp, hl, fake, big, fake, fake, ctypes.byref(out)) == _lib.EINVAL
    assert lib.apmoe_pager_create(E, 48, I, hp, hl, fake, big, fake, fake, ctypes.byref(out)) == _lib.EINVAL
    assert lib.apmoe_pager_create(E, H, 80, hp, hl, fake, big, fake, fake, ctypes.byref(out)) == _lib.EINVAL
    assert lib.apmoe_pager_create(E, H, I, None, hl, fake, big, fake, fake, ctypes.byref(out)) == _lib.EINVAL
    assert lib.apmoe_pager_create(E, H, I, hp, hl, ctypes.c_void_p((1 << 20) + 64), big, fake, fake,
                                  ctypes.byref(out)) == _lib.EINVAL     # arena not 256-aligned
    hl_null = (ctypes.c_void_p * (12 * E))(*([1 << 20] * (12 * E - 1) + [None]))
    assert lib.apmoe_pager_create(E, H, I, hp, hl_null, fake, big, fake, fake, ctypes.byref(out)) == _lib.EINVAL
    assert lib.apmoe_pager_create(E, H, I, hp, hl, fake, big, fake, fake, None) == _lib.EINVAL
    # the patch buffer (3E x 5 pointer patches and the bits) does not fit
    assert lib.apmoe_pager_create(E, H, I, hp, hl, fake, 256, fake, fake, ctypes.byref(out)) == _lib.ENOSPACE
    assert out.value is None
    for fn in ("apmoe_pager_stage", "apmoe_pager_commit", "apmoe_pager_stats"):
        args = {"apmoe_pager_stage": (None, None, None), "apmoe_pager_commit": (None, None),
                "apmoe_pager_stats": (None, None, None, None, None, None, None)}[fn]
        assert getattr(lib, fn)(*args) == _lib.EINVAL
    assert lib.apmoe_pager_destroy(None) == _lib.OK


def test_pager_binding_rejects_short_host_copies():
    """The pager reads the host planes and LUTs once, at create: the binding
    refuses host tensors smaller than a matrix's packed planes or b-bit LUT
    before any library call."""
    import torch
    E, H, I = 2, 64, 96
    planes = [torch.zeros(_lib.packed_plane_words(I if i % 3 < 2 else H, H if i % 3 < 2 else I), dtype=torch.int32)
              for i in range(3 * E)]
    luts = [torch.zeros((I if (i // 4) % 3 < 2 else H, 1 << (3 + i % 4)), dtype=torch.int16) for i in range(12 * E)]
    dummy = torch.zeros(1)
    short = list(planes)
    short[4] = planes[4][:-1]   # expert 1, up: one word short
    with pytest.raises(ValueError, match="host planes 4"):
        _lib.Pager(E, H, I, short, luts, dummy, dummy, dummy)
    short = list(luts)
    short[4 * 5 + 2] = luts[4 * 5 + 2][:-1]   # expert 1, down, 5-bit LUT: one row short
    with pytest.raises(ValueError, match="host LUT 5, 5 bits"):
        _lib.Pager(E, H, I, planes, short, dummy, dummy, dummy)


class _FakePager:
    """Stands in for PagedExperts on the host: records the plans it is asked
    to make resident and answers with a fixed status."""

    def __init__(self, status):
        self.status = status
        self.applied = []

    def apply(self, bits, stream=None):
        self.applied.append([int(b) for b in bits])
        return self.status


class _HostLayer:
    """The attributes MoELayer.commit and replan read, without device memory."""

    def __init__(self, pager):
        self.pager = pager
        self.n_shared = 0
        self.bits = None

    commit = __import__("any_precision_quantized_amd.layer", fromlist=["MoELayer"]).MoELayer.commit


def test_plans_on_paged_layer_go_through_the_pager(monkeypatch):
    """With a pager attached, a commit (directly, or from the online planner)
    stages the new residency through the pager instead of writing the bits
    table alone, which would point the kernels at planes that are not
    resident; when the pager cannot hold the plan the planner keeps its old
    plan.  No GPU work is enqueued: the device bits write is replaced by a
    trap."""
    from any_precision_quantized_amd import layer as L

    def no_direct_write(*a, **k):
        raise AssertionError("bits table written without the pager")

    monkeypatch.setattr(_lib, "commit_bits", no_direct_write)
    ok = _FakePager(_lib.OK)
    lay = _HostLayer(ok)
    assert lay.commit([6, 5, 4]) == _lib.OK
    assert ok.applied == [[6, 5, 4]]

    levels = [6, 5, 4, 3]
    nbytes = np.array([[600, 500, 400, 300]] * 3, dtype=np.uint64)
    harm = np.array([[0.0, 1.0, 3.0, 7.0]] * 3) * np.array([[1.0], [2.0], [3.0]])
    planner = L.OnlinePlanner(lay, levels, harm, nbytes, [3] * 3, [5, 4, 3], m_total=1800, hysteresis=0,
                              bits_now=[6, 6, 6])
    st, bits, stage, changed = planner.step(m_kv=400)          # budget 1400: a demotion is needed
    assert st == _lib.OK and changed and ok.applied[-1] == bits.tolist()
    assert planner.bits.tolist() == bits.tolist()

    full = _FakePager(_lib.ENOSPACE)
    lay2 = _HostLayer(full)
    planner2 = L.OnlinePlanner(lay2, levels, harm, nbytes, [3] * 3, [5, 4, 3], m_total=1800, hysteresis=0,
                               bits_now=[6, 6, 6])
    st, bits, stage, changed = planner2.step(m_kv=400)
    assert st == _lib.ENOSPACE and not changed
    assert len(full.applied) == 1 and planner2.bits.tolist() == [6, 6, 6] and bits.tolist() == [6, 6, 6]
