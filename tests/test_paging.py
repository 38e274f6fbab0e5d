"""Pins of the paging oracle: hand-worked residency and copy bytes and a
hand-worked first-fit sequence."""
import numpy as np

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
