"""Oracle of plane paging: what a change of bitwidths must keep resident and move.

Test infrastructure only: the tests, the smoke entry point and the CPU leg of
the benchmark use it; the library never does.

The paging page treats the bit-planes (and the LUTs) of each expert as pages:
demoting an expert drops its low planes, promoting it brings them back from the
host, and the changes are committed at a safe boundary while the movement runs
asynchronously ("内存的饥饿游戏：当 MoE 权重与 KV 缓存争夺 GPU 的每一字节",
zhichai.net, sections "核心洞察：权重也能分页" and "安全边界与异步搬运").
Readings taken here (the page gives no sizes or layouts):
  * an expert at b in {3,4,5,6} bits keeps planes 0..b-1 (the most significant
    b bits of each 6-bit code, which is what makes the precisions nested) and
    its b-bit LUT, for each of gate, up and down; at 16 bits it keeps neither;
  * one plane of a rows x cols matrix is rows * cols / 8 bytes and the b-bit
    LUT is rows * 2**b fp16 entries;
  * a promotion from b to b' copies planes b..b'-1 and the b'-bit LUT from the
    host; a demotion copies nothing; a change of bitwidth replaces the LUT.

The device memory is carved by a first-fit allocator.  `FirstFit` below is
the plain definition: a bitmap of 256-byte units, allocation takes the lowest
run of free units long enough, release frees units that are all in use.
"""
from __future__ import annotations

import numpy as np

UNIT = 256


def plane_bytes(rows, cols):
    """Bytes of one bit-plane of a rows x cols matrix (one bit per weight)."""
    return rows * cols // 8


def lut_bytes(rows, b):
    """Bytes of the b-bit LUT of a rows-row matrix (2**b fp16 entries a row)."""
    return rows * (1 << b) * 2


def expert_mats(H, I):
    """(rows, cols) of gate, up and down: gate and up are I x H, down is H x I."""
    return [(I, H), (I, H), (H, I)]


def resident_bytes(H, I, bits):
    """Plane and LUT bytes resident for every expert at its bitwidth."""
    total = 0
    for b in bits:
        b = int(b)
        if b == 16:
            continue
        for rows, cols in expert_mats(H, I):
            total += b * plane_bytes(rows, cols) + lut_bytes(rows, b)
    return total


def host_to_device_bytes(H, I, bits_old, bits_new):
    """Bytes a change of bitwidths copies from the host: the planes that
    become resident and the LUT of every expert whose bitwidth changes to a
    bit-plane one."""
    total = 0
    for bo, bn in zip(bits_old, bits_new):
        have = 0 if int(bo) == 16 else int(bo)
        want = 0 if int(bn) == 16 else int(bn)
        for rows, cols in expert_mats(H, I):
            if want > have:
                total += (want - have) * plane_bytes(rows, cols)
            if want != have and want:
                total += lut_bytes(rows, want)
    return total


class FirstFit:
    """Bitmap first-fit allocator over [0, size) in 256-byte units."""

    def __init__(self, size):
        self.n = size // UNIT
        self.used = np.zeros(self.n, dtype=bool)

    @staticmethod
    def units(nbytes):
        return -(-int(nbytes) // UNIT)

    def alloc(self, nbytes):
        """Offset of the lowest run of free units that holds nbytes, or None."""
        k = self.units(nbytes)
        if k == 0:
            raise ValueError("zero-byte allocation")
        run = 0
        for i in range(self.n):
            run = run + 1 if not self.used[i] else 0
            if run == k:
                start = i - k + 1
                self.used[start:i + 1] = True
                return start * UNIT
        return None

    def take(self, off, nbytes):
        """Claim exactly [off, off + nbytes) if every unit of it is free."""
        k = self.units(nbytes)
        u = off // UNIT
        if k == 0:
            return True
        if u + k > self.n or self.used[u:u + k].any():
            return False
        self.used[u:u + k] = True
        return True

    def release(self, off, nbytes):
        """Free [off, off + nbytes); False (no change) unless all of it is in use."""
        k = self.units(nbytes)
        if k == 0:
            return True
        if off % UNIT or off // UNIT + k > self.n:
            return False
        u = off // UNIT
        if not self.used[u:u + k].all():
            return False
        self.used[u:u + k] = False
        return True

    def stats(self):
        """(free bytes, largest free run in bytes, number of free runs)."""
        free = int((~self.used).sum())
        largest = runs = cur = 0
        for i in range(self.n):
            if not self.used[i]:
                cur += 1
                if cur == 1:
                    runs += 1
                largest = max(largest, cur)
            else:
                cur = 0
        return free * UNIT, largest * UNIT, runs
