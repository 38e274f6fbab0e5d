"""Paged expert weights: bit-planes and LUTs resident only as deep as each
expert's bitwidth, moved between host and GPU by the library's pager.

``PagedExperts`` keeps a host copy of every routed expert's packed planes
and LUTs (the pager takes its own pinned copy of them when it is created) and
a device arena for the resident part.  Its
``ExpertTable`` carries only the fp16 weights (for experts that may run at 16
bits); plane and LUT pointers are written by the pager's commits.  After
``attach(layer)`` the layer runs on the paged weights, and ``apply(bits)``
stages the copies on a copy stream and commits the new residency together
with the bitwidths in the layer's stream, so calls enqueued before the
commit run at the old bitwidths and later ones at the new.
"""
from __future__ import annotations

import ctypes

import numpy as np

from . import _lib
from .layer import MATS, ExpertTable


def _hip():
    return ctypes.CDLL("libamdhip64.so")


def _shares_queue(busy, cand):
    """True when `cand` sits in the same hardware queue as `busy`: an event
    recorded on the idle `cand` behind a few milliseconds of spinning on
    `busy` is still pending half a millisecond later, while the spin is.  In
    a queue of its own it completes at once."""
    import time

    import torch
    with torch.cuda.stream(busy):
        torch.cuda._sleep(10_000_000)   # a few ms of one spinning wave
        spun = torch.cuda.Event()
        spun.record(busy)
    mark = torch.cuda.Event()
    mark.record(cand)
    time.sleep(0.0005)
    waited = not mark.query() and not spun.query()
    busy.synchronize()
    cand.synchronize()
    return waited


def _copy_stream(device):
    """A non-blocking stream made with HIP itself for the pager's copies, in a
    hardware queue other than the current stream's.  Streams share a few
    hardware queues (four per process here).  A copy stream in the layer
    stream's queue was measured to make the copies' completion visible only
    once the layer's queued work had run, and an event recorded on it behind
    the copies to hold the layer up for the whole copy, so candidates that
    share the current stream's queue are set aside (and destroyed)."""
    import torch
    hip = _hip()
    busy = torch.cuda.current_stream(device)
    rejected = []
    chosen = None
    try:
        with torch.cuda.device(device):
            for _ in range(8):
                s = ctypes.c_void_p()
                rc = hip.hipStreamCreateWithFlags(ctypes.byref(s), ctypes.c_uint(1))   # hipStreamNonBlocking
                if rc != 0:
                    raise RuntimeError(f"hipStreamCreateWithFlags failed ({rc})")
                cand = torch.cuda.ExternalStream(s.value, device=device)
                if not _shares_queue(busy, cand):
                    chosen = cand
                    break
                rejected.append(s.value)
            if chosen is None:   # every candidate shared it: keep the last
                chosen = torch.cuda.ExternalStream(rejected.pop(), device=device)
    finally:
        for v in rejected:
            hip.hipStreamDestroy(ctypes.c_void_p(v))
    return chosen


def arena_bytes_for(H, I, E, bits_max=6, slack=1.25):
    """Arena size that holds E experts at bits_max with room to move blocks."""
    words = _lib.packed_plane_words
    per = 0
    for rows, cols in ((I, H), (I, H), (H, I)):
        per += words(rows, cols) // 6 * 4 * bits_max + rows * (1 << bits_max) * 2 + 512
    return int(per * E * slack) + (1 << 20)


class PagedExperts:
    def __init__(self, experts, H, I, arena_bytes, device="cuda"):
        """experts: per expert a mapping gate/up/down -> matrix with canonical
        ``planes`` uint32 [6, rows, cols/32], ``luts`` (four fp16 [rows, 2**b])
        and optional ``w16``.  The planes are packed once on the device (the
        layout the kernels read) and copied to host memory."""
        import torch
        self.E, self.H, self.I = len(experts), H, I
        self.device = device
        self.host_planes, self.host_luts = [], []
        tensors = []
        for mats in experts:
            d = {}
            for name in MATS:
                m = mats[name]
                rows, cols = m.planes.shape[1], m.planes.shape[2] * 32
                canon = torch.from_numpy(np.ascontiguousarray(m.planes).view(np.int32)).to(device)
                packed = torch.empty(_lib.packed_plane_words(rows, cols), dtype=torch.int32, device=device)
                _lib.pack_planes(canon, rows, cols, packed)
                host = torch.empty(packed.numel(), dtype=torch.int32)
                host.copy_(packed)
                self.host_planes.append(host)
                for b in range(3, 7):
                    lut = torch.empty((rows, 1 << b), dtype=torch.int16)
                    lut.copy_(torch.from_numpy(np.ascontiguousarray(m.luts[b - 3]).view(np.int16)))
                    self.host_luts.append(lut)
                w16 = None
                if m.w16 is not None:
                    w16 = torch.from_numpy(np.ascontiguousarray(m.w16).view(np.int16)).to(device)
                d[name] = {"planes": None, "luts": [None] * 4, "w16": w16}
            tensors.append(d)
        torch.cuda.synchronize()
        self.table = ExpertTable(None, device, _tensors=tensors)
        self.arena = torch.empty(int(arena_bytes), dtype=torch.uint8, device=device)
        self.pager = None
        self.layer = None
        self.bits = None
        self.copy_stream = _copy_stream(device)

    def has_w16(self, e):
        return all(self.table.tensors[e][name]["w16"] is not None for name in MATS)

    def attach(self, layer, bits):
        """Bind the pager to the layer's descriptor table and bits (the routed
        part), then make `bits` resident and commit them."""
        assert layer.experts is self.table, "build the layer on PagedExperts.table"
        n = layer.n_shared
        self.layer = layer
        self.pager = _lib.Pager(self.E, self.H, self.I, self.host_planes, self.host_luts, self.arena,
                                layer.table.desc[n:], layer.bits[n:])
        self.bits = np.zeros(self.E, dtype=np.int8)
        rc = self.apply(bits)
        if rc != _lib.OK:
            raise _lib.ApmoeError(rc, "initial residency")
        layer.pager = self    # later plans (commit, replan, OnlinePlanner) go through apply

    def _check16(self, bits):
        for e, b in enumerate(bits):
            if int(b) == 16 and not self.has_w16(e):
                raise ValueError(f"expert {e} has no fp16 weights to run at 16 bits")

    def stage(self, bits):
        """Enqueue the copies for `bits` on the copy stream; OK or ENOSPACE."""
        bits = np.asarray(bits, dtype=np.int8)
        self._check16(bits)
        return self.pager.stage(bits, self.copy_stream)

    def commit(self, bits, stream=None):
        """Commit the staged residency and `bits` in `stream` (default: current)."""
        self.pager.commit(stream)
        self.bits = np.asarray(bits, dtype=np.int8).copy()

    def apply(self, bits, stream=None):
        """stage + commit; returns OK, or ENOSPACE with nothing changed."""
        rc = self.stage(bits)
        if rc == _lib.OK:
            self.commit(bits, stream)
        return rc

    def stats(self):
        return self.pager.stats()

    def close(self):
        if self.pager is not None:
            self.pager.close()
            self.pager = None
        if self.copy_stream is not None:
            _hip().hipStreamDestroy(ctypes.c_void_p(self.copy_stream.cuda_stream))
            self.copy_stream = None
