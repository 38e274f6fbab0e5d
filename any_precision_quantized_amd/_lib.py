"""ctypes binding of libapmoe.so (C ABI in include/apmoe.h).

Argument marshalling only: every function here checks dtypes, devices and
sizes of torch tensors on the host, takes their device pointers and the
current HIP stream, and calls the entry point of the same name.  All compute
runs in the library's HIP kernels.  There is no fallback: a missing or
unloadable library raises ApmoeError.
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libapmoe.so")
HEADER = os.path.join(os.path.dirname(_HERE), "include", "apmoe.h")

OK, EINVAL, EBITS, ENOSPACE, EHIP = 0, -1, -2, -3, -4
GATE_UP_SWIGLU, DOWN = 0, 1
ONLY_GEMV, ONLY_TILE = 0x10, 0x20
MAX_EXPERTS = 256

_c_int, _c_size, _vp, _u64 = ctypes.c_int, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_uint64


class ApmoeError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        msg = _lib().apmoe_strerror(code).decode() if code < 0 else "library not available"
        super().__init__(f"{where}: {msg} ({code})")


_LIB = None


def _lib():
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m any_precision_quantized_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        sig = {
            "apmoe_route": [_vp, _c_int, _c_int, _vp, _vp, ctypes.c_float, _c_int, _c_int, _vp, _vp, _vp, _vp,
                            _c_size, _vp],
            "apmoe_route_stats": [_vp, _c_int, _c_int, _vp, _vp, _c_int, _c_int, _vp, _vp, _vp, _c_size, _vp],
            "apmoe_permute": [_vp, _c_int, _c_int, _c_int, _c_int, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                              _c_size, _vp],
            "apmoe_bitplane_lut_gemm": [_c_int, _vp, _vp, _c_int, _vp, _vp, _c_int, _vp, _vp, _c_int,
                                        _c_int, _c_int, _c_int, _vp, _c_size, _vp],
            "apmoe_bitplane_lut_gemm_noalloc": [_c_int, _vp, _vp, _c_int, _vp, _vp, _c_int, _vp, _vp, _c_int,
                                                _c_int, _c_int, _c_int, _vp],
            "apmoe_combine": [_vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int, _vp, _vp, _vp],
            "apmoe_plan_bitwidths": [_c_int, _c_int, _vp, _vp, _vp, _vp, ctypes.c_uint64, _vp],
            "apmoe_plan_online": [_c_int, _c_int, _vp, _vp, _vp, _vp, _c_int, _vp, ctypes.c_uint64,
                                  ctypes.c_uint64, ctypes.c_uint64, _vp, _vp, _vp],
            "apmoe_harm_multipliers": [_c_int, _vp, _vp, _vp],
            "apmoe_plan_routed": [_c_int, _c_int, _vp, _vp, _vp, _vp, ctypes.c_uint64, _vp, _vp, _vp],
            "apmoe_commit_bits": [_vp, _c_int, _vp, _vp],
            "apmoe_workspace_bytes": [_c_int, _c_int, _c_int, _c_int, _c_int],
            "apmoe_packed_plane_words": [_c_int, _c_int],
            "apmoe_pack_planes": [_vp, _c_int, _c_int, _vp, _vp],
            "apmoe_strerror": [_c_int],
            "apmoe_arena_create": [_u64, _vp],
            "apmoe_arena_alloc": [_vp, _u64, _vp],
            "apmoe_arena_take": [_vp, _u64, _u64],
            "apmoe_arena_release": [_vp, _u64, _u64],
            "apmoe_arena_stats": [_vp, _vp, _vp, _vp],
            "apmoe_pager_create": [_c_int, _c_int, _c_int, _vp, _vp, _vp, _u64, _vp, _vp, _vp],
            "apmoe_pager_stage": [_vp, _vp, _vp],
            "apmoe_pager_commit": [_vp, _vp],
            "apmoe_pager_stats": [_vp, _vp, _vp, _vp, _vp, _vp, _vp],
            "apmoe_pager_destroy": [_vp],
            "apmoe_exp_plan": [_vp, _u64, _vp, _vp, _vp],
            "apmoe_exp_encode": [_vp, _u64, _vp, _vp, _u64, _vp, _vp, _vp],
            "apmoe_exp_decode": [_vp, _u64, _vp, _vp, _vp, _u64, _vp, _vp],
            "apmoe_exp_decode_batch": [_c_int, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp],
        }
        for name, args in sig.items():
            fn = getattr(lib, name)
            fn.argtypes = args
            fn.restype = _c_int
        lib.apmoe_workspace_bytes.restype = _c_size
        lib.apmoe_packed_plane_words.restype = _c_size
        lib.apmoe_strerror.restype = ctypes.c_char_p
        lib.apmoe_arena_destroy.argtypes = [_vp]
        lib.apmoe_arena_destroy.restype = None
        _LIB = lib
    return _LIB


def header_symbols():
    """Entry points declared in include/apmoe.h."""
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:int|void|size_t|const char\*)\s+(apmoe_\w+)\s*\(", text, re.M)))


def strerror(code: int) -> str:
    return _lib().apmoe_strerror(int(code)).decode()


def _check(rc: int, where: str):
    if rc != OK:
        raise ApmoeError(rc, where)


# ---------------------------------------------------------------------------
# torch helpers (device memory and streams only)
# ---------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def _ptr(t, dtype=None, numel=None, name="tensor", device=True):
    if t is None:
        return None
    torch = _torch()
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if device and t.device.type != "cuda":
        raise TypeError(f"{name}: expected a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if numel is not None and t.numel() < numel:
        raise ValueError(f"{name}: needs at least {numel} elements, has {t.numel()}")
    return t.data_ptr()


def _stream(stream=None):
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


# ---------------------------------------------------------------------------
# Entry points (same names as the C ABI, without the prefix)
# ---------------------------------------------------------------------------

def route(x, w_router, bias, logit_scale, k, topk_ids, topk_w, ws=None, stream=None, x_norms=None):
    torch = _torch()
    T, H = x.shape
    E = w_router.shape[0]
    wsp, wsb = (None, 0) if ws is None else (_ptr(ws, torch.uint8, ws.numel(), "ws"), ws.numel())
    rc = _lib().apmoe_route(_ptr(x, torch.float16, T * H, "x"), T, H,
                            _ptr(w_router, torch.float32, E * H, "w_router"),
                            _ptr(bias, torch.float32, E, "bias"), float(logit_scale), E, k,
                            _ptr(topk_ids, torch.int32, T * k, "topk_ids"),
                            _ptr(topk_w, torch.float32, T * k, "topk_w"),
                            _ptr(x_norms, torch.float32, T, "x_norms"), wsp, wsb, _stream(stream))
    _check(rc, "apmoe_route")


def route_stats(x, topk_ids, topk_w, E, mass, wnorm, ws, stream=None):
    """Per-expert routing mass and routing-weighted input norm (fp32 [E] each)."""
    torch = _torch()
    T, H = x.shape
    k = topk_ids.shape[1]
    rc = _lib().apmoe_route_stats(_ptr(x, torch.float16, T * H, "x"), T, H,
                                  _ptr(topk_ids, torch.int32, T * k, "topk_ids"),
                                  _ptr(topk_w, torch.float32, T * k, "topk_w"), k, E,
                                  _ptr(mass, torch.float32, E, "mass"), _ptr(wnorm, torch.float32, E, "wnorm"),
                                  _ptr(ws, torch.uint8, ws.numel(), "ws"), ws.numel(), _stream(stream))
    _check(rc, "apmoe_route_stats")


def permute(topk_ids, E, counts, offsets, sorted_slots, pos_of_slot, n_shared=0, stream=None, stats=None):
    """Grouping over E + n_shared experts and T * (k + n_shared) slots (the
    n_shared always-on experts first).  stats: optional (topk_w, x_norms, mass,
    wnorm, ws) for the routing statistics in the same launch."""
    torch = _torch()
    T, k = topk_ids.shape
    S = T * (k + n_shared)
    tw = xn = ms = wn = wsp = None
    wsb = 0
    if stats is not None:
        w_, n_, m_, v_, ws = stats
        tw, xn = _ptr(w_, torch.float32, T * k, "topk_w"), _ptr(n_, torch.float32, T, "x_norms")
        ms, wn = _ptr(m_, torch.float32, E, "mass"), _ptr(v_, torch.float32, E, "wnorm")
        wsp, wsb = _ptr(ws, torch.uint8, S * 8, "ws"), ws.numel()
    rc = _lib().apmoe_permute(_ptr(topk_ids, torch.int32, T * k, "topk_ids"), T, k, E, n_shared,
                              _ptr(counts, torch.int32, E + n_shared, "counts"),
                              _ptr(offsets, torch.int32, E + n_shared + 1, "offsets"),
                              _ptr(sorted_slots, torch.int32, S, "sorted_slots"),
                              _ptr(pos_of_slot, torch.int32, S, "pos_of_slot"), tw, xn, ms, wn, wsp, wsb,
                              _stream(stream))
    _check(rc, "apmoe_permute")


def workspace_bytes(T, k, E, H, I) -> int:
    return int(_lib().apmoe_workspace_bytes(T, k, E, H, I))


def packed_plane_words(rows, cols) -> int:
    return int(_lib().apmoe_packed_plane_words(rows, cols))


def pack_planes(src, rows, cols, dst, stream=None):
    """Canonical planes (device int32 view of uint32 [6, rows, cols/32]) -> packed layout."""
    torch = _torch()
    rc = _lib().apmoe_pack_planes(_ptr(src, torch.int32, 6 * rows * (cols // 32), "planes"), rows, cols,
                                  _ptr(dst, torch.int32, packed_plane_words(rows, cols), "packed"),
                                  _stream(stream))
    _check(rc, "apmoe_pack_planes")


def bitplane_lut_gemm(stage, experts_desc, bits, E, offsets, sorted_slots, k, inp, out, T, H, I,
                      mfma_min_tokens, ws=None, stream=None):
    """experts_desc: device tensor holding E apmoe_expert descriptors (see ExpertTable)."""
    torch = _torch()
    S = T * k
    base = stage & ~(ONLY_GEMV | ONLY_TILE)
    if base == GATE_UP_SWIGLU:
        _ptr(inp, torch.float16, T * H, "x")
        _ptr(out, torch.float16, S * I, "A")
    elif base == DOWN:
        _ptr(inp, torch.float16, S * I, "A")
        _ptr(out, torch.float32, S * H, "Y")
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    rc = _lib().apmoe_bitplane_lut_gemm(
        int(stage), _ptr(experts_desc, torch.int64, E * 18, "experts"), _ptr(bits, torch.int8, E, "bits"), E,
        _ptr(offsets, torch.int32, E + 1, "offsets"), _ptr(sorted_slots, torch.int32, None, "sorted_slots"),
        k, inp.data_ptr(), out.data_ptr(), T, H, I, int(mfma_min_tokens),
        None if ws is None else ws.data_ptr(), ws_bytes, _stream(stream))
    _check(rc, "apmoe_bitplane_lut_gemm")


def bitplane_lut_gemm_noalloc(stage, experts_desc, bits, E, offsets, sorted_slots, k, inp, out, T, H, I,
                              mfma_min_tokens, stream=None):
    """apmoe_bitplane_lut_gemm_noalloc: the same stage with the library's static scratch."""
    torch = _torch()
    S = T * k
    base = stage & ~(ONLY_GEMV | ONLY_TILE)
    if base == GATE_UP_SWIGLU:
        _ptr(inp, torch.float16, T * H, "x")
        _ptr(out, torch.float16, S * I, "A")
    elif base == DOWN:
        _ptr(inp, torch.float16, S * I, "A")
        _ptr(out, torch.float32, S * H, "Y")
    rc = _lib().apmoe_bitplane_lut_gemm_noalloc(
        int(stage), _ptr(experts_desc, torch.int64, E * 18, "experts"), _ptr(bits, torch.int8, E, "bits"), E,
        _ptr(offsets, torch.int32, E + 1, "offsets"), _ptr(sorted_slots, torch.int32, None, "sorted_slots"),
        k, inp.data_ptr(), out.data_ptr(), T, H, I, int(mfma_min_tokens), _stream(stream))
    _check(rc, "apmoe_bitplane_lut_gemm_noalloc")


def combine(Y, pos_of_slot, topk_w, T, k, H, y_shared, out, n_shared=0, stream=None):
    torch = _torch()
    kk = k + n_shared
    rc = _lib().apmoe_combine(_ptr(Y, torch.float32, T * kk * H, "Y"),
                              _ptr(pos_of_slot, torch.int32, T * kk, "pos_of_slot"),
                              _ptr(topk_w, torch.float32, T * k, "topk_w"), T, k, n_shared, H,
                              _ptr(y_shared, torch.float32, T * H, "y_shared"),
                              _ptr(out, torch.float16, T * H, "out"), _stream(stream))
    _check(rc, "apmoe_combine")


def commit_bits(bits_host, bits_dev, stream=None):
    """bits_host: a sequence of ints; bits_dev: device int8 tensor [E]."""
    import numpy as np
    torch = _torch()
    b = np.ascontiguousarray(np.asarray(bits_host, dtype=np.int8))
    rc = _lib().apmoe_commit_bits(b.ctypes.data, len(b), _ptr(bits_dev, torch.int8, len(b), "bits_dev"),
                                  _stream(stream))
    _check(rc, "apmoe_commit_bits")


def plan_bitwidths(levels, harm, nbytes, floor_bits, budget):
    """Host planner.  Returns (status, bits int8[E]); raises only on EINVAL/EBITS."""
    import numpy as np
    lv = np.ascontiguousarray(np.asarray(levels, dtype=np.int8))
    hm = np.ascontiguousarray(np.asarray(harm, dtype=np.float64))
    nb = np.ascontiguousarray(np.asarray(nbytes, dtype=np.uint64))
    fl = np.ascontiguousarray(np.asarray(floor_bits, dtype=np.int8))
    E, L = hm.shape
    if nb.shape != (E, L) or lv.shape != (L,) or fl.shape != (E,):
        raise ValueError("planner input shapes disagree")
    out = np.zeros(E, dtype=np.int8)
    rc = _lib().apmoe_plan_bitwidths(E, L, lv.ctypes.data, hm.ctypes.data, nb.ctypes.data,
                                     fl.ctypes.data, int(budget), out.ctypes.data)
    return rc, out


def harm_multipliers(mass, wnorm):
    """Per-expert harm multipliers from routing statistics (host arrays or
    sequences of E floats).  Returns float64 [E]."""
    import numpy as np
    m = np.ascontiguousarray(np.asarray(mass, dtype=np.float32))
    n = np.ascontiguousarray(np.asarray(wnorm, dtype=np.float32))
    if m.shape != n.shape or m.ndim != 1:
        raise ValueError("mass and wnorm must be two [E] arrays")
    out = np.zeros(m.size, dtype=np.float64)
    _check(_lib().apmoe_harm_multipliers(m.size, m.ctypes.data, n.ctypes.data, out.ctypes.data),
           "apmoe_harm_multipliers")
    return out


def plan_routed(levels, harm, nbytes, floor_bits, budget, mass, wnorm):
    """Greedy plan over harm scaled by the routing multipliers.  Returns
    (status, bits int8[E]); raises only on EINVAL/EBITS."""
    import numpy as np
    lv = np.ascontiguousarray(np.asarray(levels, dtype=np.int8))
    hm = np.ascontiguousarray(np.asarray(harm, dtype=np.float64))
    nb = np.ascontiguousarray(np.asarray(nbytes, dtype=np.uint64))
    fl = np.ascontiguousarray(np.asarray(floor_bits, dtype=np.int8))
    m = np.ascontiguousarray(np.asarray(mass, dtype=np.float32))
    n = np.ascontiguousarray(np.asarray(wnorm, dtype=np.float32))
    E, L = hm.shape
    if nb.shape != (E, L) or lv.shape != (L,) or fl.shape != (E,) or m.shape != (E,) or n.shape != (E,):
        raise ValueError("planner input shapes disagree")
    out = np.zeros(E, dtype=np.int8)
    rc = _lib().apmoe_plan_routed(E, L, lv.ctypes.data, hm.ctypes.data, nb.ctypes.data, fl.ctypes.data,
                                  int(budget), m.ctypes.data, n.ctypes.data, out.ctypes.data)
    if rc not in (OK, ENOSPACE):
        _check(rc, "apmoe_plan_routed")
    return rc, out


def plan_online(levels, harm, nbytes, floor_bits, stage_bits, m_total, m_kv, hysteresis, bits_now):
    """Online planner step.  Returns (status, bits int8[E], stage); stage is -1
    when the current plan is kept.  Raises only on EINVAL/EBITS."""
    import numpy as np
    lv = np.ascontiguousarray(np.asarray(levels, dtype=np.int8))
    hm = np.ascontiguousarray(np.asarray(harm, dtype=np.float64))
    nb = np.ascontiguousarray(np.asarray(nbytes, dtype=np.uint64))
    fl = np.ascontiguousarray(np.asarray(floor_bits, dtype=np.int8))
    sb = np.ascontiguousarray(np.asarray(stage_bits, dtype=np.int8))
    now = np.ascontiguousarray(np.asarray(bits_now, dtype=np.int8))
    E, L = hm.shape
    if nb.shape != (E, L) or lv.shape != (L,) or fl.shape != (E,) or now.shape != (E,):
        raise ValueError("planner input shapes disagree")
    out = np.zeros(E, dtype=np.int8)
    stage = ctypes.c_int(0)
    rc = _lib().apmoe_plan_online(E, L, lv.ctypes.data, hm.ctypes.data, nb.ctypes.data, fl.ctypes.data, len(sb),
                                  sb.ctypes.data, int(m_total), int(m_kv), int(hysteresis), now.ctypes.data,
                                  out.ctypes.data, ctypes.byref(stage))
    if rc not in (OK, ENOSPACE):
        _check(rc, "apmoe_plan_online")
    return rc, out, stage.value


# ---------------------------------------------------------------------------
# Plane paging: the host-side arena allocator and the pager
# ---------------------------------------------------------------------------

class Arena:
    """apmoe_arena_*: first-fit over [0, nbytes) in 256-byte units (host only)."""

    def __init__(self, nbytes: int):
        h = _vp()
        _check(_lib().apmoe_arena_create(int(nbytes), ctypes.byref(h)), "apmoe_arena_create")
        self._h = h

    def alloc(self, nbytes: int):
        """Offset of the new range, or None when no free range holds it."""
        off = ctypes.c_uint64()
        rc = _lib().apmoe_arena_alloc(self._h, int(nbytes), ctypes.byref(off))
        if rc == ENOSPACE:
            return None
        _check(rc, "apmoe_arena_alloc")
        return off.value

    def take(self, off: int, nbytes: int) -> bool:
        rc = _lib().apmoe_arena_take(self._h, int(off), int(nbytes))
        if rc == ENOSPACE:
            return False
        _check(rc, "apmoe_arena_take")
        return True

    def release(self, off: int, nbytes: int) -> int:
        return _lib().apmoe_arena_release(self._h, int(off), int(nbytes))

    def stats(self):
        """(free bytes, largest free range, number of free ranges)."""
        f, l, n = ctypes.c_uint64(), ctypes.c_uint64(), ctypes.c_int()
        _check(_lib().apmoe_arena_stats(self._h, ctypes.byref(f), ctypes.byref(l), ctypes.byref(n)),
               "apmoe_arena_stats")
        return f.value, l.value, n.value

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and _LIB is not None:
            _LIB.apmoe_arena_destroy(h)
            self._h = None


class Pager:
    """apmoe_pager_*: residency of E experts' planes and LUTs in a device arena.

    host_planes / host_luts: host tensors as the C ABI describes; the pager
    copies them into its own pinned memory when it is created."""

    def __init__(self, E, H, I, host_planes, host_luts, arena, desc, bits):
        torch = _torch()
        assert len(host_planes) == 3 * E and len(host_luts) == 12 * E
        for t in list(host_planes) + list(host_luts):
            if t.device.type != "cpu" or not t.is_contiguous():
                raise TypeError("host copies must be contiguous host tensors")
        for i in range(3 * E):
            rows, cols = (I, H) if i % 3 < 2 else (H, I)
            if host_planes[i].numel() * host_planes[i].element_size() < 4 * packed_plane_words(rows, cols):
                raise ValueError(f"host planes {i}: too small for a {rows} x {cols} matrix")
            for b in range(3, 7):
                t = host_luts[4 * i + b - 3]
                if t.numel() * t.element_size() < rows * (1 << b) * 2:
                    raise ValueError(f"host LUT {i}, {b} bits: too small for {rows} rows")
        self._keep = (list(host_planes), list(host_luts), arena, desc, bits)
        self.E = E
        hp = (_vp * (3 * E))(*[t.data_ptr() for t in host_planes])
        hl = (_vp * (12 * E))(*[t.data_ptr() for t in host_luts])
        h = _vp()
        rc = _lib().apmoe_pager_create(E, H, I, hp, hl, _ptr(arena, torch.uint8, None, "arena"), arena.numel(),
                                       _ptr(desc, None, None, "desc"), _ptr(bits, torch.int8, E, "bits"),
                                       ctypes.byref(h))
        _check(rc, "apmoe_pager_create")
        self._h = h

    def stage(self, bits_new, copy_stream=None) -> int:
        """Returns OK or ENOSPACE (nothing staged); raises on other errors."""
        import numpy as np
        b = np.ascontiguousarray(np.asarray(bits_new, dtype=np.int8))
        if b.size != self.E:
            raise ValueError(f"bits: expected {self.E} entries")
        rc = _lib().apmoe_pager_stage(self._h, b.ctypes.data, _stream(copy_stream))
        if rc == ENOSPACE:
            return rc
        _check(rc, "apmoe_pager_stage")
        return rc

    def commit(self, stream=None):
        _check(_lib().apmoe_pager_commit(self._h, _stream(stream)), "apmoe_pager_commit")

    def stats(self):
        """dict: resident, free, largest_free, h2d, d2d (bytes), ranges (copied by the last stage)."""
        v = [ctypes.c_uint64() for _ in range(6)]
        _check(_lib().apmoe_pager_stats(self._h, *[ctypes.byref(x) for x in v]), "apmoe_pager_stats")
        return dict(zip(("resident", "free", "largest_free", "h2d", "d2d", "ranges"), (x.value for x in v)))

    def close(self):
        h = getattr(self, "_h", None)
        if h is not None and _LIB is not None:
            self._h = None
            _check(_LIB.apmoe_pager_destroy(h), "apmoe_pager_destroy")

    def __del__(self):
        import sys
        if sys.is_finalizing():   # the HIP runtime may already be gone
            return
        try:
            self.close()
        except Exception:
            pass


# ---------------------------------------------------------------------------
# Lossless exponent codec (fp16 weights)
# ---------------------------------------------------------------------------

def exp_encode(w16):
    """Host encoder: w16 numpy uint16 [n] -> dict(lengths, words, block_off,
    lo, table) of numpy arrays (the library's apmoe_exp_plan + _encode)."""
    import numpy as np
    w = np.ascontiguousarray(np.asarray(w16, dtype=np.uint16).reshape(-1))
    n = w.size
    lengths = np.zeros(256, dtype=np.uint8)
    nwords, nblocks = ctypes.c_uint64(), ctypes.c_uint64()
    _check(_lib().apmoe_exp_plan(w.ctypes.data, n, lengths.ctypes.data, ctypes.byref(nwords),
                                 ctypes.byref(nblocks)), "apmoe_exp_plan")
    words = np.zeros(nwords.value, dtype=np.uint32)
    offs = np.zeros(nblocks.value, dtype=np.uint32)
    lo = np.zeros(n, dtype=np.uint8)
    table = np.zeros(4096, dtype=np.uint16)
    _check(_lib().apmoe_exp_encode(w.ctypes.data, n, lengths.ctypes.data, words.ctypes.data, words.size,
                                   offs.ctypes.data, lo.ctypes.data, table.ctypes.data), "apmoe_exp_encode")
    return {"lengths": lengths, "words": words, "block_off": offs, "lo": lo, "table": table, "n": n}


def exp_decode(words, block_off, lo, table, out, stream=None):
    """Device decoder: int32/uint8/int16 device tensors as exp_encode's arrays
    (words int32 [nwords], block_off int32, lo uint8 [n], table int16 [4096]) ->
    out int16 [n] (fp16 bit patterns)."""
    torch = _torch()
    n = out.numel()
    rc = _lib().apmoe_exp_decode(_ptr(words, torch.int32, 2, "words"), words.numel(),
                                 _ptr(block_off, torch.int32, None, "block_off"), _ptr(lo, torch.uint8, n, "lo"),
                                 _ptr(table, torch.int16, 4096, "table"), n, _ptr(out, torch.int16, n, "out"),
                                 _stream(stream))
    _check(rc, "apmoe_exp_decode")


EXP_MAX_BATCH = 16


def exp_decode_batch(streams, stream=None):
    """One launch over several coded matrices: streams is a list of dicts with
    the device tensors words, block_off, lo, table and out, as exp_decode takes."""
    torch = _torch()
    c = len(streams)
    if not 1 <= c <= EXP_MAX_BATCH:
        raise ValueError(f"1..{EXP_MAX_BATCH} matrices per call, got {c}")
    vp = ctypes.c_void_p * c
    u64 = ctypes.c_uint64 * c
    words = vp(*[_ptr(d["words"], torch.int32, 2, "words") for d in streams])
    nwords = u64(*[d["words"].numel() for d in streams])
    boff = vp(*[_ptr(d["block_off"], torch.int32, None, "block_off") for d in streams])
    lo = vp(*[_ptr(d["lo"], torch.uint8, d["out"].numel(), "lo") for d in streams])
    tab = vp(*[_ptr(d["table"], torch.int16, 4096, "table") for d in streams])
    n = u64(*[d["out"].numel() for d in streams])
    out = vp(*[_ptr(d["out"], torch.int16, d["out"].numel(), "out") for d in streams])
    rc = _lib().apmoe_exp_decode_batch(c, words, nwords, boff, lo, tab, n, out, _stream(stream))
    _check(rc, "apmoe_exp_decode_batch")
