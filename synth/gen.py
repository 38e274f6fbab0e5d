"""Seeded generation of one layer's inputs in the bit-plane + LUT storage format.

Storage format of one quantized matrix W [rows x cols] (cols = the contraction
dimension K, a multiple of 32):

* a 6-bit code per weight, uniform over 0..63;
* six bit-planes ``planes[p][row][w]`` (uint32), plane 0 holding the most
  significant code bit; bit i of word w is column 32*w + i (packed along K);
* one lookup table per bitwidth b in 3..6, ``luts[b-3][row][v]`` with 2**b fp16
  centroids in ascending order (each its own sorted N(0, 0.02) draw);
* for experts that run in the fp16 fallback, plain fp16 weights ``w16``.

The b-bit code of a weight is the top b planes, so a b-bit expert reads only
the leading b plane slabs.  The format follows the any-precision bit-plane +
LUT description (zhichai.net page, section "核心洞察"); word width, bit order
and the per-bitwidth tables are fixed here because the pages leave them open.

Random streams: ``SeedSequence(seed).spawn(4)`` -> [control (bits, router),
expert weights, shared expert, activations], each a PCG64 generator, so the
expert weights are identical for every token count of the same shape.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Optional

import numpy as np

from .configs import LUT_BITS, N_PLANES, LayerConfig


@dataclass
class MatrixData:
    rows: int
    cols: int
    planes: np.ndarray                  # uint32 [6, rows, cols // 32]
    luts: List[np.ndarray]              # fp16 [rows, 2**b] for b = 3, 4, 5, 6
    w16: Optional[np.ndarray] = None    # fp16 [rows, cols] (fallback experts only)
    code6: Optional[np.ndarray] = None  # uint8 [rows, cols], kept on request for tests

    def lut(self, b: int) -> np.ndarray:
        return self.luts[b - 3]


@dataclass
class LayerInputs:
    cfg: LayerConfig
    seed: int
    x: np.ndarray                       # fp16 [T, H]
    w_router: np.ndarray                # fp32 [E, H]
    bias: Optional[np.ndarray]          # fp32 [E] or None
    bits: Optional[np.ndarray]          # int8 [E]; None when a planner must choose
    experts: List[Dict[str, MatrixData]]        # per expert: gate, up [I x H]; down [H x I]
    shared: Optional[Dict[str, MatrixData]] = None  # fp16 shared expert (w16 only)
    plan: Optional[dict] = None         # planner inputs when bits come from the planner
    route_p: Optional[np.ndarray] = None  # the Zipf routing prior, when one is used


def pack_planes(code6: np.ndarray) -> np.ndarray:
    """Lay 6-bit codes [rows, cols] out as six uint32 bit-planes [6, rows, cols//32]."""
    rows, cols = code6.shape
    if cols % 32:
        raise ValueError("cols must be a multiple of 32")
    out = np.empty((N_PLANES, rows, cols // 32), dtype=np.uint32)
    for p in range(N_PLANES):
        bit = ((code6 >> (N_PLANES - 1 - p)) & 1).astype(np.uint8)
        packed = np.packbits(bit, axis=1, bitorder="little")      # [rows, cols//8]
        out[p] = np.ascontiguousarray(packed).view("<u4").reshape(rows, cols // 32)
    return out


def plane_bytes(rows: int, cols: int, b: int) -> int:
    """Bytes a matrix occupies at bitwidth b: the top-b planes plus LUT_b, or fp16 rows."""
    if b == 16:
        return rows * cols * 2
    return rows * cols * b // 8 + rows * (1 << b) * 2


def _gen_matrix(rng: np.random.Generator, rows: int, cols: int, w_std: float,
                with_w16: bool, keep_code6: bool) -> MatrixData:
    code6 = rng.integers(0, 64, size=(rows, cols), dtype=np.uint8)
    luts = []
    for b in LUT_BITS:
        v = rng.normal(0.0, w_std, size=(rows, 1 << b))
        v.sort(axis=1)
        luts.append(v.astype(np.float16))
    w16 = None
    if with_w16:
        w16 = rng.normal(0.0, w_std, size=(rows, cols)).astype(np.float16)
    planes = pack_planes(code6)
    return MatrixData(rows, cols, planes, luts, w16, code6 if keep_code6 else None)


def _gen_fp16_matrix(rng: np.random.Generator, rows: int, cols: int, w_std: float) -> MatrixData:
    w16 = rng.normal(0.0, w_std, size=(rows, cols)).astype(np.float16)
    return MatrixData(rows, cols, np.zeros((N_PLANES, 0, 0), np.uint32), [], w16, None)


def zipf_prior(E: int, s: float) -> np.ndarray:
    p = (np.arange(1, E + 1, dtype=np.float64)) ** (-s)
    return p / p.sum()


def planner_inputs(cfg: LayerConfig, p: np.ndarray) -> dict:
    """Planner inputs for a Zipf-skewed layer.

    Levels 6 > 5 > 4 > 3 bits; harm[e][l] = p_e * 2**-b (a step size that halves
    per bit, weighted by the expert's routing share); bytes are the plane + LUT
    bytes of gate, up and down; every floor is 3 bits; the budget is the mean of
    the all-4-bit and all-5-bit footprints (a 4.5-bit average).
    """
    levels = np.array([6, 5, 4, 3], dtype=np.int8)
    E, H, I = cfg.E, cfg.H, cfg.I
    harm = np.array([[p[e] * 2.0 ** (-int(b)) for b in levels] for e in range(E)], dtype=np.float64)
    nbytes = np.array([[2 * plane_bytes(I, H, int(b)) + plane_bytes(H, I, int(b)) for b in levels]
                       for e in range(E)], dtype=np.uint64)
    floors = np.full(E, 3, dtype=np.int8)
    budget = int((int(nbytes[:, 2].sum()) + int(nbytes[:, 1].sum())) // 2)
    return dict(levels=levels, harm=harm, bytes=nbytes, floors=floors, budget=budget)


def make_inputs(cfg: LayerConfig, seed: int = 0, keep_code6: bool = False) -> LayerInputs:
    s_ctrl, s_w, s_sh, s_x = np.random.SeedSequence(seed).spawn(4)
    r_ctrl = np.random.Generator(np.random.PCG64(s_ctrl))
    r_w = np.random.Generator(np.random.PCG64(s_w))
    r_sh = np.random.Generator(np.random.PCG64(s_sh))
    r_x = np.random.Generator(np.random.PCG64(s_x))
    E, H, I, T = cfg.E, cfg.H, cfg.I, cfg.T

    bits = None
    if cfg.bits_mode == "fixed":
        if cfg.bits is None or len(cfg.bits) != E:
            raise ValueError("fixed bits need one entry per expert")
        bits = np.array(cfg.bits, dtype=np.int8)
    elif cfg.bits_mode == "uniform":
        bits = r_ctrl.choice(np.array([3, 4, 5, 6], dtype=np.int8), size=E)
    elif cfg.bits_mode != "planner_zipf":
        raise ValueError(cfg.bits_mode)

    w_router = r_ctrl.normal(0.0, cfg.w_std, size=(E, H)).astype(np.float32)

    bias = None
    route_p = None
    plan = None
    if cfg.router_bias == "zipf" or cfg.bits_mode == "planner_zipf":
        route_p = zipf_prior(E, cfg.zipf_s)
    if cfg.router_bias == "zipf":
        bias = np.log(route_p).astype(np.float32)
    if cfg.bits_mode == "planner_zipf":
        plan = planner_inputs(cfg, route_p)

    experts = []
    for e in range(E):
        fp16_expert = bits is not None and int(bits[e]) == 16
        mats = {}
        for name, (rows, cols) in (("gate", (I, H)), ("up", (I, H)), ("down", (H, I))):
            mats[name] = _gen_matrix(r_w, rows, cols, cfg.w_std, fp16_expert, keep_code6)
        experts.append(mats)

    shared = None
    if cfg.shared_I:
        Is = cfg.shared_I
        shared = {name: _gen_fp16_matrix(r_sh, rows, cols, cfg.w_std)
                  for name, (rows, cols) in (("gate", (Is, H)), ("up", (Is, H)), ("down", (H, Is)))}

    x = r_x.normal(0.0, cfg.x_std, size=(T, H)).astype(np.float16)
    return LayerInputs(cfg, seed, x, w_router, bias, bits, experts, shared, plan, route_p)
