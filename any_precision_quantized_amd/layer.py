"""Device-resident expert weights and the layer's call sequence.

``ExpertTable`` uploads per-expert bit-planes, LUTs and fp16 rows and builds
the device array of ``apmoe_expert`` descriptors.  ``MoELayer`` owns the
per-call buffers and chains the C-ABI entry points:

    route -> permute -> gemm(GATE_UP_SWIGLU) -> gemm(DOWN) [-> shared expert] -> combine

An fp16 shared expert whose intermediate size is n times the routed one runs
inside the routed launches as n always-on experts (its gate/up row blocks and
its down column blocks, placed first in the descriptor table); otherwise it
runs as its own launches on a side stream.

PyTorch only provides device memory and the HIP stream; every step runs in
libapmoe's kernels.
"""
from __future__ import annotations

from typing import List, Optional

import numpy as np

from . import _lib

MATS = ("gate", "up", "down")
DESC_WORDS = 18          # 3 matrices x (planes, lut[4], w16) pointers
# Groups of at least this many slots take the dequantise-to-LDS + MFMA tile path;
# smaller ones take the bit-plane GEMV path (one pass over K covers 64 tokens,
# a larger group takes several).  Measured on the Mixtral-shaped layer (8
# experts, top-2): groups of 52-76 slots run 1.8x faster on the GEMV path,
# groups of 114-158 equally fast on both, groups of 226-293 1.3x faster as
# tiles, so the crossover sits at about 160.
DEFAULT_MFMA_MIN_TOKENS = 160


def auto_mfma_min_tokens(T: int, k: int, E: int) -> int:
    """The layer's default path choice: groups of at least
    DEFAULT_MFMA_MIN_TOKENS slots take the tile path, unless the mean group
    T * k / E is under half of that, where even a group twice the mean stays
    on the GEMV side of the crossover: then every group takes the GEMV path
    and no tile kernel is launched at all (a tile launch that finds no group
    still costs a few microseconds)."""
    if T * k < E * (DEFAULT_MFMA_MIN_TOKENS // 2):
        return 1 << 30
    return DEFAULT_MFMA_MIN_TOKENS


class ExpertTable:
    """Expert weights in device memory plus their descriptor array.

    ``experts``: sequence of mappings name -> matrix, each matrix exposing
    ``planes`` (canonical uint32 [6, rows, cols/32]), ``luts`` (four fp16
    arrays [rows, 2**b]) and ``w16`` (fp16 [rows, cols] or None).  The planes
    are repacked once on the device into the layout the kernels read
    (apmoe_pack_planes).
    """

    def __init__(self, experts, device="cuda", _tensors=None):
        import torch
        self.device = device
        self.E = len(experts) if experts is not None else len(_tensors)
        self.tensors: List[dict] = []
        if _tensors is None:
            for mats in experts:
                d = {}
                for name in MATS:
                    m = mats[name]
                    ent = {"planes": None, "luts": [None] * 4, "w16": None}
                    if m.planes is not None and m.planes.size:
                        # canonical planes in, kernel-native packed planes kept
                        canon = torch.from_numpy(np.ascontiguousarray(m.planes).view(np.int32)).to(device)
                        rows, cols = m.planes.shape[1], m.planes.shape[2] * 32
                        packed = torch.empty(_lib.packed_plane_words(rows, cols), dtype=torch.int32, device=device)
                        _lib.pack_planes(canon, rows, cols, packed)
                        ent["planes"] = packed
                        del canon
                    for i, lut in enumerate(m.luts or []):
                        ent["luts"][i] = torch.from_numpy(np.ascontiguousarray(lut).view(np.int16)).to(device)
                    if m.w16 is not None:
                        ent["w16"] = torch.from_numpy(np.ascontiguousarray(m.w16).view(np.int16)).to(device)
                    d[name] = ent
                self.tensors.append(d)
        else:
            self.tensors = _tensors
        self.desc = self._descriptors()

    def _descriptors(self):
        import torch
        desc = np.zeros((self.E, DESC_WORDS), dtype=np.int64)
        for e, d in enumerate(self.tensors):
            for mi, name in enumerate(MATS):
                ent = d[name]
                base = 6 * mi
                if ent["planes"] is not None:
                    desc[e, base] = ent["planes"].data_ptr()
                for i in range(4):
                    if ent["luts"][i] is not None:
                        desc[e, base + 1 + i] = ent["luts"][i].data_ptr()
                if ent["w16"] is not None:
                    desc[e, base + 5] = ent["w16"].data_ptr()
        return torch.from_numpy(desc).to(self.device)

    def replicate(self) -> "ExpertTable":
        """A second copy of every weight tensor (device-side clone)."""
        copies = []
        for d in self.tensors:
            copies.append({name: {"planes": None if ent["planes"] is None else ent["planes"].clone(),
                                  "luts": [None if t is None else t.clone() for t in ent["luts"]],
                                  "w16": None if ent["w16"] is None else ent["w16"].clone()}
                           for name, ent in d.items()})
        return ExpertTable(None, self.device, _tensors=copies)

    @staticmethod
    def concat(*tables: "ExpertTable") -> "ExpertTable":
        """One descriptor array over the experts of several tables (no copies)."""
        tensors = [d for t in tables for d in t.tensors]
        return ExpertTable(None, tables[0].device, _tensors=tensors)

    def split_rows(self, H: int, I: int) -> "ExpertTable":
        """An fp16 single-expert table with intermediate size n*I as n experts of
        size I: gate/up row blocks (views) and down column blocks (copied once
        to contiguous [H, I])."""
        assert self.E == 1
        d = self.tensors[0]
        g, u, dn = d["gate"]["w16"], d["up"]["w16"], d["down"]["w16"]
        Is = g.numel() // H
        assert Is % I == 0 and u.numel() == Is * H and dn.numel() == H * Is
        g2, u2, d2 = g.view(Is, H), u.view(Is, H), dn.view(H, Is)
        parts = []
        for v in range(Is // I):
            rows = slice(v * I, (v + 1) * I)
            parts.append({"gate": {"planes": None, "luts": [None] * 4, "w16": g2[rows].reshape(-1)},
                          "up": {"planes": None, "luts": [None] * 4, "w16": u2[rows].reshape(-1)},
                          "down": {"planes": None, "luts": [None] * 4,
                                   "w16": d2[:, rows].contiguous().reshape(-1)}})
        return ExpertTable(None, self.device, _tensors=parts)

    def nbytes(self) -> int:
        n = 0
        for d in self.tensors:
            for ent in d.values():
                for t in [ent["planes"], ent["w16"], *ent["luts"]]:
                    if t is not None:
                        n += t.numel() * t.element_size()
        return n


class MoELayer:
    """One MoE expert-FFN layer call on the GPU through libapmoe."""

    def __init__(self, E, H, I, k, T, w_router, bias, logit_scale, experts: ExpertTable, bits,
                 shared: Optional[ExpertTable] = None, shared_I: int = 0, mfma_min_tokens: Optional[int] = None,
                 device="cuda"):
        import torch
        self.E, self.H, self.I, self.k, self.T = E, H, I, k, T
        self.logit_scale = float(logit_scale)
        # None: the default policy (auto_mfma_min_tokens); an explicit value is used as given
        self.mfma_min_tokens = int(auto_mfma_min_tokens(T, k, E) if mfma_min_tokens is None else mfma_min_tokens)
        self.device = device
        dev = dict(device=device)
        self.w_router = torch.as_tensor(np.ascontiguousarray(w_router), dtype=torch.float32).to(device)
        self.bias = None if bias is None else torch.as_tensor(np.ascontiguousarray(bias), dtype=torch.float32).to(device)
        self.experts = experts
        self.shared = shared
        self.shared_I = shared_I
        # set by PagedExperts.attach: plans then go through the pager, which
        # makes the new planes and LUTs resident before the bits take effect
        self.pager = None
        # always-on experts: the shared expert split into n of the routed size
        self.n_shared = shared_I // I if (shared is not None and shared_I % I == 0) else 0
        n = self.n_shared
        E2, kk = E + n, k + n
        self.E2, self.kk = E2, kk
        self.bits = torch.zeros(E2, dtype=torch.int8, **dev)
        if n:
            _lib.commit_bits([16] * n, self.bits[:n])
            self._tables = {}
            self.table = self._fused(experts, shared)
        else:
            self.table = experts
        self.commit(bits)
        S = T * kk
        self.topk_ids = torch.empty((T, k), dtype=torch.int32, **dev)
        self.topk_w = torch.empty((T, k), dtype=torch.float32, **dev)
        self.counts = torch.empty(E2, dtype=torch.int32, **dev)
        self.offsets = torch.empty(E2 + 1, dtype=torch.int32, **dev)
        self.sorted_slots = torch.empty(S, dtype=torch.int32, **dev)
        self.pos_of_slot = torch.empty(S, dtype=torch.int32, **dev)
        self.A = torch.empty((S, I), dtype=torch.float16, **dev)
        self.Y = torch.empty((S, H), dtype=torch.float32, **dev)
        self.out = torch.empty((T, H), dtype=torch.float16, **dev)
        nws = _lib.workspace_bytes(T, kk, E2, H, I)
        self.ws = torch.empty(nws, dtype=torch.uint8, **dev) if nws else None
        # routing statistics for the planner (per routed expert), computed in
        # every forward by the router (token norms) and the grouping (sums)
        self.mass = torch.zeros(E, dtype=torch.float32, **dev)
        self.wnorm = torch.zeros(E, dtype=torch.float32, **dev)
        self.x_norms = torch.zeros(max(T, 1), dtype=torch.float32, **dev)
        self.ws_stats = torch.empty(max(8 * S, 4 * T, 4), dtype=torch.uint8, **dev)
        if shared is not None and not n:
            # the shared expert runs on a side stream (default priority) with
            # its own workspace, overlapping routing and the routed experts
            self.side = torch.cuda.Stream(device=device)
            self.ev_fork = torch.cuda.Event()
            self.ev_join = torch.cuda.Event()
            nws_sh = _lib.workspace_bytes(T, 1, 1, H, shared_I)
            self.ws_sh = torch.empty(nws_sh, dtype=torch.uint8, **dev) if nws_sh else None
            self.sh_bits = torch.tensor([16], dtype=torch.int8, **dev)
            self.sh_offsets = torch.tensor([0, T], dtype=torch.int32, **dev)
            self.sh_slots = torch.arange(T, dtype=torch.int32, **dev)
            self.A_sh = torch.empty((T, shared_I), dtype=torch.float16, **dev)
            self.Y_sh = torch.empty((T, H), dtype=torch.float32, **dev)

    def _fused(self, experts: ExpertTable, shared: ExpertTable) -> ExpertTable:
        """Descriptor table [shared parts..., routed experts...] (cached per pair)."""
        key = (id(experts), id(shared))
        if key not in self._tables:
            self._tables[key] = (ExpertTable.concat(shared.split_rows(self.H, self.I), experts), experts, shared)
        return self._tables[key][0]

    def commit(self, bits):
        """Commit routed bitwidths in stream order (the always-on parts stay at
        16).  On paged weights the pager stages the planes and LUTs the new
        bitwidths need and commits them together with the bits; writing the
        bits table alone would point the kernels at planes that are not
        resident.  Returns OK, or ENOSPACE when the pager's arena cannot hold
        the plan (nothing changed)."""
        if self.pager is not None:
            return self.pager.apply(bits)
        _lib.commit_bits(bits, self.bits[self.n_shared:])
        return _lib.OK

    def route_stats(self, x=None):
        """Routing mass and routing-weighted input norm of every routed expert
        over the last forward's routing, fp32 [E] device tensors (reused by
        later calls).  The forward computes them in its router and grouping
        launches; given x, they are recomputed with apmoe_route_stats instead
        (two launches of their own)."""
        if x is not None:
            _lib.route_stats(x, self.topk_ids, self.topk_w, self.E, self.mass, self.wnorm, self.ws_stats)
        return self.mass, self.wnorm

    def replan(self, x, levels, harm, nbytes, floor_bits, budget):
        """Re-plan the routed experts' bitwidths from the offline harm table
        corrected by the last forward's routing statistics (apmoe_plan_routed),
        commit the plan in stream order and return (status, bits).
        Synchronises to read the statistics back."""
        mass, wnorm = self.route_stats()
        status, bits = _lib.plan_routed(levels, harm, nbytes, floor_bits, budget, mass.cpu().numpy(),
                                        wnorm.cpu().numpy())
        if status == _lib.OK:
            status = self.commit(bits)
        return status, bits

    def forward(self, x, experts: Optional[ExpertTable] = None, shared: Optional[ExpertTable] = None):
        """x: device fp16 [T, H].  Returns the fp16 output [T, H] (a buffer reused by later calls)."""
        import torch
        ex = self.experts if experts is None else experts
        sh = self.shared if shared is None else shared
        T, H, I, E, k, n = self.T, self.H, self.I, self.E, self.k, self.n_shared
        side = sh is not None and not n
        ysh = None
        if side:
            main = torch.cuda.current_stream()
            self.ev_fork.record(main)
            self.side.wait_event(self.ev_fork)
            x.record_stream(self.side)
            with torch.cuda.stream(self.side):
                _lib.bitplane_lut_gemm(_lib.GATE_UP_SWIGLU, sh.desc, self.sh_bits, 1, self.sh_offsets,
                                       self.sh_slots, 1, x, self.A_sh, T, H, self.shared_I,
                                       self.mfma_min_tokens, self.ws_sh)
                _lib.bitplane_lut_gemm(_lib.DOWN, sh.desc, self.sh_bits, 1, self.sh_offsets, self.sh_slots,
                                       1, self.A_sh, self.Y_sh, T, H, self.shared_I, self.mfma_min_tokens,
                                       self.ws_sh)
            self.ev_join.record(self.side)
            ysh = self.Y_sh
        table = self._fused(ex, sh) if n else ex
        E2, kk = self.E2, self.kk
        _lib.route(x, self.w_router, self.bias, self.logit_scale, k, self.topk_ids, self.topk_w, self.ws,
                   x_norms=self.x_norms)
        _lib.permute(self.topk_ids, E, self.counts, self.offsets, self.sorted_slots, self.pos_of_slot, n,
                     stats=(self.topk_w, self.x_norms, self.mass, self.wnorm, self.ws_stats))
        _lib.bitplane_lut_gemm(_lib.GATE_UP_SWIGLU, table.desc, self.bits, E2, self.offsets, self.sorted_slots,
                               kk, x, self.A, T, H, I, self.mfma_min_tokens, self.ws)
        _lib.bitplane_lut_gemm(_lib.DOWN, table.desc, self.bits, E2, self.offsets, self.sorted_slots,
                               kk, self.A, self.Y, T, H, I, self.mfma_min_tokens, self.ws)
        if side:
            torch.cuda.current_stream().wait_event(self.ev_join)
        _lib.combine(self.Y, self.pos_of_slot, self.topk_w, T, k, H, ysh, self.out, n)
        return self.out

    def graph(self, x, experts: Optional[ExpertTable] = None, shared: Optional[ExpertTable] = None):
        """One forward step captured as a HIP graph: g.replay() reruns the
        whole layer on x with these weights (router, grouping, both expert
        stages, combine) and leaves the result in the buffer forward()
        returns.  The step enqueues kernels only (no copies, fills or
        allocations); an eager warm-up call first builds the descriptor table
        of the fused shared expert.  A shared expert that runs on the second
        stream (its size no multiple of the routed one) is not captured."""
        import torch
        sh = self.shared if shared is None else shared
        if sh is not None and not self.n_shared:
            raise ValueError("graph(): only a layer whose shared expert runs as always-on experts can be captured")
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            self.forward(x, experts, shared)
        torch.cuda.current_stream().wait_stream(s)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            self.forward(x, experts, shared)
        return g


class OnlinePlanner:
    """The layer's bitwidth plan kept up to date as the KV cache grows and
    shrinks: each step recomputes the weight budget M_w = m_total - m_kv and
    runs the staged, floored, hysteretic planner step (apmoe_plan_online); a
    changed plan is committed to the layer in stream order, so the next
    forward call uses it.  `harm` may be replaced per step (for example by the
    offline table scaled with the library's harm multipliers of the last
    routing, _lib.harm_multipliers)."""

    def __init__(self, layer, levels, harm, nbytes, floor_bits, stage_bits, m_total, hysteresis, bits_now):
        self.layer = layer
        self.levels = np.asarray(levels, dtype=np.int8)
        self.harm = np.asarray(harm, dtype=np.float64)
        self.nbytes = np.asarray(nbytes, dtype=np.uint64)
        self.floor_bits = np.asarray(floor_bits, dtype=np.int8)
        self.stage_bits = np.asarray(stage_bits, dtype=np.int8)
        self.m_total = int(m_total)
        self.hysteresis = int(hysteresis)
        self.bits = np.asarray(bits_now, dtype=np.int8).copy()
        self.stage = -1

    def step(self, m_kv, harm=None):
        """Returns (status, bits, stage, changed); stage -1 = plan kept."""
        if harm is not None:
            self.harm = np.asarray(harm, dtype=np.float64)
        status, bits, stage = _lib.plan_online(self.levels, self.harm, self.nbytes, self.floor_bits,
                                               self.stage_bits, self.m_total, m_kv, self.hysteresis, self.bits)
        changed = bits.tolist() != self.bits.tolist()
        if changed:
            rc = self.layer.commit(bits)
            if rc != _lib.OK:     # the pager could not make the plan resident: keep the old one
                return rc, self.bits.copy(), -1, False
            self.bits = bits
        if stage >= 0:
            self.stage = stage
        return status, bits, stage, changed


def from_inputs(inp, bits=None, mfma_min_tokens=None, device="cuda"):
    """Build device weights and a layer from a generated input set (duck-typed)."""
    cfg = inp.cfg
    experts = ExpertTable(inp.experts, device)
    shared = ExpertTable([inp.shared], device) if inp.shared is not None else None
    b = inp.bits if bits is None else bits
    layer = MoELayer(cfg.E, cfg.H, cfg.I, cfg.k, cfg.T, inp.w_router, inp.bias, cfg.logit_scale, experts,
                     b, shared, cfg.shared_I, mfma_min_tokens, device)
    return layer
