#!/usr/bin/env python3
"""Benchmark of one any-precision MoE-layer step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload qwen_decode]

A step is the whole layer on one batch: route -> permute -> gate/up+SwiGLU ->
down (each on the bit-plane GEMV path and/or the MFMA tile path) -> the fp16
shared expert where the layer has one -> weighted combine.  Inputs are
synthetic and already resident in HBM; the expert weights rotate over R
device replicas so every step reads its planes from HBM rather than from the
256 MB MALL.  Prints one JSON line.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0            # MI355X HBM3E, GB/s
FP16_MFMA_PEAK_TFLOPS = 2500.0   # MI355X dense fp16 MFMA
METRIC = "MoE-layer tokens/s + effective HBM GB/s (% of peak) at mixed 3–6 bit experts"


def expert_bytes(H, I, b):
    """Algorithmic weight bytes of gate+up and of down at bitwidth b."""
    if b == 16:
        return 2 * I * H * 2, H * I * 2
    return 2 * (I * H * b // 8 + I * (1 << b) * 2), H * I * b // 8 + H * (1 << b) * 2


def algorithmic(cfg, bits, counts, mfma_min, n_shared=0):
    """Bytes each launch must move (planes of the top b bits + LUT_b, or fp16 rows,
    plus activations in and out), the expert flops, and the flops per launch.  With n_shared > 0 the
    shared expert runs as n always-on fp16 experts inside the stage launches
    (counts then cover those n experts first, then the routed ones)."""
    H, I, T, k, E = cfg.H, cfg.I, cfg.T, cfg.k, cfg.E
    kk = k + n_shared
    by = {"route": T * H * 2 + E * H * 4 + (E * 4 if cfg.router_bias else 0) + T * k * 8,
          "permute": T * k * 4 + (2 * (E + n_shared) + 1) * 4 + T * kk * 8,
          "gate_up_gemv": 0, "gate_up_tile": 0, "down_gemv": 0, "down_tile": 0,
          "shared_gate_up": 0, "shared_down": 0,
          "combine": T * kk * (H * 4 + 4) + T * k * 4 + T * H * 2
          + (T * H * 4 if cfg.shared_I and not n_shared else 0)}
    flops = 0
    fl = {}
    all_bits = [16] * n_shared + [int(b) for b in bits]
    for e in range(E + n_shared):
        m = int(counts[e])
        if m == 0:
            continue
        wgu, wd = expert_bytes(H, I, all_bits[e])
        path = "tile" if m >= mfma_min else "gemv"
        by["gate_up_" + path] += wgu + m * H * 2 + m * I * 2
        by["down_" + path] += wd + m * I * 2 + m * H * 4
        fl["gate_up_" + path] = fl.get("gate_up_" + path, 0) + 4 * m * H * I
        fl["down_" + path] = fl.get("down_" + path, 0) + 2 * m * H * I
        flops += 6 * m * H * I
    if cfg.shared_I and not n_shared:
        Is = cfg.shared_I
        by["shared_gate_up"] = 2 * Is * H * 2 + T * H * 2 + T * Is * 2
        by["shared_down"] = H * Is * 2 + T * Is * 2 + T * H * 4
        flops += 6 * T * H * Is
    return by, flops, fl


def cpu_baseline(inp, bits, min_s=10.0):
    """The float64 oracle on the host cores: whole layer steps of the same
    workload, repeated until about min_s seconds of work (at least one)."""
    from threadpoolctl import threadpool_info
    from oracle import moe
    t0 = time.perf_counter()
    moe.layer(inp, bits=bits)
    first = time.perf_counter() - t0
    reps = max(1, int(math.ceil(min_s / max(first, 1e-3))))
    for _ in range(reps - 1):
        moe.layer(inp, bits=bits)
    dt = time.perf_counter() - t0
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    return {"value": inp.cfg.T * reps / dt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{reps} full layer step(s) ({inp.cfg.T} tokens each) of the same workload in float64 "
                      f"NumPy, {dt:.1f} s; BLAS threads {threads} of {len(os.sched_getaffinity(0))} host cores"}


def planner_probe(inp, reps=200):
    """Host planner calls at this layer's size (the library's C++ planner):
    one greedy plan, and one online step per KV size while the KV footprint
    sweeps from nothing to the budget slack and back."""
    import numpy as np
    import synth
    from any_precision_quantized_amd import _lib

    cfg = inp.cfg
    pl = inp.plan if inp.plan is not None else synth.gen.planner_inputs(cfg, synth.gen.zipf_prior(cfg.E, 1.1))
    args = (pl["levels"], pl["harm"], pl["bytes"], pl["floors"], pl["budget"])
    _lib.plan_bitwidths(*args)
    t0 = time.perf_counter()
    for _ in range(reps):
        st, bits = _lib.plan_bitwidths(*args)
    greedy_us = (time.perf_counter() - t0) / reps * 1e6
    nb = np.asarray(pl["bytes"], dtype=np.uint64)
    m_total = int(nb[:, 0].sum())
    slack = m_total - int(nb[:, -1].sum())
    stage_bits = np.asarray(pl["levels"][1:], dtype=np.int8)
    kv = [int(slack * (1 - abs(1 - 2 * i / (reps - 1)))) for i in range(reps)]
    now = np.full(cfg.E, int(pl["levels"][0]), dtype=np.int8)
    t0 = time.perf_counter()
    for m_kv in kv:
        st, now, stage = _lib.plan_online(pl["levels"], pl["harm"], nb, pl["floors"], stage_bits, m_total, m_kv,
                                          slack // 64, now)
    online_us = (time.perf_counter() - t0) / reps * 1e6
    return {"experts": int(cfg.E), "levels": len(pl["levels"]), "plan_bitwidths_us": round(greedy_us, 2),
            "plan_online_step_us": round(online_us, 2)}


def counted_traffic(kernel, workload):
    """HBM bytes per launch of `kernel` on `workload` from a committed counter
    summary under profiles/, or None when there is none for that kernel and
    workload or the kernel's sources changed since the counters were taken."""
    import glob
    import hashlib
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "*.md"))):
        fields = {}
        with open(path) as f:
            for line in f:
                line = line.strip()
                for key in ("traffic_kernel", "traffic_workload", "traffic_bytes_per_launch", "sources",
                            "sources_sha256"):
                    if line.startswith(key + ":"):
                        fields[key] = line.split(":", 1)[1].strip()
        if fields.get("traffic_kernel") != kernel or fields.get("traffic_workload") != workload \
                or "sources" not in fields:
            continue
        h = hashlib.sha256()
        try:
            for src in fields["sources"].split():
                with open(os.path.join(ROOT, src), "rb") as f:
                    h.update(f.read())
        except OSError:
            return None
        if h.hexdigest() == fields.get("sources_sha256"):
            return float(fields["traffic_bytes_per_launch"])
        return None
    return None


def paging_probe(cfg, inp, bits, mfma_min, R=1, steps=60, reps=3):
    """Throughput while a re-plan's plane copies run (plane paging).

    R copies of the layer run on paged weights (PagedExperts, one arena and
    pager each), their steps captured as HIP graphs and replayed in turn, so
    that, as in the timed steps, each step reads its weights from HBM rather
    than from the memory-side cache; the first copy is re-planned.  Each
    repetition demotes every bit-plane expert above 3 bits
    by one bit (committed, so only the lower LUTs move), enqueues `steps`
    graph replays and, when two thirds of them are still queued, stages the
    promotion back to `bits` (the host issues the copies; the copy engines
    move them while the replays run), enqueues `steps` more replays, waits
    for the copies and commits (the commit places the staged planes and LUTs
    on the layer's stream; its time between two steps is `commit_us`).  The
    host stays milliseconds ahead of the GPU, so every step interval comes
    from GPU events.  The copy window opens at the event of the step the host
    saw end just before staging and closes when the host sees a 4-byte
    device-to-host copy, queued on the copy stream behind the staged copies,
    land in pinned memory.  With the copy stream in the same hardware queue
    as the layer's stream that copy waits for the replays queued before it,
    so the window would be an upper bound; PagedExperts picks a copy stream
    outside the current stream's queue (`copy_ms_idle` times the same copies
    on an idle GPU, with events on the copy stream).  The replays before the
    window (same bitwidths, no copies) are the baseline; the steps that
    overlap the window, against it, give the loss, and `lost_us` is the time
    every replay after the stage call took beyond the baseline, per re-plan
    (wherever the copies landed)."""
    import numpy as np
    import torch
    from any_precision_quantized_amd import _lib
    from any_precision_quantized_amd import layer as L
    from any_precision_quantized_amd.paging import PagedExperts, arena_bytes_for

    x = torch.from_numpy(np.ascontiguousarray(inp.x).view(np.int16)).cuda().view(torch.float16)
    pes, graphs = [], []
    for _ in range(max(1, R)):
        p_ = PagedExperts(inp.experts, cfg.H, cfg.I, arena_bytes_for(cfg.H, cfg.I, cfg.E))
        shared = L.ExpertTable([inp.shared]) if inp.shared is not None else None
        lay = L.MoELayer(cfg.E, cfg.H, cfg.I, cfg.k, cfg.T, inp.w_router, inp.bias, cfg.logit_scale, p_.table, bits,
                         shared, cfg.shared_I, mfma_min)
        p_.attach(lay, bits)
        pes.append(p_)
        graphs.append(lay.graph(x))
    pe = pes[0]
    stream = torch.cuda.current_stream()
    low = np.where((bits > 3) & (bits <= 6), bits - 1, bits).astype(np.int8)
    turn = [0]

    def event(s=stream):
        e = torch.cuda.Event(enable_timing=True)
        e.record(s)
        return e

    def enqueue(n, evs):
        for _ in range(n):
            graphs[turn[0] % len(graphs)].replay()
            turn[0] += 1
            evs.append(event())

    hip = ctypes.CDLL("libamdhip64.so")
    flag_dev = [torch.full((1,), v, dtype=torch.int32, device="cuda") for v in (1, 2)]
    flag_host = torch.zeros(1, dtype=torch.int32, pin_memory=True)
    flag_view = flag_host.numpy()
    for g in graphs:
        g.replay()
    torch.cuda.synchronize()
    before, during, lost, copy_ms, stage_us, commit_us = [], [], [], [], [], []
    for rep in range(reps):
        if pe.apply(low) != _lib.OK:
            raise RuntimeError("paging probe: demotion did not fit")
        torch.cuda.synchronize()
        evs = [event()]
        enqueue(steps, evs)
        anchor = evs[-1 - max(5, 2 * steps // 3)]
        give_up = time.perf_counter() + 30.0
        while not anchor.query():
            if time.perf_counter() > give_up:
                raise RuntimeError("paging probe: the layer did not advance within 30 s")
        ta = time.perf_counter()
        if pe.stage(bits) != _lib.OK:
            raise RuntimeError("paging probe: promotion did not fit")
        stage_us.append((time.perf_counter() - ta) * 1e6)
        mark = rep % 2 + 1
        if hip.hipMemcpyAsync(ctypes.c_void_p(flag_host.data_ptr()), ctypes.c_void_p(flag_dev[rep % 2].data_ptr()),
                              ctypes.c_size_t(4), 2, ctypes.c_void_p(pe.copy_stream.cuda_stream)) != 0:
            raise RuntimeError("paging probe: marker copy failed")
        enqueue(steps, evs)
        while int(flag_view[0]) != mark:
            if time.perf_counter() > give_up:
                raise RuntimeError("paging probe: the copies did not finish within 30 s")
        tb = time.perf_counter()
        k0 = event()
        pe.commit(bits)
        k1 = event()
        torch.cuda.synchronize()
        commit_us.append(k0.elapsed_time(k1) * 1e3)
        lo = evs[0].elapsed_time(anchor)
        hi = lo + (tb - ta) * 1e3
        copy_ms.append(hi - lo)
        t = [evs[0].elapsed_time(e) for e in evs]
        iv = [(t[i + 1] - t[i]) * 1e3 for i in range(len(t) - 1)]
        base = [iv[i] for i in range(len(iv)) if t[i + 1] <= lo and i > 0]
        over = [iv[i] for i in range(len(iv)) if t[i + 1] > lo and t[i] < hi]
        after = [iv[i] for i in range(len(iv)) if t[i + 1] > lo]
        before += base
        during += over
        lost.append(sum(after) - len(after) * float(np.mean(base)))
    st = pe.stats()
    # the same promotion on an idle GPU, timed on the copy stream
    idle_ms = []
    for _ in range(reps):
        if pe.apply(low) != _lib.OK:
            raise RuntimeError("paging probe: demotion did not fit")
        torch.cuda.synchronize()
        e0 = event(pe.copy_stream)
        if pe.stage(bits) != _lib.OK:
            raise RuntimeError("paging probe: promotion did not fit")
        e1 = event(pe.copy_stream)
        pe.commit(bits)
        torch.cuda.synchronize()
        idle_ms.append(e0.elapsed_time(e1))
    del graphs
    for p_ in pes:
        p_.close()
    base_us, dur_us = float(np.mean(before)), float(np.mean(during))
    cm, ci = float(np.mean(copy_ms)), float(np.median(idle_ms))
    h2d = int(st["h2d"])
    return {"replan": "every bit-plane expert above 3 bits promoted by one plane (b-1 -> b) while the layer runs",
            "copy_ranges": int(st["ranges"]),
            "stage_host_us": round(float(np.median(stage_us)), 1),
            "commit_us": round(float(np.median(commit_us)), 1),
            "h2d_bytes": h2d, "d2d_bytes": int(st["d2d"]),
            "copy_ms_idle": round(ci, 3), "h2d_GBps": round(h2d / (ci * 1e-3) / 1e9, 2),
            "copy_ms": round(cm, 3),
            "step_us_before": round(base_us, 2),
            "step_us_during_copy": round(dur_us, 2),
            "steps_overlapping_copy": len(during),
            "loss": round(dur_us / base_us - 1.0, 4),
            "paged_layers": len(pes),
            "lost_us": round(float(np.mean(lost)), 1)}


def codec_probe(inp, reps=5):
    """Lossless exponent codec on the layer's fp16 weights (the shared expert,
    else the routed experts at 16 bits): host encode time, coded size, and
    the GPU decode of all of them (one batched launch, `reps` of them replayed
    from a HIP graph) timed with events on the current stream."""
    import numpy as np
    import torch
    from any_precision_quantized_amd import _lib

    cfg = inp.cfg
    mats = []
    if inp.shared is not None:
        mats += [inp.shared[m].w16 for m in ("gate", "up", "down")]
    for e, b in enumerate(inp.bits if inp.bits is not None else []):
        if int(b) == 16:
            mats += [inp.experts[e][m].w16 for m in ("gate", "up", "down")]
    mats = [m for m in mats if m is not None]
    if not mats:
        return None
    t0 = time.perf_counter()
    encs = [_lib.exp_encode(np.ascontiguousarray(m).view(np.uint16).reshape(-1)) for m in mats]
    enc_s = time.perf_counter() - t0
    dev = []
    for enc in encs:
        d = {k: torch.from_numpy(np.ascontiguousarray(enc[k]).view(v)).cuda()
             for k, v in (("words", np.int32), ("block_off", np.int32), ("lo", np.uint8), ("table", np.int16))}
        d["out"] = torch.empty(enc["n"], dtype=torch.int16, device="cuda")
        dev.append(d)
    stream = torch.cuda.current_stream()

    def run():   # every matrix in one launch (a matrix alone leaves most of the GPU idle)
        for i in range(0, len(dev), _lib.EXP_MAX_BATCH):
            _lib.exp_decode_batch(dev[i:i + _lib.EXP_MAX_BATCH])

    run()
    torch.cuda.synchronize()
    for d, m in zip(dev, mats):   # lossless on every matrix
        ref = torch.from_numpy(np.ascontiguousarray(m).view(np.int16).reshape(-1)).cuda()
        if not torch.equal(d["out"], ref):
            raise RuntimeError("exponent codec: decode differs from the weights")
    # the decodes replayed from a HIP graph: launched one by one from Python,
    # the host takes longer per call than a small decode takes on the GPU
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(reps):
            run()
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) / reps * 1e3
    del g
    raw = sum(2 * enc["n"] for enc in encs)
    coded = sum(4 * enc["words"].size + enc["lo"].size + 4 * enc["block_off"].size + 2 * 4096 for enc in encs)
    moved = coded + raw                       # read the coded form, write the weights
    return {"weights": "fp16 " + ("shared expert" if inp.shared is not None else "experts at 16 bits"),
            "matrices": len(mats), "raw_bytes": raw, "coded_bytes": coded, "ratio": round(coded / raw, 4),
            "encode_host_s": round(enc_s, 3), "decode_us": round(us, 2),
            "decode_GBps": round(raw / (us * 1e-6) / 1e9, 1),
            "decode_hbm_frac": round(moved / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}


def measure(args, cfg, inp, bits, steps, warmup, probe_steps, time_stats=True):
    """Time `steps` whole layer steps of one workload (HIP graph replays over
    rotating weight replicas) and, in a separate pass, every launch of a step
    with events on its stream.  Returns the bench fields of that workload."""
    import numpy as np
    import torch

    from any_precision_quantized_amd import _lib
    from any_precision_quantized_amd import layer as L

    layer = L.from_inputs(inp, bits=bits, mfma_min_tokens=args.mfma_min_tokens)
    mfma_min = layer.mfma_min_tokens
    x = torch.from_numpy(np.ascontiguousarray(inp.x).view(np.int16)).cuda().view(torch.float16)
    layer.forward(x)
    torch.cuda.synchronize()
    counts = layer.counts.cpu().numpy()
    nsh = layer.n_shared
    by, flops, launch_flops = algorithmic(cfg, bits, counts, mfma_min, nsh)
    step_bytes = sum(by.values())
    weight_bytes = sum(v for k_, v in by.items() if k_.startswith(("gate_up", "down", "shared")))
    R = max(2, math.ceil(args.replica_bytes / max(1, weight_bytes)))
    tables = [layer.experts] + [layer.experts.replicate() for _ in range(R - 1)]
    shared = [layer.shared] + ([layer.shared.replicate() for _ in range(R - 1)] if layer.shared else [None] * (R - 1))

    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream
    side = getattr(layer, "side", None)           # the shared expert's stream (when not fused)
    if args.serial_shared and side is not None:
        side = stream
    sp2 = side.cuda_stream if side is not None else None
    ev_fork, ev_join = torch.cuda.Event(), torch.cuda.Event()
    lib = _lib._lib()
    T, H, I, E, k = cfg.T, cfg.H, cfg.I, cfg.E, cfg.k
    p = lambda t: None if t is None else t.data_ptr()  # noqa: E731
    ws, wsb = (p(layer.ws), layer.ws.numel()) if layer.ws is not None else (None, 0)
    ws_sh = getattr(layer, "ws_sh", None)
    ws2, wsb2 = (p(ws_sh), ws_sh.numel()) if ws_sh is not None else (None, 0)

    # Every launch of a step as (name, callable, stream) with its raw arguments
    # bound once; "fork"/"join" entries order the shared expert's side stream.
    E2, kk = E + nsh, k + nsh

    def launches(r):
        tab, sh = tables[r], shared[r]
        if nsh:
            tab, sh = layer._fused(tab, sh), None   # shared parts run as always-on experts
        seq = []
        if sh is not None:
            Is = cfg.shared_I
            seq.append(("fork", None, None))
            seq.append(("shared_gate_up", lambda: lib.apmoe_bitplane_lut_gemm(
                _lib.GATE_UP_SWIGLU, p(sh.desc), p(layer.sh_bits), 1, p(layer.sh_offsets), p(layer.sh_slots), 1,
                p(x), p(layer.A_sh), T, H, Is, mfma_min, ws2, wsb2, sp2), side))
            seq.append(("shared_down", lambda: lib.apmoe_bitplane_lut_gemm(
                _lib.DOWN, p(sh.desc), p(layer.sh_bits), 1, p(layer.sh_offsets), p(layer.sh_slots), 1,
                p(layer.A_sh), p(layer.Y_sh), T, H, Is, mfma_min, ws2, wsb2, sp2), side))
            seq.append(("side_done", None, None))
        seq += [
            ("route", lambda: lib.apmoe_route(p(x), T, H, p(layer.w_router), p(layer.bias), layer.logit_scale,
                                              E, k, p(layer.topk_ids), p(layer.topk_w), p(layer.x_norms), ws, wsb,
                                              sp), stream),
            ("permute", lambda: lib.apmoe_permute(p(layer.topk_ids), T, k, E, nsh, p(layer.counts), p(layer.offsets),
                                                  p(layer.sorted_slots), p(layer.pos_of_slot), p(layer.topk_w),
                                                  p(layer.x_norms), p(layer.mass), p(layer.wnorm), p(layer.ws_stats),
                                                  layer.ws_stats.numel(), sp), stream),
        ]
        for stage, name, src, dst in ((_lib.GATE_UP_SWIGLU, "gate_up", x, layer.A),
                                      (_lib.DOWN, "down", layer.A, layer.Y)):
            # below T = mfma_min_tokens the library launches no tile kernel
            paths = ((_lib.ONLY_GEMV, "gemv"),) + (((_lib.ONLY_TILE, "tile"),) if T >= mfma_min else ())
            for flag, path in paths:
                seq.append((f"{name}_{path}", (lambda st=stage | flag, s_=src, d_=dst: lib.apmoe_bitplane_lut_gemm(
                    st, p(tab.desc), p(layer.bits), E2, p(layer.offsets), p(layer.sorted_slots), kk, p(s_), p(d_),
                    T, H, I, mfma_min, ws, wsb, sp)), stream))
        ysh = p(layer.Y_sh) if sh is not None else None
        if sh is not None:
            seq.append(("join", None, None))
        seq.append(("combine", lambda: lib.apmoe_combine(p(layer.Y), p(layer.pos_of_slot), p(layer.topk_w), T, k,
                                                          nsh, H, ysh, p(layer.out), sp), stream))
        return seq

    seqs = [launches(r) for r in range(R)]
    names = [n for n, fn, _ in seqs[0] if fn is not None]

    def run(seq, timed_name=None, ev=None):
        for n, fn, st in seq:
            if n == "fork":
                ev_fork.record(stream)
                side.wait_event(ev_fork)
                continue
            if n == "side_done":
                ev_join.record(side)
                continue
            if n == "join":
                stream.wait_event(ev_join)
                continue
            if n == timed_name:   # events on the stream the launch runs on
                ev[0].record(st)
                rc = fn()
                ev[1].record(st)
            else:
                rc = fn()
            if rc != 0:
                raise _lib.ApmoeError(rc, n)

    # Per-launch durations (separate pass) to find the dominant kernel.
    per = {n: 0.0 for n in names}
    for i in range(warmup):
        run(seqs[i % R])
    torch.cuda.synchronize()
    for name in names:
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(probe_steps)]
        for i in range(probe_steps):
            run(seqs[i % R], name, evs[i])
        torch.cuda.synchronize()
        per[name] = sum(a.elapsed_time(b) for a, b in evs) / probe_steps * 1e3   # us
    dominant = max(names, key=lambda n: per[n])
    route_stats_us = route_stats_in_step_us = None
    if time_stats:
        # routing statistics for the planner (outside the layer step: the planner
        # reads them at a step boundary), timed the same way
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(probe_steps)]
        for i in range(probe_steps):
            evs[i][0].record(stream)
            rc = lib.apmoe_route_stats(p(x), T, H, p(layer.topk_ids), p(layer.topk_w), k, E, p(layer.mass),
                                       p(layer.wnorm), p(layer.ws_stats), layer.ws_stats.numel(), sp)
            evs[i][1].record(stream)
            if rc != 0:
                raise _lib.ApmoeError(rc, "route_stats")
        torch.cuda.synchronize()
        route_stats_us = sum(a.elapsed_time(b) for a, b in evs) / probe_steps * 1e3

        # what the statistics cost inside the step: router + grouping with the
        # token norms and per-expert sums, against the same two launches without
        def pair(stats):
            nrm = p(layer.x_norms) if stats else None
            rc = lib.apmoe_route(p(x), T, H, p(layer.w_router), p(layer.bias), layer.logit_scale, E, k,
                                 p(layer.topk_ids), p(layer.topk_w), nrm, ws, wsb, sp)
            if rc == 0:
                rc = lib.apmoe_permute(p(layer.topk_ids), T, k, E, nsh, p(layer.counts), p(layer.offsets),
                                       p(layer.sorted_slots), p(layer.pos_of_slot),
                                       p(layer.topk_w) if stats else None, nrm,
                                       p(layer.mass) if stats else None, p(layer.wnorm) if stats else None,
                                       p(layer.ws_stats) if stats else None,
                                       layer.ws_stats.numel() if stats else 0, sp)
            if rc != 0:
                raise _lib.ApmoeError(rc, "route + permute")

        # each variant captured as a HIP graph of n back-to-back pairs (the way
        # the step runs), replayed in alternation with the other
        n = 50
        graphs = {}
        for stats in (False, True):
            for _ in range(3):
                pair(stats)
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                sp = torch.cuda.current_stream().cuda_stream
                for _ in range(n):
                    pair(stats)
            graphs[stats] = g
        sp = stream.cuda_stream
        torch.cuda.synchronize()
        pair_us = {}
        for stats in (False, True) * 4:
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            graphs[stats].replay()
            e1.record(stream)
            torch.cuda.synchronize()
            pair_us.setdefault(stats, []).append(e0.elapsed_time(e1) * 1e3 / n)
        del graphs
        route_stats_in_step_us = float(np.median(pair_us[True]) - np.median(pair_us[False]))

    # Timed region: K whole steps; the dominant launch is bracketed by events.
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for i in range(warmup):
        run(seqs[i % R])
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        run(seqs[i % R], dominant, evs[i])
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    dom_us = sum(a.elapsed_time(b) for a, b in evs) / steps * 1e3

    ms_eager = dt / steps * 1e3
    # The same K steps replayed as HIP graphs (one per weight replica): what a
    # serving loop that captures the layer pays, without per-launch host work.
    use_graph = not args.no_graph and side is None
    if use_graph:
        graphs = [layer.graph(x, tables[r], shared[r]) for r in range(R)]
        for i in range(warmup):
            graphs[i % R].replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            graphs[i % R].replay()
        torch.cuda.synchronize()
        dt = time.perf_counter() - t0
        del graphs
    ms_per_step = dt / steps * 1e3
    tokens_per_s = T * steps / dt

    # The heavy launches' average durations from HIP graphs of that launch
    # alone: 4R launches over the weight replicas in turn, replayed with events
    # on the stream around the replays.  This is the kernels' own time; an
    # event pair around one eager launch also holds its dispatch gap.
    def launch_graph_us(name, reps=4):
        nonlocal sp
        fns = [next(fn for n_, fn, _ in seqs[r] if n_ == name) for r in range(R)]
        n = 4 * R
        g = torch.cuda.CUDAGraph()
        keep = sp
        try:
            with torch.cuda.graph(g):
                sp = torch.cuda.current_stream().cuda_stream   # the launches read sp when called
                for i in range(n):
                    rc = fns[i % R]()
                    if rc != 0:
                        raise _lib.ApmoeError(rc, name)
        finally:
            sp = keep
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        del g
        return e0.elapsed_time(e1) * 1e3 / (reps * n)

    graph_us = {}
    if use_graph:
        for name in names:
            if name.endswith(("_gemv", "_tile")):
                graph_us[name] = launch_graph_us(name)
    dom_us_eager = dom_us
    dom_us = graph_us.get(dominant, dom_us)
    layer_gbs = step_bytes / (ms_per_step * 1e-3) / 1e9
    dom_bytes = by.get(dominant, 0)
    if dominant.endswith("_tile"):
        # the MFMA tile path is bound by the matrix cores: flops against the fp16 peak
        dom_flops = launch_flops.get(dominant, 0)
        roofline = {"bound": "mfma", "kernel": dominant, "achieved": dom_flops / (dom_us * 1e-6) / 1e12,
                    "peak": FP16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                    "frac": dom_flops / (dom_us * 1e-6) / 1e12 / FP16_MFMA_PEAK_TFLOPS,
                    "traffic": counted_traffic(dominant, cfg.name), "algorithmic_flops": dom_flops,
                    "algorithmic_bytes": dom_bytes, "avg_us": dom_us, "avg_us_eager": dom_us_eager}
    else:
        achieved = dom_bytes / (dom_us * 1e-6) / 1e9
        roofline = {"bound": "hbm", "kernel": dominant, "achieved": achieved, "peak": HBM_PEAK_GBS,
                    "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS, "traffic": counted_traffic(dominant, cfg.name),
                    "algorithmic_bytes": dom_bytes, "avg_us": dom_us, "avg_us_eager": dom_us_eager}
    result = {
        "metric": METRIC,
        "value": tokens_per_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": f"{cfg.name}: E{E} H{H} I{I} top-{k} T{T}"
                               + (f" + fp16 shared expert I{cfg.shared_I}" if cfg.shared_I else "")
                               + f", bits {dict(sorted((int(b), int((bits == b).sum())) for b in set(bits.tolist())))}",
                   "mfma_min_tokens": mfma_min, "weight_replicas": R, "hip_graph": use_graph,
                   "shared_as_always_on_experts": nsh,
                   "groups": sorted([int(c) for c in counts[nsh:] if c > 0], reverse=True)},
        "ms_per_step_eager": ms_eager,
        "hbm_gbs": layer_gbs,
        "hbm_frac": layer_gbs / HBM_PEAK_GBS,
        "expert_tflops": flops / (ms_per_step * 1e-3) / 1e12,
        "roofline": roofline,
        "per_launch_us": {n: round(per[n], 2) for n in names},
        "launch_us_graph": {n: round(v, 2) for n, v in graph_us.items()},
        "route_stats_us": None if route_stats_us is None else round(route_stats_us, 2),
        "route_stats_in_step_us": None if route_stats_in_step_us is None else round(route_stats_in_step_us, 2),
        "per_launch_bytes": {n: int(by.get(n, 0)) for n in names},
    }
    gu = graph_us.get("gate_up_gemv", per.get("gate_up_gemv"))
    dn = graph_us.get("down_gemv", per.get("down_gemv"))
    if gu and dn and by["gate_up_gemv"] + by["down_gemv"] > 0:   # the two GEMV stages together against HBM peak
        gb = (by["gate_up_gemv"] + by["down_gemv"]) / ((gu + dn) * 1e-6) / 1e9
        result["gemv_stages"] = {"algorithmic_bytes": int(by["gate_up_gemv"] + by["down_gemv"]),
                                 "us": round(gu + dn, 2), "GBps": round(gb, 1), "frac": round(gb / HBM_PEAK_GBS, 4)}
    return result


def planned_bits(inp):
    """Bitwidths of a generated layer: fixed by the workload, or from the host planner."""
    import numpy as np
    from any_precision_quantized_amd import _lib
    if inp.bits is not None:
        return np.asarray(inp.bits, dtype=np.int8)
    pl = inp.plan
    st, bits = _lib.plan_bitwidths(pl["levels"], pl["harm"], pl["bytes"], pl["floors"], pl["budget"])
    if st != _lib.OK:
        raise RuntimeError(f"planner: {_lib.strerror(st)}")
    return bits


WORKLOADS = ["tiny", "qwen_decode", "mixtral_decode_t1", "mixtral_decode_t8", "mixtral_decode_t32", "e128_decode",
             "mixtral_prefill"]


def other_workloads(args, primary):
    """A compact line for every other workload of the layer: whole-step time
    and tokens/s (graph replays), the dominant launch against its roofline,
    and the two GEMV stages together against HBM peak.  The Mixtral-shaped
    decode batches share one draw of weights (they differ only in tokens)."""
    import dataclasses
    import gc

    import torch

    import synth
    out = {}
    mixtral = None
    for name in WORKLOADS:
        if name == primary:
            continue
        cfg = synth.get(name)
        if name.startswith("mixtral_decode_t"):
            if mixtral is None:
                mixtral = synth.make_inputs(synth.get("mixtral_decode_t32"), seed=0)
            inp = dataclasses.replace(mixtral, cfg=cfg, x=mixtral.x[: cfg.T])
        else:
            inp = synth.make_inputs(cfg, seed=0)
        prefill = cfg.T > 1024
        steps, warmup, probe = (args.workload_steps // 5, 3, 5) if prefill else (args.workload_steps, 10, 20)
        r = measure(args, cfg, inp, planned_bits(inp), steps, warmup, probe, time_stats=False)
        rf = r["roofline"]
        out[name] = {"workload": r["config"]["workload"], "ms_per_step": round(r["ms_per_step"], 4),
                     "tokens_per_s": round(r["value"], 1), "steps": steps,
                     "dominant": {k: rf[k] for k in ("kernel", "bound", "achieved", "peak", "unit", "frac", "avg_us")},
                     "gemv_stages": r.get("gemv_stages"), "per_launch_us": r["per_launch_us"]}
        del inp
        gc.collect()
        torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="qwen_decode")
    ap.add_argument("--mfma-min-tokens", type=int, default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-paging-probe", action="store_true",
                    help="skip the throughput-under-plane-paging probe")
    ap.add_argument("--no-codec-probe", action="store_true",
                    help="skip the exponent-codec decode probe")
    ap.add_argument("--no-graph", action="store_true",
                    help="time eager launches only (no HIP graph replay of the step)")
    ap.add_argument("--serial-shared", action="store_true",
                    help="run the shared expert on the main stream instead of the side stream")
    ap.add_argument("--replica-bytes", type=float, default=1.0e9,
                    help="weight bytes the rotating replicas must span (MALL defeat)")
    ap.add_argument("--no-workloads", action="store_true",
                    help="measure only --workload (no compact line per other workload)")
    ap.add_argument("--workload-steps", type=int, default=50,
                    help="timed steps per other workload (a fifth of it for the prefill)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only copy MIB MiB device to device five times (scale for HBM byte counters)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: this layer runs on one GPU; --gpus must be 1 (no multi-GPU path is built)",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import synth
    from any_precision_quantized_amd import _lib
    from any_precision_quantized_amd import layer as L

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    if args.calibrate_copy:
        n = args.calibrate_copy << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "launches": 5}), flush=True)
        return
    cfg = synth.get(args.workload)
    inp = synth.make_inputs(cfg, seed=0)
    bits = planned_bits(inp)
    result = measure(args, cfg, inp, bits, args.steps, args.warmup, max(5, min(50, args.steps)))
    mfma_min = args.mfma_min_tokens or L.auto_mfma_min_tokens(cfg.T, cfg.k, cfg.E)
    if not args.no_workloads:
        result["workloads"] = other_workloads(args, cfg.name)
    if not args.no_paging_probe:
        result["paging"] = paging_probe(cfg, inp, bits, mfma_min, R=result["config"]["weight_replicas"])
    if not args.no_codec_probe:
        result["exp_codec"] = codec_probe(inp, reps=10)
    result["planner"] = planner_probe(inp)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(inp, bits)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
