"""Helpers for the GPU parity tests: run the layer step by step through the
C ABI and compare each step with the oracle."""
from __future__ import annotations

import dataclasses
import sys

import numpy as np

import synth
from any_precision_quantized_amd import _lib
from any_precision_quantized_amd import layer as L
from oracle import moe

REL, ABS = 2e-3, 1e-5           # |y - y_ref| <= REL * sum|w||x| + ABS per element
GATE_ATOL = 1e-6                # fp64 softmax stored as fp32
ROUTE_EPS = 1e-12               # near-tie guard, relative to scale * sum|x||Wr|


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


_INPUT_CACHE = {}


def inputs(name_or_cfg, seed=0):
    """Generated inputs; the Mixtral decode token counts share one draw."""
    cfg = synth.get(name_or_cfg) if isinstance(name_or_cfg, str) else name_or_cfg
    key = (cfg, seed)
    if key in _INPUT_CACHE:
        return _INPUT_CACHE[key]
    if cfg.name.startswith("mixtral_decode_t") and cfg.name != "mixtral_decode_t32":
        big = inputs("mixtral_decode_t32", seed)
        inp = dataclasses.replace(big, cfg=cfg, x=big.x[: cfg.T])
    else:
        inp = synth.make_inputs(cfg, seed=seed)
    _INPUT_CACHE[key] = inp
    return inp


def run_layer(inp, bits, mfma_min_tokens=None, table=None, shared=None, layer=None):
    import torch
    if layer is None:
        layer = L.from_inputs(inp, bits=bits, mfma_min_tokens=mfma_min_tokens)
    elif mfma_min_tokens is not None:
        layer.mfma_min_tokens = mfma_min_tokens
    x = torch.from_numpy(np.ascontiguousarray(inp.x).view(np.int16)).cuda().view(torch.float16)
    out = layer.forward(x, table, shared)
    torch.cuda.synchronize()
    got = dict(ids=layer.topk_ids.cpu().numpy(), gates=layer.topk_w.cpu().numpy(),
               counts=layer.counts.cpu().numpy(), offsets=layer.offsets.cpu().numpy(),
               sorted_slots=layer.sorted_slots.cpu().numpy(), pos_of_slot=layer.pos_of_slot.cpu().numpy(),
               A=layer.A.float().cpu().numpy(), Y=layer.Y.cpu().numpy(), out=out.float().cpu().numpy())
    if layer.n_shared:
        got = routed_view(got, layer.T, layer.k, layer.n_shared)
    return layer, got


def routed_view(got, T, k, n):
    """The grouping of a layer whose shared expert runs as n always-on experts
    (experts 0..n-1, slots t*(k+n) + j for j < n), checked for those experts and
    returned in the routed-only frame (experts 0..E-1, slots t*k + j)."""
    kk = k + n
    counts, offsets, ss, pos = got["counts"], got["offsets"], got["sorted_slots"], got["pos_of_slot"]
    assert counts[:n].tolist() == [T] * n, "every token reaches every always-on expert once"
    for v in range(n):
        assert np.array_equal(ss[v * T:(v + 1) * T], np.arange(T) * kk + v), "always-on slots in token order"
    base = n * T
    rs = ss[base:]
    slot = (rs // kk) * k + (rs % kk - n)
    routed_pos = pos.reshape(T, kk)[:, n:].reshape(-1) - base
    out = dict(got)
    out.update(counts=counts[n:], offsets=offsets[n:] - base, sorted_slots=slot.astype(ss.dtype),
               pos_of_slot=routed_pos.astype(pos.dtype), A=got["A"][base:], Y=got["Y"][base:])
    return out


def check_route(inp, got, ref_ids, ref_gates, ref_logits):
    cfg = inp.cfg
    k = cfg.k
    mag = cfg.logit_scale * (np.abs(inp.x.astype(np.float64)) @ np.abs(inp.w_router.astype(np.float64)).T)
    eps = ROUTE_EPS * mag.max(axis=1) + 1e-300
    margin = moe.route_margin(ref_logits, k)
    clear = margin >= eps
    n_amb = int((~clear).sum())
    assert np.array_equal(got["ids"][clear], ref_ids[clear]), "routing ids differ"
    # ambiguous tokens: the chosen set must still be a valid top-k within eps
    for t in np.nonzero(~clear)[0]:
        chosen = ref_logits[t][got["ids"][t]]
        kth = np.sort(ref_logits[t])[::-1][k - 1]
        assert np.all(chosen >= kth - eps[t])
    tok = clear
    assert np.all(np.abs(got["gates"][tok] - ref_gates[tok]) <= GATE_ATOL), \
        float(np.abs(got["gates"][tok] - ref_gates[tok]).max())
    return n_amb


def check_grouping(cfg, got):
    counts, offsets, ss, pos = moe.group(got["ids"], cfg.E)
    assert np.array_equal(got["counts"], counts)
    assert np.array_equal(got["offsets"], offsets)
    assert np.array_equal(got["sorted_slots"], ss)
    assert np.array_equal(got["pos_of_slot"], pos)


def check_experts(inp, bits, got, experts=None):
    """Per-expert A (against the oracle on the same grouping) and Y (against the
    oracle fed with the GPU's own A)."""
    cfg = inp.cfg
    offs = got["offsets"]
    worst = 0.0
    es = range(cfg.E) if experts is None else experts
    for e in es:
        lo, hi = int(offs[e]), int(offs[e + 1])
        if hi == lo:
            continue
        A_ref, A_bound = moe.expert_gate_up_sorted(inp, bits, offs, got["sorted_slots"], e)
        dA = np.abs(got["A"][lo:hi] - A_ref)
        assert np.all(dA <= A_bound), f"A of expert {e} (bits {bits[e]}): worst {(dA / A_bound).max():.3g}"
        Y_ref, Y_bound = moe.expert_down_sorted(inp, bits, offs, got["A"], e)
        dY = np.abs(got["Y"][lo:hi] - Y_ref)
        assert np.all(dY <= Y_bound), f"Y of expert {e} (bits {bits[e]}): worst {(dY / Y_bound).max():.3g}"
        worst = max(worst, float((dA / A_bound).max()), float((dY / Y_bound).max()))
    return worst


def check_out(got, ref, tokens=None):
    tok = np.arange(got["out"].shape[0]) if tokens is None else np.asarray(tokens)
    d = np.abs(got["out"][tok] - ref["out"][tok])
    bound = REL * ref["mag"][tok] + ABS
    ratio = float((d / bound).max())
    assert np.all(d <= bound), f"layer output: worst error / bound = {ratio:.3g}"
    return ratio
