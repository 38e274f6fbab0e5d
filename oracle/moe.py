"""Plain float64 oracle of one MoE expert-FFN layer over any-precision weights.

What it follows:

* Weights: each expert weight matrix is split into bit-planes plus per-row
  lookup tables, and one stored weight set serves 3, 4, 5 or 6 bits or an
  fp16 fallback ("内存的饥饿游戏：当 MoE 权重与 KV 缓存争夺 GPU 的每一字节",
  zhichai.net, section "核心洞察：权重也能分页").  The b-bit code of a weight is
  its top b bit-planes; the weight is that row's b-bit table entry.
* Routing: top-k of the router logits, then a softmax over the k chosen
  logits; grouping of the token slots by expert in (expert, slot) order.
* Expert FFN: SwiGLU, a = silu(W_gate x) * (W_up x), y = W_down a.
* Combine: out[t] = sum_j gate[t, j] * y_{expert(t, j)}(t), plus an always-on
  fp16 shared expert with weight 1 where the layer has one.

The page gives no formulas for the routing or the FFN; the readings above are
the plain ones for an MoE layer and are listed with the other readings in the
design notes of this repository.
"""
from __future__ import annotations

import math

import numpy as np

F64 = np.float64


# ----------------------------------------------------------------------------
# Storage format: bit-planes -> codes -> weights
# ----------------------------------------------------------------------------

def plane_bit(planes: np.ndarray, p: int) -> np.ndarray:
    """Bit of every weight in plane p: bit i of word w is column 32*w + i."""
    words = planes[p]                                   # [rows, W] uint32
    rows, W = words.shape
    shifts = np.arange(32, dtype=np.uint32)
    bits = (words[:, :, None] >> shifts[None, None, :]) & np.uint32(1)
    return bits.reshape(rows, W * 32).astype(np.uint8)


def decode_codes(planes: np.ndarray, b: int) -> np.ndarray:
    """b-bit code of every weight: plane 0 is the most significant bit,
    code_b = sum over p < b of bit_p << (b - 1 - p)."""
    if not 1 <= b <= planes.shape[0]:
        raise ValueError("b out of range")
    code = None
    for p in range(b):
        term = plane_bit(planes, p).astype(np.int64) << (b - 1 - p)
        code = term if code is None else code + term
    return code


def dequant(mat, b: int) -> np.ndarray:
    """Dense float64 weights of one matrix at bitwidth b (16 = fp16 fallback)."""
    if b == 16:
        return mat.w16.astype(F64)
    code = decode_codes(mat.planes, b)
    lut = mat.luts[b - 3].astype(F64)                   # [rows, 2**b]
    return np.take_along_axis(lut, code, axis=1)


# ----------------------------------------------------------------------------
# Router: top-k, then softmax over the selected logits
# ----------------------------------------------------------------------------

def router_logits(x, w_router, bias=None, scale=1.0) -> np.ndarray:
    """L[t, e] = scale * (x[t] . w_router[e] + bias[e]), in float64."""
    L = x.astype(F64) @ w_router.astype(F64).T
    if bias is not None:
        L = L + bias.astype(F64)[None, :]
    return F64(scale) * L


def route(x, w_router, bias=None, scale=1.0, k=1):
    """Top-k experts per token (descending logit, ties to the lower index) and
    their gates, a softmax over the k chosen logits."""
    L = router_logits(x, w_router, bias, scale)
    T, E = L.shape
    if not 1 <= k <= E:
        raise ValueError("k out of range")
    order = np.argsort(-L, axis=1, kind="stable")       # stable: equal logits keep index order
    ids = order[:, :k]
    sel = np.take_along_axis(L, ids, axis=1)
    z = np.exp(sel - sel.max(axis=1, keepdims=True))
    gates = z / z.sum(axis=1, keepdims=True)
    return ids.astype(np.int64), gates, L


def route_margin(L: np.ndarray, k: int) -> np.ndarray:
    """Gap between the k-th and (k+1)-th largest logit per token (inf when k = E)."""
    s = -np.sort(-L, axis=1)
    if k >= L.shape[1]:
        return np.full(L.shape[0], np.inf)
    return s[:, k - 1] - s[:, k]


# ----------------------------------------------------------------------------
# Routing statistics: the planner's online inputs
# ----------------------------------------------------------------------------

def route_stats(x, ids, gates, E):
    """Per-expert routing mass and routing-weighted input norm, float64.

    The page's planner ("内存的饥饿游戏…", zhichai.net, section "三层感知：离线 +
    路由 + 提示词") weighs a live count of how much routing each expert gets
    (to protect the busy ones) and a prompt-dependent correction taken from
    routing-weighted input norms.  Read plainly:
        mass[e]  = sum over slots (t, j) routed to e of gates[t, j]
        wnorm[e] = sum over the same slots of gates[t, j] * ||x_t||_2
    """
    xs = np.asarray(x, dtype=F64)
    ids = np.asarray(ids)
    g = np.asarray(gates, dtype=F64)
    T, k = ids.shape
    norms = [math.sqrt(sum(float(v) * float(v) for v in xs[t])) for t in range(T)]
    mass = np.zeros(E, dtype=F64)
    wnorm = np.zeros(E, dtype=F64)
    for t in range(T):
        for j in range(k):
            e = int(ids[t, j])
            mass[e] += g[t, j]
            wnorm[e] += g[t, j] * norms[t]
    return mass, wnorm


# ----------------------------------------------------------------------------
# Grouping token slots by expert
# ----------------------------------------------------------------------------

def group(ids: np.ndarray, E: int):
    """Slot s = t*k + j.  counts[e] = slots routed to e; offsets = exclusive
    prefix sum (length E+1); sorted_slots lists slots by (expert, slot);
    pos_of_slot is its inverse."""
    flat = [int(v) for v in np.asarray(ids).reshape(-1)]
    counts = np.zeros(E, dtype=np.int64)
    for e in flat:
        counts[e] += 1
    offsets = np.zeros(E + 1, dtype=np.int64)
    for e in range(E):
        offsets[e + 1] = offsets[e] + counts[e]
    sorted_slots = np.array(sorted(range(len(flat)), key=lambda s: (flat[s], s)), dtype=np.int64)
    pos_of_slot = np.empty(len(flat), dtype=np.int64)
    for p, s in enumerate(sorted_slots):
        pos_of_slot[s] = p
    return counts, offsets, sorted_slots, pos_of_slot


# ----------------------------------------------------------------------------
# Expert FFN (SwiGLU) and combine
# ----------------------------------------------------------------------------

def silu(z: np.ndarray) -> np.ndarray:
    """z * sigmoid(z), evaluated without overflow for large |z|."""
    z = np.asarray(z, dtype=F64)
    out = np.empty_like(z)
    pos = z >= 0
    out[pos] = z[pos] / (1.0 + np.exp(-z[pos]))
    ez = np.exp(z[~pos])
    out[~pos] = z[~pos] * ez / (1.0 + ez)
    return out


def silu_grad(z: np.ndarray) -> np.ndarray:
    z = np.asarray(z, dtype=F64)
    s = np.empty_like(z)
    pos = z >= 0
    s[pos] = 1.0 / (1.0 + np.exp(-z[pos]))
    ez = np.exp(z[~pos])
    s[~pos] = ez / (1.0 + ez)
    return s * (1.0 + z * (1.0 - s))


def gate_up(Wg: np.ndarray, Wu: np.ndarray, X: np.ndarray):
    """g = Wg x, u = Wu x, a = silu(g) * u for every row of X (float64)."""
    X = X.astype(F64)
    G = X @ Wg.T
    U = X @ Wu.T
    return G, U, silu(G) * U


def down(Wd: np.ndarray, A: np.ndarray) -> np.ndarray:
    return A.astype(F64) @ Wd.T


def gate_up_bound(Wg, Wu, X, G, U, rel=2e-3, abs_=1e-5):
    """Per-element tolerance of a = silu(g) u from the error propagated out of
    |g - g*| <= rel * sum|Wg||x| and the same for u."""
    Xa = np.abs(X.astype(F64))
    mg = Xa @ np.abs(Wg).T
    mu = Xa @ np.abs(Wu).T
    return rel * (np.abs(silu_grad(G)) * np.abs(U) * mg + np.abs(silu(G)) * mu) + abs_


def down_mag(Wd, A) -> np.ndarray:
    """sum_c |Wd[h, c]| |a[c]| for every row of A."""
    return np.abs(A.astype(F64)) @ np.abs(Wd).T


# ----------------------------------------------------------------------------
# Whole layer
# ----------------------------------------------------------------------------

def layer(inp, bits=None, tokens=None):
    """Run the whole layer on ``inp`` (a ``synth.LayerInputs``) in float64.

    ``bits``   per-expert bitwidths (defaults to ``inp.bits``).
    ``tokens`` optional subset of token indices whose outputs are wanted; the
               routing and grouping are still computed for every token, the
               expert FFN only for slots of the chosen tokens.

    Returns a dict with ids, gates, logits, counts, offsets, sorted_slots,
    pos_of_slot, A (sorted order, rows of chosen tokens only, others NaN),
    Y (same), y_shared, out [T, H] (rows of chosen tokens) and mag, the
    per-element magnitude sum_j gate * sum_c |W_down||a| (+ shared) used by
    the tolerance |out - out_ref| <= 2e-3 * mag + 1e-5.
    """
    cfg = inp.cfg
    bits = np.asarray(inp.bits if bits is None else bits).astype(int)
    T, E, H, I, k = cfg.T, cfg.E, cfg.H, cfg.I, cfg.k
    tok = np.arange(T) if tokens is None else np.asarray(sorted(set(int(t) for t in tokens)))
    want = np.zeros(T, dtype=bool)
    want[tok] = True

    ids, gates, L = route(inp.x, inp.w_router, inp.bias, cfg.logit_scale, k)
    counts, offsets, sorted_slots, pos_of_slot = group(ids, E)

    S = T * k
    A = np.full((S, I), np.nan)
    Y = np.full((S, H), np.nan)
    Ymag = np.full((S, H), np.nan)
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        pos = np.arange(lo, hi)
        slots = sorted_slots[lo:hi]
        keep = want[slots // k]
        if not keep.any():
            continue
        pos, slots = pos[keep], slots[keep]
        b = int(bits[e])
        Wg = dequant(inp.experts[e]["gate"], b)
        Wu = dequant(inp.experts[e]["up"], b)
        Wd = dequant(inp.experts[e]["down"], b)
        X = inp.x[slots // k]
        _, _, Ae = gate_up(Wg, Wu, X)
        A[pos] = Ae
        Y[pos] = down(Wd, Ae)
        Ymag[pos] = down_mag(Wd, Ae)

    y_sh = None
    sh_mag = None
    if inp.shared is not None:
        Wg = dequant(inp.shared["gate"], 16)
        Wu = dequant(inp.shared["up"], 16)
        Wd = dequant(inp.shared["down"], 16)
        y_sh = np.full((T, H), np.nan)
        sh_mag = np.full((T, H), np.nan)
        _, _, As = gate_up(Wg, Wu, inp.x[tok])
        y_sh[tok] = down(Wd, As)
        sh_mag[tok] = down_mag(Wd, As)

    out = np.full((T, H), np.nan)
    mag = np.full((T, H), np.nan)
    for t in tok:
        acc = np.zeros(H)
        m = np.zeros(H)
        for j in range(k):
            p = pos_of_slot[t * k + j]
            acc += gates[t, j] * Y[p]
            m += gates[t, j] * Ymag[p]
        if y_sh is not None:
            acc += y_sh[t]
            m += sh_mag[t]
        out[t] = acc
        mag[t] = m
    return dict(ids=ids, gates=gates, logits=L, counts=counts, offsets=offsets,
                sorted_slots=sorted_slots, pos_of_slot=pos_of_slot, A=A, Y=Y,
                y_shared=y_sh, out=out, mag=mag, tokens=tok)


def expert_gate_up_sorted(inp, bits, offsets, sorted_slots, e):
    """Oracle A rows of expert e (sorted order) and their tolerance, given a
    grouping (used to test the gate/up kernel on its own)."""
    k = inp.cfg.k
    lo, hi = int(offsets[e]), int(offsets[e + 1])
    slots = np.asarray(sorted_slots[lo:hi])
    b = int(bits[e])
    Wg = dequant(inp.experts[e]["gate"], b)
    Wu = dequant(inp.experts[e]["up"], b)
    X = inp.x[slots // k]
    G, U, A = gate_up(Wg, Wu, X)
    return A, gate_up_bound(Wg, Wu, X, G, U)


def expert_down_sorted(inp, bits, offsets, A_in, e, rel=2e-3, abs_=1e-5):
    """Oracle Y rows of expert e from a given A (e.g. the GPU's) and tolerance."""
    lo, hi = int(offsets[e]), int(offsets[e + 1])
    b = int(bits[e])
    Wd = dequant(inp.experts[e]["down"], b)
    Ae = np.asarray(A_in[lo:hi], dtype=F64)
    return down(Wd, Ae), rel * down_mag(Wd, Ae) + abs_
