"""Pins of the CPU oracle against facts that do not come from the oracle itself.

* hand-derived bit-plane words (tests/golden/bitplane_layout.json);
* the nesting of bitwidths: the b-bit code is the 6-bit code shifted right
  by 6 - b (one weight set serves every bitwidth, zhichai.net page, section
  "核心洞察：权重也能分页");
* a bit-serial closed form for affine lookup tables;
* brute force with scalar Python loops on micro inputs;
* the fp16 fallback against a direct matmul;
* special cases (k = 1, E = 1, softmax identities, tie-breaking).
"""
import itertools
import json
import math
import os

import numpy as np
import pytest

import synth
from oracle import moe
from synth.gen import MatrixData

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "bitplane_layout.json")


def _fixture_planes(case):
    hexes = case["planes_hex"]
    return np.array([[[int(h, 16) for h in row] for row in plane] for plane in hexes], dtype=np.uint32)


def _fixture_codes(case):
    if "codes" in case:
        return np.array(case["codes"], dtype=np.uint8)
    codes = np.zeros((case["rows"], case["cols"]), dtype=np.uint8)
    for c, v in case["nonzero"].items():
        codes[0, int(c)] = v
    return codes


# ---------------------------------------------------------------------------
# Format
# ---------------------------------------------------------------------------

def test_golden_plane_layout_decode():
    cases = json.load(open(GOLDEN))["cases"]
    for case in cases:
        planes = _fixture_planes(case)
        codes = _fixture_codes(case)
        assert np.array_equal(moe.decode_codes(planes, 6), codes.astype(np.int64)), case["name"]


def test_golden_plane_layout_pack():
    for case in json.load(open(GOLDEN))["cases"]:
        assert np.array_equal(synth.pack_planes(_fixture_codes(case)), _fixture_planes(case)), case["name"]


def test_golden_code_b():
    case = [c for c in json.load(open(GOLDEN))["cases"] if c["name"] == "sparse"][0]
    planes = _fixture_planes(case)
    for b in (3, 4, 5, 6):
        code = moe.decode_codes(planes, b)
        assert code[0, 5] == case["code_b_at_5"][str(b)]
        assert code[0, 37] == case["code_b_at_37"][str(b)]


@pytest.mark.parametrize("rows,cols", [(3, 32), (17, 96), (64, 256)])
def test_roundtrip_and_nesting(rows, cols):
    rng = np.random.default_rng(rows * 1000 + cols)
    code6 = rng.integers(0, 64, size=(rows, cols), dtype=np.uint8)
    planes = synth.pack_planes(code6)
    assert planes.shape == (6, rows, cols // 32)
    assert np.array_equal(moe.decode_codes(planes, 6), code6.astype(np.int64))
    for b in (3, 4, 5, 6):
        assert np.array_equal(moe.decode_codes(planes, b), (code6 >> (6 - b)).astype(np.int64))


def _bits_by_unpack(planes, p):
    """Independent bit extraction: bytes of the little-endian words, unpacked LSB first."""
    words = np.ascontiguousarray(planes[p]).astype("<u4")
    by = words.view(np.uint8).reshape(words.shape[0], -1)
    return np.unpackbits(by, axis=1, bitorder="little").astype(np.float64)


@pytest.mark.parametrize("b", [3, 4, 5, 6])
def test_bitserial_closed_form(b):
    """With an affine table lut[n][v] = alpha_n v + beta_n the LUT GEMV equals
    alpha_n * sum_p 2^(b-1-p) (plane_p . x) + beta_n * sum(x)."""
    rng = np.random.default_rng(7 + b)
    rows, cols = 24, 160
    code6 = rng.integers(0, 64, size=(rows, cols), dtype=np.uint8)
    planes = synth.pack_planes(code6)
    alpha = rng.normal(size=rows)
    beta = rng.normal(size=rows)
    luts = []
    for bb in (3, 4, 5, 6):
        v = np.arange(1 << bb, dtype=np.float64)
        luts.append(alpha[:, None] * v[None, :] + beta[:, None])
    mat = MatrixData(rows, cols, planes, luts)
    x = rng.normal(size=cols)
    y = moe.dequant(mat, b) @ x
    y_bs = np.zeros(rows)
    for p in range(b):
        y_bs += (2.0 ** (b - 1 - p)) * (_bits_by_unpack(planes, p) @ x)
    y_bs = alpha * y_bs + beta * x.sum()
    np.testing.assert_allclose(y, y_bs, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------------------
# Brute force on micro inputs
# ---------------------------------------------------------------------------

def _scalar_weight(mat, b, n, c):
    if b == 16:
        return float(mat.w16[n, c])
    word_idx, bit = divmod(c, 32)
    code = 0
    for p in range(b):
        code = code * 2 + ((int(mat.planes[p, n, word_idx]) >> bit) & 1)
    return float(mat.luts[b - 3][n, code])


def _scalar_silu(z):
    return z / (1.0 + math.exp(-z)) if z >= 0 else z * math.exp(z) / (1.0 + math.exp(z))


def _brute_layer(inp, bits):
    cfg = inp.cfg
    T, E, H, I, k = cfg.T, cfg.E, cfg.H, cfg.I, cfg.k
    x = inp.x.astype(np.float64)
    W = [{m: [[_scalar_weight(inp.experts[e][m], int(bits[e]), n, c)
                for c in range(inp.experts[e][m].cols)]
               for n in range(inp.experts[e][m].rows)] for m in ("gate", "up", "down")}
         for e in range(E)]
    out = np.zeros((T, H))
    for t in range(T):
        logits = []
        for e in range(E):
            s = 0.0
            for h in range(H):
                s += float(x[t, h]) * float(inp.w_router[e, h])
            if inp.bias is not None:
                s += float(inp.bias[e])
            logits.append(cfg.logit_scale * s)
        # top-k by enumerating every k-subset: the chosen set maximises the logit
        # sum; among equal sums the lexicographically smallest index set wins.
        best = None
        for sub in itertools.combinations(range(E), k):
            tot = sum(logits[e] for e in sub)
            if best is None or tot > best[0]:
                best = (tot, sub)
        sub = best[1]
        mx = max(logits[e] for e in sub)
        z = {e: math.exp(logits[e] - mx) for e in sub}
        zs = sum(z.values())
        for e in range(E):
            gate = z[e] / zs if e in sub else 0.0       # one-hot mask, no grouping
            a = []
            for n in range(I):
                g = sum(W[e]["gate"][n][h] * x[t, h] for h in range(H))
                u = sum(W[e]["up"][n][h] * x[t, h] for h in range(H))
                a.append(_scalar_silu(g) * u)
            for h in range(H):
                out[t, h] += gate * sum(W[e]["down"][h][n] * a[n] for n in range(I))
    return out


@pytest.mark.parametrize("k", [1, 2])
def test_brute_force_micro(k):
    cfg = synth.custom("micro", E=4, H=64, I=64, k=k, T=4, bits=(3, 4, 6, 16))
    inp = synth.make_inputs(cfg, seed=3)
    ref = moe.layer(inp)
    bf = _brute_layer(inp, inp.bits)
    np.testing.assert_allclose(ref["out"], bf, rtol=1e-11, atol=1e-13)


def test_brute_force_micro_bias_scale():
    cfg = synth.custom("micro_b", E=5, H=32, I=32, k=3, T=3, bits=(5, 3, 16, 6, 4), logit_scale=4.0)
    inp = synth.make_inputs(cfg, seed=11)
    inp.bias = np.linspace(-1, 1, 5).astype(np.float32)
    ref = moe.layer(inp)
    np.testing.assert_allclose(ref["out"], _brute_layer(inp, inp.bits), rtol=1e-11, atol=1e-13)


# ---------------------------------------------------------------------------
# fp16 fallback
# ---------------------------------------------------------------------------

def test_fp16_fallback_direct_matmul():
    import torch
    rng = np.random.default_rng(5)
    rows, cols = 48, 128
    w16 = rng.normal(0, 0.02, size=(rows, cols)).astype(np.float16)
    mat = MatrixData(rows, cols, np.zeros((6, 0, 0), np.uint32), [], w16)
    x = rng.normal(size=(7, cols)).astype(np.float16)
    y = x.astype(np.float64) @ moe.dequant(mat, 16).T
    np.testing.assert_allclose(y, x.astype(np.float64) @ w16.astype(np.float64).T, rtol=1e-12)
    yt = torch.matmul(torch.from_numpy(x.astype(np.float32)), torch.from_numpy(w16.astype(np.float32)).T)
    bound = 1e-5 * (np.abs(x.astype(np.float64)) @ np.abs(w16.astype(np.float64)).T) + 1e-7
    assert np.all(np.abs(yt.numpy() - y) <= bound)


# ---------------------------------------------------------------------------
# Special cases and invariants
# ---------------------------------------------------------------------------

def test_k1_is_dense_ffn_of_chosen_expert():
    cfg = synth.custom("k1", E=3, H=64, I=96, k=1, T=5, bits=(4, 6, 16))
    inp = synth.make_inputs(cfg, seed=2)
    ref = moe.layer(inp)
    assert np.allclose(ref["gates"], 1.0)
    for t in range(cfg.T):
        e = int(ref["ids"][t, 0])
        b = int(inp.bits[e])
        Wg = moe.dequant(inp.experts[e]["gate"], b)
        Wu = moe.dequant(inp.experts[e]["up"], b)
        Wd = moe.dequant(inp.experts[e]["down"], b)
        xt = inp.x[t].astype(np.float64)
        g, u = Wg @ xt, Wu @ xt
        y = Wd @ (g / (1 + np.exp(-g)) * u)
        np.testing.assert_allclose(ref["out"][t], y, rtol=1e-12, atol=1e-14)


def test_single_expert_is_dense_layer():
    cfg = synth.custom("e1", E=1, H=32, I=64, k=1, T=4, bits=(5,))
    inp = synth.make_inputs(cfg, seed=9)
    ref = moe.layer(inp)
    Wg = moe.dequant(inp.experts[0]["gate"], 5)
    Wu = moe.dequant(inp.experts[0]["up"], 5)
    Wd = moe.dequant(inp.experts[0]["down"], 5)
    X = inp.x.astype(np.float64)
    G, U = X @ Wg.T, X @ Wu.T
    Y = (G / (1 + np.exp(-G)) * U) @ Wd.T
    np.testing.assert_allclose(ref["out"], Y, rtol=1e-12, atol=1e-14)


def test_router_softmax_identities():
    rng = np.random.default_rng(1)
    x = rng.normal(size=(50, 64)).astype(np.float16)
    w = rng.normal(0, 0.05, size=(12, 64)).astype(np.float32)
    ids, gates, L = moe.route(x, w, None, 1.0, 4)
    np.testing.assert_allclose(gates.sum(axis=1), 1.0, rtol=0, atol=1e-15)
    full = np.exp(L - L.max(axis=1, keepdims=True))
    full /= full.sum(axis=1, keepdims=True)
    sel = np.take_along_axis(full, ids, axis=1)
    np.testing.assert_allclose(gates, sel / sel.sum(axis=1, keepdims=True), rtol=1e-12)
    # descending logits, the k-th above every unselected logit
    sl = np.take_along_axis(L, ids, axis=1)
    assert np.all(np.diff(sl, axis=1) <= 0)
    for t in range(50):
        rest = np.delete(L[t], ids[t])
        assert sl[t, -1] >= rest.max()


def test_router_ties_go_to_lower_index():
    x = np.ones((2, 32), dtype=np.float16)
    w = np.zeros((6, 32), dtype=np.float32)
    w[1] = w[4] = 0.5
    w[2] = w[5] = 0.25
    ids, gates, _ = moe.route(x, w, None, 1.0, 3)
    assert ids.tolist() == [[1, 4, 2], [1, 4, 2]]
    np.testing.assert_allclose(gates[:, 0], gates[:, 1])


def test_route_stats_hand_example():
    # three tokens, rows of four ones (norm 2), k = 2 over four experts:
    # expert 0 gets 0.7 + 0.1, expert 1 0.3 + 0.5, expert 2 0.5 + 0.9, expert 3 nothing
    x = np.ones((3, 4), dtype=np.float16)
    ids = np.array([[0, 1], [1, 2], [0, 2]])
    gates = np.array([[0.7, 0.3], [0.5, 0.5], [0.1, 0.9]])
    mass, wnorm = moe.route_stats(x, ids, gates, 4)
    np.testing.assert_allclose(mass, [0.8, 0.8, 1.4, 0.0], rtol=0, atol=1e-15)
    np.testing.assert_allclose(wnorm, [1.6, 1.6, 2.8, 0.0], rtol=0, atol=1e-15)


def test_route_stats_invariants():
    rng = np.random.default_rng(11)
    T, H, E, k = 40, 64, 9, 3
    x = rng.normal(size=(T, H)).astype(np.float16)
    w = rng.normal(0, 0.05, size=(E, H)).astype(np.float32)
    ids, gates, _ = moe.route(x, w, None, 1.0, k)
    mass, wnorm = moe.route_stats(x, ids, gates, E)
    # every token's gates sum to one, so the masses sum to T
    assert abs(mass.sum() - T) < 1e-12
    # the same sums written as one-hot matrix products
    onehot = np.zeros((T, E))
    for j in range(k):
        onehot[np.arange(T), ids[:, j]] += gates[:, j]
    norms = np.linalg.norm(x.astype(np.float64), axis=1)
    np.testing.assert_allclose(mass, onehot.sum(axis=0), rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(wnorm, onehot.T @ norms, rtol=1e-13, atol=1e-15)
    # each expert's norm-weighted sum lies between its mass times the smallest
    # and the largest input norm; unrouted experts have exactly zero
    assert np.all(wnorm >= mass * norms.min() - 1e-12) and np.all(wnorm <= mass * norms.max() + 1e-12)
    unused = np.setdiff1d(np.arange(E), ids.reshape(-1))
    assert np.all(mass[unused] == 0) and np.all(wnorm[unused] == 0)


def test_grouping_invariants():
    rng = np.random.default_rng(4)
    E, T, k = 9, 37, 3
    ids = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)])
    counts, offsets, ss, pos = moe.group(ids, E)
    assert counts.sum() == T * k
    assert offsets[0] == 0 and offsets[-1] == T * k and np.all(np.diff(offsets) >= 0)
    flat = ids.reshape(-1)
    for e in range(E):
        seg = ss[offsets[e]:offsets[e + 1]]
        assert np.all(flat[seg] == e)
        assert np.all(np.diff(seg) > 0)            # stable: slot order inside an expert
    assert np.array_equal(ss[pos], np.arange(T * k))


def test_silu_textbook_and_extremes():
    z = np.linspace(-30, 30, 601)
    np.testing.assert_allclose(moe.silu(z), z / (1 + np.exp(-z)), rtol=1e-14, atol=1e-300)
    big = np.array([-1e4, -800.0, 800.0, 1e4])
    s = moe.silu(big)
    assert np.all(np.isfinite(s))
    np.testing.assert_allclose(s[2:], big[2:])
    assert np.all(s[:2] <= 0) and np.all(s[:2] > -1e-300)
    h = 1e-6
    for zz in (-3.0, -0.5, 0.0, 0.7, 4.0):
        num = (moe.silu(np.array([zz + h])) - moe.silu(np.array([zz - h]))) / (2 * h)
        np.testing.assert_allclose(moe.silu_grad(np.array([zz])), num, rtol=1e-7)


def test_layer_token_subset_matches_full():
    cfg = synth.custom("sub", E=6, H=64, I=64, k=2, T=9, bits=(3, 4, 5, 6, 16, 4))
    inp = synth.make_inputs(cfg, seed=21)
    full = moe.layer(inp)
    sub = moe.layer(inp, tokens=[0, 4, 8])
    for t in (0, 4, 8):
        # same arithmetic on fewer rows; only BLAS blocking may reorder sums
        np.testing.assert_allclose(sub["out"][t], full["out"][t], rtol=1e-12, atol=1e-16)
        np.testing.assert_allclose(sub["mag"][t], full["mag"][t], rtol=1e-12)
    assert np.isnan(sub["out"][1]).all()


def test_mag_bounds_output():
    cfg = synth.get("tiny")
    inp = synth.make_inputs(cfg, seed=0)
    ref = moe.layer(inp)
    assert np.all(np.abs(ref["out"]) <= ref["mag"] * (1 + 1e-12))


# ---------------------------------------------------------------------------
# Planted mistakes: each pin above must fail on a plausible oracle bug.
# ---------------------------------------------------------------------------

def test_pins_catch_planted_decode_mistakes(monkeypatch):
    cases = json.load(open(GOLDEN))["cases"]
    good = moe.decode_codes

    def lsb_first(planes, b):           # planes read in the wrong significance order
        code = None
        for p in range(b):
            term = moe.plane_bit(planes, p).astype(np.int64) << p
            code = term if code is None else code + term
        return code

    def low_planes(planes, b):          # b-bit code from the bottom b planes
        code = None
        for i, p in enumerate(range(6 - b, 6)):
            term = moe.plane_bit(planes, p).astype(np.int64) << (b - 1 - i)
            code = term if code is None else code + term
        return code

    for bad in (lsb_first, low_planes):
        monkeypatch.setattr(moe, "decode_codes", bad)
        caught = False
        for case in cases:
            planes, codes = _fixture_planes(case), _fixture_codes(case)
            for b in (3, 4, 5, 6):
                if not np.array_equal(moe.decode_codes(planes, b), (codes >> (6 - b)).astype(np.int64)):
                    caught = True
        assert caught, bad.__name__
    monkeypatch.setattr(moe, "decode_codes", good)


def test_pins_catch_planted_word_bit_order(monkeypatch):
    def msb_column_first(planes, p):    # bit 31 taken as the lowest column
        words = planes[p]
        rows, W = words.shape
        shifts = np.arange(31, -1, -1, dtype=np.uint32)
        bits = (words[:, :, None] >> shifts[None, None, :]) & np.uint32(1)
        return bits.reshape(rows, W * 32).astype(np.uint8)

    monkeypatch.setattr(moe, "plane_bit", msb_column_first)
    case = json.load(open(GOLDEN))["cases"][1]
    assert not np.array_equal(moe.decode_codes(_fixture_planes(case), 6), _fixture_codes(case).astype(np.int64))
