"""Pins of the exponent-codec oracle: the textbook Huffman example, the tie
rule, a lone symbol, a hand-assembled bit stream, the Kraft equality and the
entropy bound, the length limit on Fibonacci counts, and lossless round trips
(including a partial last group)."""
import numpy as np
import pytest

from oracle import expcodec as X


def test_textbook_example_lengths_and_canonical_codes():
    # counts 5, 2, 1, 1: c and d merge first, then b with that node, then a
    counts = np.zeros(256, np.int64)
    counts[[0, 1, 2, 3]] = [5, 2, 1, 1]
    L = X.huffman_lengths(counts)
    assert L[:4] == [1, 2, 3, 3] and sum(L[4:]) == 0
    assert X.canonical_codes(L) == {0: 0b0, 1: 0b10, 2: 0b110, 3: 0b111}


def test_tie_rule_equal_counts_and_lone_symbol():
    counts = np.zeros(256, np.int64)
    counts[[7, 9, 200, 201]] = 3
    assert [X.huffman_lengths(counts)[s] for s in (7, 9, 200, 201)] == [2, 2, 2, 2]
    assert X.canonical_codes(X.huffman_lengths(counts)) == {7: 0, 9: 1, 200: 2, 201: 3}
    one = np.zeros(256, np.int64)
    one[60] = 10
    assert X.huffman_lengths(one)[60] == 1 and sum(X.huffman_lengths(one)) == 1


def test_hand_assembled_stream():
    # 64 weights: one group of 64 blocks of one symbol each; high bytes 0x3C
    # (code 0) except weights 1, 31, 32 and 63 (0xBC, code 1); block l = weight l
    w = np.full(64, 0x3C00, np.uint16) | np.arange(64, dtype=np.uint16)
    for i in (1, 31, 32, 63):
        w[i] = 0xBC00 | i
    lengths, words, offs, lo = X.encode(w)
    assert lengths[0x3C] == 1 and lengths[0xBC] == 1 and sum(lengths) == 2
    assert offs.tolist() == list(range(64))
    assert words.tolist() == [(1 << 30) | 1, (1 << 31) | 1, 0, 0]
    assert lo.tolist() == list(range(64))
    assert np.array_equal(X.decode(lengths, words, offs, lo, 64), w)


def test_kraft_equality_and_entropy_bound():
    rng = np.random.default_rng(5)
    for _ in range(10):
        counts = np.zeros(256, np.int64)
        sym = rng.choice(256, size=rng.integers(2, 60), replace=False)
        counts[sym] = rng.integers(1, 5000, size=sym.size)
        L = X.huffman_lengths(counts)
        assert sum(2.0 ** -l for l in L if l) == pytest.approx(1.0, abs=1e-12)
        bits, H = X.coded_bits(L, counts), X.entropy_bits(counts)
        assert H - 1e-6 <= bits < H + counts.sum()


def test_length_limit_on_fibonacci_counts():
    fib = [1, 1]
    while len(fib) < 24:
        fib.append(fib[-1] + fib[-2])
    counts = np.zeros(256, np.int64)
    counts[:24] = fib
    assert max(X.huffman_lengths(counts)) == 23          # the textbook worst case
    L = X.limited_lengths(counts)
    assert max(L) <= 12 and all(L[s] > 0 for s in range(24))
    assert sum(2.0 ** -l for l in L if l) <= 1.0
    # a stream that uses every symbol still round-trips
    w = np.repeat(np.arange(24, dtype=np.uint16) << 8, 64 * 3)[: 64 * 70] | np.uint16(0x55)
    lengths, words, offs, lo = X.encode(w)
    assert max(lengths) <= 12
    assert np.array_equal(X.decode(lengths, words, offs, lo, w.size), w)


@pytest.mark.parametrize("n", [64, 64 * X.S, 64 * X.S + 64 * 37])
def test_round_trip_fp16_weights(n):
    rng = np.random.default_rng(n)
    w = rng.normal(0.0, 0.02, n).astype(np.float16).view(np.uint16)
    lengths, words, offs, lo = X.encode(w)
    assert offs.size == 64 * (-(-n // (64 * X.S)))
    assert np.array_equal(X.decode(lengths, words, offs, lo, n), w)
    if n >= 64 * X.S:
        # N(0, 0.02) weights: the high byte carries ~5.5 bits of information
        coded = X.coded_bits(lengths, X.histogram(w >> 8))
        assert coded / n < 6.5


# ---------------------------------------------------------------------------
# The library's host encoder against the oracle (bit-exact)
# ---------------------------------------------------------------------------

def _native_vs_oracle(w):
    from any_precision_quantized_amd import _lib
    got = _lib.exp_encode(w)
    lengths, words, offs, lo = X.encode(w)
    assert got["lengths"].tolist() == list(lengths)
    assert np.array_equal(got["words"], words)
    assert np.array_equal(got["block_off"], offs)
    assert np.array_equal(got["lo"], lo)
    # table entry p: the symbol whose canonical code prefixes the 12 bits p, and its length
    codes = X.canonical_codes(lengths)
    want = np.zeros(4096, np.uint16)
    for s, c in codes.items():
        L = lengths[s]
        want[c << (12 - L):(c + 1) << (12 - L)] = (L << 8) | s
    assert np.array_equal(got["table"], want)


@pytest.mark.parametrize("case", ["normal", "partial_group", "one_symbol", "fibonacci"])
def test_native_encoder_matches_oracle(case):
    rng = np.random.default_rng(11)
    if case == "normal":
        w = rng.normal(0.0, 0.02, 64 * X.S * 2).astype(np.float16).view(np.uint16)
    elif case == "partial_group":
        w = rng.normal(0.0, 1.0, 64 * X.S + 64 * 5).astype(np.float16).view(np.uint16)
    elif case == "one_symbol":
        w = (np.full(64 * 9, 0x3C00, np.uint16) | rng.integers(0, 256, 64 * 9).astype(np.uint16))
    else:
        fib = [1, 1]
        while len(fib) < 24:
            fib.append(fib[-1] + fib[-2])
        hi = np.repeat(np.arange(24), [max(1, f // 200) for f in fib])
        hi = np.resize(hi, 64 * 300)
        w = (hi.astype(np.uint16) << 8) | rng.integers(0, 256, hi.size).astype(np.uint16)
    _native_vs_oracle(w)


def test_native_encoder_argument_errors():
    import ctypes
    from any_precision_quantized_amd import _lib
    lib = _lib._lib()
    w = np.zeros(128, np.uint16)
    lengths = np.zeros(256, np.uint8)
    nw, nb = ctypes.c_uint64(), ctypes.c_uint64()
    assert lib.apmoe_exp_plan(w.ctypes.data, 100, lengths.ctypes.data, ctypes.byref(nw), ctypes.byref(nb)) == _lib.EINVAL
    assert lib.apmoe_exp_plan(None, 128, lengths.ctypes.data, ctypes.byref(nw), ctypes.byref(nb)) == _lib.EINVAL
    assert lib.apmoe_exp_plan(w.ctypes.data, 128, lengths.ctypes.data, ctypes.byref(nw), ctypes.byref(nb)) == _lib.OK
    assert (nw.value, nb.value) == (4 + 2, 64) and lengths[0] == 1   # one symbol: 128 one-bit codes
    words = np.zeros(nw.value, np.uint32)
    offs = np.zeros(nb.value, np.uint32)
    lo = np.zeros(128, np.uint8)
    table = np.zeros(4096, np.uint16)
    args = (offs.ctypes.data, lo.ctypes.data, table.ctypes.data)
    assert lib.apmoe_exp_encode(w.ctypes.data, 128, lengths.ctypes.data, words.ctypes.data, 3, *args) == _lib.ENOSPACE
    bad = lengths.copy()
    bad[0] = 0                                   # the only symbol has no code
    assert lib.apmoe_exp_encode(w.ctypes.data, 128, bad.ctypes.data, words.ctypes.data, nw.value, *args) == _lib.EINVAL
    assert lib.apmoe_exp_encode(w.ctypes.data, 128, lengths.ctypes.data, words.ctypes.data, nw.value, *args) == _lib.OK
    assert lib.apmoe_exp_decode(None, 6, None, None, None, 128, None, None) == _lib.EINVAL
    # batched decode: count out of range, missing arrays, one bad entry
    vp2 = (ctypes.c_void_p * 2)(0x1000, 0x2000)
    u2 = (ctypes.c_uint64 * 2)(6, 6)
    n2 = (ctypes.c_uint64 * 2)(128, 100)         # 100 is not a multiple of 64
    assert lib.apmoe_exp_decode_batch(0, vp2, u2, vp2, vp2, vp2, n2, vp2, None) == _lib.EINVAL
    assert lib.apmoe_exp_decode_batch(_lib.EXP_MAX_BATCH + 1, vp2, u2, vp2, vp2, vp2, n2, vp2, None) == _lib.EINVAL
    assert lib.apmoe_exp_decode_batch(2, None, u2, vp2, vp2, vp2, n2, vp2, None) == _lib.EINVAL
    assert lib.apmoe_exp_decode_batch(2, vp2, u2, vp2, vp2, vp2, n2, vp2, None) == _lib.EINVAL
