"""Oracle of the lossless exponent codec for fp16 weights.

Test infrastructure only: the tests, the smoke entry point and the CPU leg of
the benchmark use it; the library never does.

A page on expert paging describes a lossless compression tier for expert
weights: the exponent bits of the floating-point weights are Huffman-coded
offline and decoded in GPU memory, in parallel with transfers from host
memory ("专家分页机制：7倍MoE推理吞吐背后的显存解耦革命", mubeitech.com, the
passage on its third mechanism, bandwidth-balanced storage tiering).
Readings taken here (the page gives no format):
  * a weight is fp16; its high byte (sign, the five exponent bits, the top two
    mantissa bits) is the coded symbol, its low byte is stored raw.  The sign
    and mantissa bits are close to uniform, so the code spends about their
    raw three bits on them and compresses what the exponent leaves;
  * the code is a Huffman code over the high bytes of one matrix, built with
    a fixed tie rule (a node's key is (weight, id); leaves have id = symbol,
    merged nodes ids 256, 257, ... in creation order; the two smallest keys
    merge first); a lone symbol gets length 1;
  * code lengths are limited to 12 bits: while the longest code exceeds 12,
    every non-zero count is raised to at least total >> (12 - r) for
    r = 2, 3, ... (the first r that makes the code fit) and the code is
    rebuilt.  Codes are canonical: by (length, symbol), consecutive values;
  * layout: weights are taken in groups of 64 * S (S = 144); block (g, l),
    l = 0..63, holds the weights g*64*S + 64*j + l for j = 0..S_g - 1, with
    S_g = min(S, (n - g*64*S) / 64) (n a multiple of 64).  The bit stream is
    the blocks' codes in block order, each block's codes in j order, most
    significant bit first inside 32-bit words; block_off[g*64 + l] is the bit
    where block (g, l) starts; two zero words end the stream;
  * lo[w] = low byte of weight w, in weight order.
"""
from __future__ import annotations

import heapq

import numpy as np

NSYM = 256
LMAX = 12
S = 144          # symbols per block
LANES = 64       # blocks per group


def histogram(hi):
    return np.bincount(np.asarray(hi, dtype=np.int64), minlength=NSYM).astype(np.int64)


def huffman_lengths(counts):
    """Code length per symbol (0 for absent symbols), tie rule as above."""
    counts = [int(c) for c in counts]
    live = [s for s in range(len(counts)) if counts[s] > 0]
    lengths = [0] * len(counts)
    if not live:
        return lengths
    if len(live) == 1:
        lengths[live[0]] = 1
        return lengths
    heap = [(counts[s], s) for s in live]
    heapq.heapify(heap)
    parent = {}
    nxt = NSYM
    while len(heap) > 1:
        w1, a = heapq.heappop(heap)
        w2, b = heapq.heappop(heap)
        parent[a] = nxt
        parent[b] = nxt
        heapq.heappush(heap, (w1 + w2, nxt))
        nxt += 1
    for s in live:
        d, node = 0, s
        while node in parent:
            node = parent[node]
            d += 1
        lengths[s] = d
    return lengths


def limited_lengths(counts, lmax=LMAX):
    """Huffman lengths, with counts raised as described until they fit lmax."""
    counts = np.asarray(counts, dtype=np.int64)
    lengths = huffman_lengths(counts)
    total = int(counts.sum())
    r = 2
    while max(lengths) > lmax:
        floor = max(1, total >> (lmax - r))
        raised = np.where(counts > 0, np.maximum(counts, floor), 0)
        lengths = huffman_lengths(raised)
        r += 1
    return lengths


def canonical_codes(lengths):
    """code[s] for every symbol with a length: by (length, symbol), consecutive."""
    order = sorted((L, s) for s, L in enumerate(lengths) if L > 0)
    codes = {}
    code, prev = 0, 0
    for L, s in order:
        code <<= (L - prev)
        codes[s] = code
        code += 1
        prev = L
    return codes


def block_weights(n, g, l):
    """Weight indices of block (g, l) in code order."""
    sg = min(S, (n - g * LANES * S) // LANES)
    return [g * LANES * S + LANES * j + l for j in range(sg)]


def encode(w16):
    """w16: uint16 array of n fp16 bit patterns (n % 64 == 0).  Returns
    (lengths[256], words uint32[], block_off uint32[], lo uint8[n])."""
    w = np.asarray(w16, dtype=np.uint16).reshape(-1)
    n = w.size
    assert n % LANES == 0
    hi = (w >> 8).astype(np.int64)
    lo = (w & 0xFF).astype(np.uint8)
    lengths = limited_lengths(histogram(hi))
    codes = canonical_codes(lengths)
    ngroups = -(-n // (LANES * S))
    bits = []
    offs = []
    for g in range(ngroups):
        for l in range(LANES):
            offs.append(len(bits))
            for idx in block_weights(n, g, l):
                s = int(hi[idx])
                L = lengths[s]
                c = codes[s]
                bits.extend((c >> (L - 1 - i)) & 1 for i in range(L))
    nwords = -(-len(bits) // 32) + 2
    words = np.zeros(nwords, dtype=np.uint32)
    for k, b in enumerate(bits):
        if b:
            words[k >> 5] |= np.uint32(1 << (31 - (k & 31)))
    return lengths, words, np.asarray(offs, dtype=np.uint32), lo


def decode(lengths, words, block_off, lo, n):
    """Walk the bit stream code by code (prefix matching), rebuild the weights."""
    codes = canonical_codes(lengths)
    by_code = {(lengths[s], c): s for s, c in codes.items()}
    words = np.asarray(words, dtype=np.uint32)
    out = np.zeros(n, dtype=np.uint16)
    ngroups = -(-n // (LANES * S))
    for g in range(ngroups):
        for l in range(LANES):
            k = int(block_off[g * LANES + l])
            for idx in block_weights(n, g, l):
                c, L = 0, 0
                while True:
                    c = (c << 1) | int((int(words[k >> 5]) >> (31 - (k & 31))) & 1)
                    k += 1
                    L += 1
                    if (L, c) in by_code:
                        break
                    if L > LMAX:
                        raise ValueError("not a code of this table")
                out[idx] = (by_code[(L, c)] << 8) | int(lo[idx])
    return out


def coded_bits(lengths, counts):
    return int(sum(int(L) * int(c) for L, c in zip(lengths, counts)))


def entropy_bits(counts):
    c = np.asarray(counts, dtype=np.float64)
    p = c[c > 0] / c.sum()
    return float(-(p * np.log2(p)).sum() * c.sum())
