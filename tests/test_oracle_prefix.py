"""Pins of the oracle's comparison exponent codes (Cassandra review,
marsggbo.github.io, section 3.2: Huffman codes are slightly shorter than the
unary code but parse serially, bit by bit or through a 2^N-entry table).

  * length-limited Huffman (package-merge): on alphabets of up to 6 symbols
    its cost equals the minimum over every length vector that satisfies
    Kraft's inequality within the limit (brute force); without a binding
    limit its cost equals a textbook heap-built Huffman code's, and the mean
    length lies in [H, H + 1) (Shannon);
  * canonical code values are prefix-free and complete;
  * the encoder's bits, parsed by a numpy dictionary decoder, give back the
    symbols; block offsets are the prefix sums of the code lengths;
  * the unary code as a prefix code reproduces, bit for bit, the exponent
    code section of a Cassandra-1 speculation stream.
"""
import heapq
import itertools
import math

import numpy as np
import pytest

import synth
import streamparse as sp


def cost(hist, ln):
    return int(sum(int(hist[s]) * int(ln[s]) for s in range(256)))


def random_hist(rng, n, spread=8):
    h = np.zeros(256, dtype=np.uint64)
    syms = rng.choice(256, size=n, replace=False)
    h[syms] = (2.0 ** rng.uniform(0, spread, size=n)).astype(np.uint64) + 1
    return h


@pytest.mark.parametrize("seed", range(12))
def test_huffman_limited_bruteforce(orc, seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(2, 7))
    h = random_hist(rng, n)
    syms = np.flatnonzero(h)
    for L in range(max(1, math.ceil(math.log2(n))), 6):
        ln, code = orc.huffman_code(h, L)
        assert ln.max() <= L and sum(2.0 ** -int(ln[s]) for s in syms) <= 1.0
        assert np.all(ln[h == 0] == 0)
        best = min(sum(int(h[s]) * l for s, l in zip(syms, ls))
                   for ls in itertools.product(range(1, L + 1), repeat=n)
                   if sum(2.0 ** -l for l in ls) <= 1.0)
        assert cost(h, ln) == best, (n, L)


def textbook_huffman_cost(weights):
    heap = [int(w) for w in weights]
    heapq.heapify(heap)
    total = 0
    while len(heap) > 1:
        a, b = heapq.heappop(heap), heapq.heappop(heap)
        total += a + b
        heapq.heappush(heap, a + b)
    return total


@pytest.mark.parametrize("seed", range(8))
def test_huffman_unlimited_matches_textbook_and_shannon(orc, seed):
    rng = np.random.default_rng(100 + seed)
    h = random_hist(rng, int(rng.integers(2, 60)), spread=16)
    ln, code = orc.huffman_code(h, 32)
    syms = np.flatnonzero(h)
    assert cost(h, ln) == textbook_huffman_cost(h[syms])
    p = h[syms].astype(np.float64) / h.sum()
    H = float(-(p * np.log2(p)).sum())
    mean = cost(h, ln) / float(h.sum())
    assert H - 1e-12 <= mean < H + 1
    # canonical codes: complete and prefix-free
    assert abs(sum(2.0 ** -int(ln[s]) for s in syms) - 1.0) < 1e-12
    for a in syms:
        for b in syms:
            if a == b or ln[a] > ln[b]:
                continue
            assert (int(code[b]) >> int(ln[b] - ln[a])) != int(code[a]), (a, b)


def test_single_symbol_and_empty(orc):
    h = np.zeros(256, dtype=np.uint64)
    ln, _ = orc.huffman_code(h, 12)
    assert not ln.any()
    h[7] = 5
    ln, code = orc.huffman_code(h, 12)
    assert ln[7] == 1 and ln.sum() == 1 and code[7] == 0


def numpy_parse(stream, n, ln, code):
    table = {(int(ln[s]), int(code[s])): s for s in range(256) if ln[s]}
    bits = sp.bits_of(stream)
    out, pos = [], 0
    for _ in range(n):
        c, l = 0, 0
        while True:
            c = (c << 1) | int(bits[pos])
            pos += 1
            l += 1
            if (l, c) in table:
                out.append(table[(l, c)])
                break
            assert l < 40
    return np.array(out, dtype=np.uint8), pos


@pytest.mark.parametrize("kind", ["huffman12", "huffman32", "unary"])
def test_prefix_stream_roundtrip(orc, kind):
    w = synth.weight(64, 1024, 21, outlier_frac=0.01)
    keep = orc.select(w, 307)
    sym = ((w[keep] >> 7) & 0xFF).astype(np.uint8)
    hist = np.bincount(sym, minlength=256).astype(np.uint64)
    if kind == "unary":
        ln, code = orc.unary_code(hist)
    else:
        ln, code = orc.huffman_code(hist, 12 if kind == "huffman12" else 32)
    stream, blkoff, bits = orc.prefix_encode(sym, 256, ln, code)
    lens = ln[sym].astype(np.int64)
    assert bits == int(lens.sum())
    starts = np.concatenate([[0], np.cumsum(lens)[:-1]])
    assert np.array_equal(blkoff, starts[::256])
    got, end = numpy_parse(stream, sym.size, ln, code)
    assert np.array_equal(got, sym) and end == bits
    assert np.array_equal(orc.prefix_decode(stream, sym.size, ln, code), sym)
    assert not sp.bits_of(stream)[bits:].any(), "pad bits are zero"


def test_unary_prefix_code_is_cassandra1_code_section(orc):
    w = synth.weight(40, 1024, 33, outlier_frac=0.01)
    k = 307
    spec, _ = orc.encode(w, k, 3, fmt=1)
    keep = orc.select(w, k)
    sym = ((w[keep] >> 7) & 0xFF).astype(np.uint8)  # kept exponents, row-major
    hist = np.bincount(sym, minlength=256).astype(np.uint64)
    ln, code = orc.unary_code(hist)
    stream, _, bits = orc.prefix_encode(sym, 1024, ln, code)
    h = sp.parse_header(spec)
    sec = sp.section(spec, h, 6)
    assert h["secs"][6][1] == (bits + 7) // 8
    assert np.array_equal(stream[:sec.size], sec)
