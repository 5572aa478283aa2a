"""Pins of the CPU oracle against what the pages and mathematics fix.

None of these compare the oracle with itself: each check is brute force on a
tiny input, a closed form, an invariant stated by the pages, or a special case
that reduces to a textbook computation.  Sources (page title, section):
  * Cassandra review, marsggbo.github.io, section 3.1 -- pruning by saliency,
    mantissa truncation, speculation/verification split, zero-filled draft,
    lossless reassembly;
  * same page, section 3.2 -- unary exponent code (count zeros up to the one),
    frequent exponents get short codes; MX shared exponent for Cassandra-2;
  * OCP MX specification (cited by the paper) -- 32-element blocks, one shared
    8-bit exponent;
  * Shannon's source coding theorem (cited by the paper) -- entropy is a lower
    bound on the mean code length.
"""
import itertools
import math
from fractions import Fraction

import numpy as np
import pytest

import synth
import streamparse as sp

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def key(b):
    return np.asarray(b, dtype=np.int64) & 0x7FFF


def exact(b):
    """bf16 pattern -> exact Fraction (finite values only)."""
    f = float(synth.f32_from_bf16(np.array([b], dtype=np.uint16))[0])
    return Fraction(f)


def semantic_draft_c1(w, keep_mask, m):
    """Draft by the pages' rule written on the original bits: kept values lose
    their low 7-m mantissa bits, pruned values become +0."""
    low = (1 << (7 - m)) - 1
    return np.where(keep_mask, w & ~np.uint16(low), np.uint16(0)).astype(np.uint16)


# ---------------------------------------------------------------- pruning


def brute_select_row(row, k):
    """Among all k-subsets choose the one with the largest magnitudes (sorted
    descending, compared lexicographically); ties -> lexicographically smallest
    column set."""
    best, best_key = None, None
    keys = key(row)
    for S in itertools.combinations(range(len(row)), k):
        kk = tuple(sorted((int(keys[j]) for j in S), reverse=True))
        cand = (kk, tuple(-j for j in S))
        if best_key is None or cand > best_key:
            best, best_key = S, cand
    out = np.zeros(len(row), dtype=bool)
    out[list(best)] = True
    return out


@pytest.mark.parametrize("seed", range(6))
def test_select_bruteforce_8x8(orc, seed):
    rng = np.random.default_rng(seed)
    w = synth.bf16_from_f32(rng.standard_normal((8, 8)).astype(np.float32))
    if seed % 2:  # force ties: repeated magnitudes with both signs
        w[:, 4] = w[:, 1] ^ 0x8000
        w[:, 6] = w[:, 1]
        w[:, 7] = w[:, 0]
    for k in range(9):
        got = orc.select(w, k)
        want = np.stack([brute_select_row(w[r], k) for r in range(8)])
        assert (got == want).all(), (seed, k)


def test_select_invariants(orc):
    w = synth.weight(64, 1024, 11, outlier_frac=0.01)
    w[:, 100:140] = w[:, 0:40]  # many ties
    for k in (0, 1, 307, 512, 1023, 1024):
        keep = orc.select(w, k)
        assert (keep.sum(axis=1) == k).all()
        for r in range(0, 64, 7):
            kk, kp = key(w[r][keep[r]]), key(w[r][~keep[r]])
            if k and k < 1024:
                thr = kk.min()
                assert thr >= kp.max()
                # among values equal to the threshold, the kept ones come first
                eq = np.flatnonzero(key(w[r]) == thr)
                kept_eq = keep[r][eq]
                assert (np.sort(kept_eq)[::-1] == kept_eq).all()


# --------------------------------------------------------- exponent stats


def test_exponent_histogram_gaussian_closed_form(orc):
    """bf16(N(0, s^2)) has exponent e with probability 2[Phi(u/s) - Phi(l/s)],
    l = 2^(e-127)(1-2^-9), u = 2^(e-126)(1-2^-9) (round-to-nearest-even edges)."""
    sigma = 0.02
    w = synth.weight(1024, 1024, 1_000_000, sigma=sigma)
    hk, hp = orc.histograms(w, np.ones(w.shape, dtype=bool))
    assert hp.sum() == 0
    n = w.size
    Phi = lambda z: 0.5 * (1 + math.erf(z / math.sqrt(2)))
    for e in range(100, 140):
        lo = 2.0 ** (e - 127) * (1 - 2 ** -9)
        hi = 2.0 ** (e - 126) * (1 - 2 ** -9)
        p = 2 * (Phi(hi / sigma) - Phi(lo / sigma))
        sd = math.sqrt(n * p * (1 - p)) + 1e-9
        assert abs(int(hk[e]) - n * p) <= 5 * sd + 1, (e, int(hk[e]), n * p)


def test_rank_table_bruteforce(orc):
    rng = np.random.default_rng(3)
    for trial in range(40):
        nsym = int(rng.integers(1, 7))
        syms = rng.choice(256, size=nsym, replace=False)
        hist = np.zeros(256, dtype=np.uint64)
        counts = rng.integers(1, 6, size=nsym)  # small range -> many ties
        hist[syms] = counts
        perm = orc.rank_table(hist)
        assert sorted(perm.tolist()) == list(range(256)), "total permutation"
        rank = np.empty(256, dtype=np.int64)
        rank[perm] = np.arange(256)
        cost = int((hist.astype(np.int64) * (rank + 1)).sum())
        best = min(sum(int(hist[s]) * (i + 1) for i, s in enumerate(p))
                   for p in itertools.permutations(syms.tolist()))
        assert cost == best, "expected code length is minimal"
        # canonical choice: count descending, then symbol ascending; absent last ascending
        want = sorted(range(256), key=lambda s: (-int(hist[s]), s))
        assert perm.tolist() == want


# --------------------------------------------------------- format round trip


@pytest.mark.parametrize("m", range(8))
def test_all_bf16_patterns_roundtrip_c1(orc, m):
    w = synth.all_bf16_patterns(seed=m)
    for k in (0, 1, 77, 128, 255, 256):
        spec, verif = orc.encode(w, k, m, block=64)
        draft = orc.draft_decode(spec)
        rec = orc.reconstruct(spec, verif)
        assert (rec == w).all(), "lossless reassembly"
        assert ((draft & ~w) == 0).all(), "draft bits are a subset of the original bits"
        keep = orc.select(w, k)
        assert (draft == semantic_draft_c1(w, keep, m)).all()
        d2, o2, _ = sp.parse_c1(spec, verif)
        assert (d2 == draft).all() and (o2 == w).all()


def test_keep_all_full_mantissa_is_identity(orc):
    w = synth.weight(32, 512, 9, outlier_frac=0.01)
    spec, verif = orc.encode(w, 512, 7)
    assert (orc.draft_decode(spec) == w).all()


def mx_semantic_draft(w, keep, m):
    """Cassandra-2 draft from the MX definition on real values: the shared
    exponent of each 32-block is the largest (sub)normal-adjusted exponent of its
    kept values; a kept value is truncated toward zero onto the grid of step
    2^(E-127-m); pruned values are +0."""
    R, C = w.shape
    e = (w.astype(np.int64) >> 7) & 0xFF
    eff = np.maximum(e, 1)
    E = np.where(keep, eff, 0).reshape(R, C // 32, 32).max(axis=2)
    Eb = np.repeat(E, 32, axis=1)
    v = synth.f32_from_bf16(w).astype(np.float64)
    step = np.ldexp(1.0, (Eb - 127 - m))
    q = np.trunc(v / step) * step
    out = (q.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    out[q == 0] = 0
    out[~keep] = 0
    return out, Eb


@pytest.mark.parametrize("m", range(8))
def test_all_bf16_patterns_roundtrip_c2(orc, m):
    w = synth.all_bf16_patterns(seed=100 + m)
    for k in (0, 40, 128, 256):
        spec, verif = orc.encode(w, k, m, block=64, fmt=orc.FMT_C2)
        draft = orc.draft_decode(spec)
        rec = orc.reconstruct(spec, verif)
        assert (rec == w).all(), "lossless reassembly"
        assert ((draft & ~w) == 0).all(), "draft bits are a subset of the original bits"
        keep = orc.select(w, k)
        want, Eb = mx_semantic_draft(w, keep, m)
        finite = ((w >> 7) & 0xFF) != 0xFF
        assert (draft[finite] == want[finite]).all()
        # Inf/NaN: the low bits of the significand are cleared, the exponent kept
        shift = 7 - m + (Eb - 255)
        nf = ~finite & keep
        if nf.any():
            assert (draft[nf] == (w[nf] & ~((1 << shift[nf].clip(0, 7)) - 1))).all()


def test_c2_shared_exponent_offsets(orc):
    """Rows built so that every 32-block mixes exponents 0..6 below its maximum."""
    rng = np.random.default_rng(5)
    base = rng.integers(1, 250, size=(64, 8))
    w = np.zeros((64, 256), dtype=np.uint16)
    for r in range(64):
        for g in range(8):
            E = int(base[r, g])
            e = np.clip(E - rng.integers(0, 7, size=32), 0, 254)
            f = rng.integers(0, 128, size=32)
            s = rng.integers(0, 2, size=32)
            w[r, g * 32:(g + 1) * 32] = (s << 15) | (e << 7) | f
    for m in range(8):
        spec, verif = orc.encode(w, 256, m, block=64, fmt=orc.FMT_C2)
        assert (orc.reconstruct(spec, verif) == w).all()
        want, _ = mx_semantic_draft(w, np.ones_like(w, dtype=bool), m)
        assert (orc.draft_decode(spec) == want).all()
        d2, o2, _ = sp.parse_c2(spec, verif)
        assert (d2 == want).all() and (o2 == w).all()


# ------------------------------------------------------------ closed forms


@pytest.mark.parametrize("k,m", [(0, 3), (307, 2), (512, 3), (205, 4), (1024, 7)])
def test_stream_sizes_closed_form(orc, k, m):
    R, C, B = 48, 1024, 256
    w = synth.weight(R, C, 21, outlier_frac=0.01)
    spec, verif = orc.encode(w, k, m, block=B)
    h = sp.parse_header(spec)
    hv = sp.parse_header(verif)
    # kept set by an independent numpy sort: magnitude desc, column asc
    keep = np.zeros((R, C), dtype=bool)
    for r in range(R):
        order = np.lexsort((np.arange(C), -key(w[r])))
        keep[r, order[:k]] = True
    e = (w.astype(np.int64) >> 7) & 0xFF
    Hk = np.bincount(e[keep], minlength=256)
    Hp = np.bincount(e[~keep], minlength=256)
    _, _, info = sp.parse_c1(spec, verif)
    rank_s = np.empty(256, np.int64); rank_s[info["perm"]] = np.arange(256)
    rank_v = np.empty(256, np.int64); rank_v[info["perm_v"]] = np.arange(256)
    spec_code_bits = int((Hk * (rank_s + 1)).sum())
    verif_code_bits = int((Hp * (rank_v + 1)).sum())
    nb = C // B
    want_spec = [256, R * C // 8, 8 * R, 4 * R * nb, 2 * R * nb,
                 -(-R * k * (1 + m) // 8), -(-spec_code_bits // 8)]
    want_verif = [256, 8 * R, 4 * R * nb, -(-R * k * (7 - m) // 8), R * (C - k),
                  -(-verif_code_bits // 8)]
    assert [n for _, n in h["secs"]] == want_spec
    assert [n for _, n in hv["secs"]] == want_verif
    # sections are 256-aligned, in order, each followed by >= 16 padding bytes
    pos = 256
    for off, n in h["secs"]:
        assert off == pos
        pos = (off + n + 16 + 255) // 256 * 256
    assert h["total"] == pos == spec.size


def entropy_bits(H):
    p = H[H > 0] / H.sum()
    return float(-(p * np.log2(p)).sum())


def test_shannon_bound_and_page_statistics(orc):
    """Mean unary length >= exponent entropy (Shannon).  Also records the
    statistics the pages print (weight exponent entropy about 2.6 bits, unary
    mean about 2.85 bits; those were measured on trained models)."""
    w = synth.weight(512, 4096, 2_000_000, outlier_frac=0.01)
    spec, verif = orc.encode(w, w.shape[1], 3)  # keep all: whole-tensor exponents
    _, _, info = sp.parse_c1(spec, verif)
    e = (w.astype(np.int64) >> 7) & 0xFF
    H = np.bincount(e.ravel(), minlength=256)
    ent = entropy_bits(H)
    mean_len = info["code_bits"] / w.size
    assert ent <= mean_len + 1e-12
    assert 2.3 < ent < 2.9 and mean_len < 3.2  # same regime as the pages' numbers
    for k in (2048, 1229, 819):
        spec, verif = orc.encode(w, k, 3)
        _, _, info = sp.parse_c1(spec, verif)
        keep = info["bitmap"]
        assert entropy_bits(np.bincount(e[keep], minlength=256)) <= info["code_bits"] / keep.sum()
        assert entropy_bits(np.bincount(e[~keep], minlength=256)) <= \
            info["verif_code_bits"] / (~keep).sum()


# --------------------------------------------------------------- products


@pytest.mark.parametrize("fmt", [1, 2])
def test_product_exact_fraction_8x8(orc, fmt):
    rng = np.random.default_rng(17 + fmt)
    w = synth.bf16_from_f32((rng.standard_normal((8, 64)) * 0.05).astype(np.float32))
    x = synth.bf16_from_f32(rng.standard_normal((2, 64)).astype(np.float32))
    for k, m in [(0, 3), (19, 3), (32, 0), (64, 7), (40, 5)]:
        spec, verif = orc.encode(w, k, m, block=32, fmt=fmt)
        keep = orc.select(w, k)
        if fmt == 1:
            d = semantic_draft_c1(w, keep, m)
        else:
            d, _ = mx_semantic_draft(w, keep, m)
        y, absy = orc.product(spec, x)
        Y, absY = orc.product(spec, x, verif=verif)
        for t in range(2):
            for n in range(8):
                ex = sum(exact(d[n, j]) * exact(x[t, j]) for j in range(64))
                ab = sum(abs(exact(d[n, j]) * exact(x[t, j])) for j in range(64))
                assert abs(Fraction(y[t, n]) - ex) <= Fraction(1, 10 ** 12) * (ab + 1)
                assert abs(Fraction(absy[t, n]) - ab) <= Fraction(1, 10 ** 12) * (ab + 1)
                ex = sum(exact(w[n, j]) * exact(x[t, j]) for j in range(64))
                ab = sum(abs(exact(w[n, j]) * exact(x[t, j])) for j in range(64))
                assert abs(Fraction(Y[t, n]) - ex) <= Fraction(1, 10 ** 12) * (ab + 1)


@pytest.mark.parametrize("fmt", [1, 2])
def test_product_rows_exact_fraction(orc, fmt):
    """The row-restricted product: for a shuffled subset of rows (with a
    repeat), y[t][i] is the exact sum over row rows[i] -- draft weights without
    verif, original weights with it -- and the |w||x| sums likewise."""
    rng = np.random.default_rng(29 + fmt)
    w = synth.bf16_from_f32((rng.standard_normal((8, 64)) * 0.05).astype(np.float32))
    x = synth.bf16_from_f32(rng.standard_normal((3, 64)).astype(np.float32))
    rows = np.array([5, 0, 7, 5, 2])
    for k, m in [(19, 3), (64, 7), (0, 2)]:
        spec, verif = orc.encode(w, k, m, block=32, fmt=fmt)
        keep = orc.select(w, k)
        d = semantic_draft_c1(w, keep, m) if fmt == 1 else mx_semantic_draft(w, keep, m)[0]
        for wt, vf in ((d, None), (w, verif)):
            y, absy = orc.product_rows(spec, x, rows, verif=vf)
            assert y.shape == (3, rows.size)
            for t in range(3):
                for i, n in enumerate(rows):
                    ex = sum(exact(wt[n, j]) * exact(x[t, j]) for j in range(64))
                    ab = sum(abs(exact(wt[n, j]) * exact(x[t, j])) for j in range(64))
                    assert abs(Fraction(y[t, i]) - ex) <= Fraction(1, 10 ** 12) * (ab + 1)
                    assert abs(Fraction(absy[t, i]) - ab) <= Fraction(1, 10 ** 12) * (ab + 1)
    with pytest.raises(orc.OracleError):
        orc.product_rows(spec, x, np.array([8]))


def test_product_dense_special_cases(orc):
    """keep=all with m=7 is the plain dense product; the verification product is
    the dense product of the original weights for any k, m; keep=0 gives 0."""
    w = synth.weight(96, 1024, 31, outlier_frac=0.01)
    x = synth.activations(5, 1024, 1)
    W = synth.f32_from_bf16(w).astype(np.float64)
    X = synth.f32_from_bf16(x).astype(np.float64)
    dense = X @ W.T
    spec, verif = orc.encode(w, 1024, 7)
    y, _ = orc.product(spec, x)
    np.testing.assert_allclose(y, dense, rtol=1e-12, atol=1e-12)
    for k, m in [(307, 3), (0, 0), (512, 2)]:
        for fmt in (1, 2):
            spec, verif = orc.encode(w, k, m, fmt=fmt)
            Y, _ = orc.product(spec, x, verif=verif, threads=4)
            np.testing.assert_allclose(Y, dense, rtol=1e-12, atol=1e-12)
    spec, verif = orc.encode(w, 0, 3)
    y, absy = orc.product(spec, x)
    assert (y == 0).all() and (absy == 0).all()


# ------------------------------------------------------------- corruption


def test_corrupt_streams_are_rejected(orc):
    w = synth.weight(8, 512, 41)
    spec, verif = orc.encode(w, 150, 3)
    bad = spec.copy(); bad[0] ^= 1
    with pytest.raises(orc.OracleError):
        orc.draft_decode(bad)
    h = sp.parse_header(spec)
    off, _ = h["secs"][3]  # block offsets
    bad = spec.copy(); bad[off + 4 * 3] ^= 0x10
    with pytest.raises(orc.OracleError):
        orc.draft_decode(bad)
    off, _ = h["secs"][4]  # kept-before counts
    bad = spec.copy(); bad[off + 2] ^= 1
    with pytest.raises(orc.OracleError):
        orc.draft_decode(bad)
    bad = verif.copy(); bad[24] ^= 1  # cols field
    with pytest.raises(orc.OracleError):
        orc.reconstruct(spec, bad)
