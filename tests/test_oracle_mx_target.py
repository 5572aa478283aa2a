"""Pins of the oracle's format 3: Cassandra-2 with an MX-quantised target.

Reading (Cassandra review, marsggbo.github.io, section 3.2: Cassandra-2
shares one MX exponent per 32 values, compressing further at a slight loss of
precision; OCP MX specification: one shared exponent per 32-element block):
in this mode the loss reaches the target as well.  Per group of 32 positions
of a row the target keeps every value truncated toward zero to a multiple of
2^(X-134), X being the group's largest max(e,1) -- an 8-bit significand
aligned to the shared exponent.  The draft is Cassandra-2's.

The checks use float arithmetic and numpy bit unpacking, never the oracle's
own helpers:
  * every finite value of every bf16 pattern, in groups whose maximum sits 0 to
    40 binades above it: target == trunc(w / 2^(X-134)) * 2^(X-134) exactly;
    zeros come out as +0; Inf and NaN leaders keep their bits;
  * the target is idempotent and never larger in magnitude than w;
  * the draft equals the target truncated to multiples of 2^(X-127-m) (kept
    values) or +0 (pruned), so draft bits are a subset of the target's;
  * the verification stream's sections, unpacked with numpy, hold the group
    maxima, the low 7-m bits of each kept t and (sign, t) of each pruned value,
    with closed-form sizes;
  * the product with the target is numpy's fp64 matmul of the target.
"""
import numpy as np
import pytest

import synth
import streamparse as sp

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def f64(b):
    return synth.f32_from_bf16(np.asarray(b, dtype=np.uint16)).astype(np.float64)


def group_max_eff(w):
    e = (w.astype(np.int64) >> 7) & 0xFF
    eff = np.maximum(e, 1)
    R, C = w.shape
    return eff.reshape(R, C // 32, 32).max(axis=2)


def target_by_floats(w):
    """trunc(w / 2^(X-134)) * 2^(X-134) per group (finite groups only)."""
    X = np.repeat(group_max_eff(w), 32, axis=1)
    q = np.ldexp(1.0, X - 134)
    return np.trunc(f64(w) / q) * q


def groups_around(seed):
    """Every bf16 pattern once, each in a group whose largest value sits
    0..40 binades above it (the leader is finite and placed at position 0)."""
    rng = np.random.default_rng(seed)
    pats = rng.permutation(np.arange(65536, dtype=np.uint16))
    per = 31
    n_groups = (pats.size + 8 * per - 1) // (8 * per) * 8  # whole rows of 8 groups
    pats = np.concatenate([pats, np.zeros(n_groups * per - pats.size, np.uint16)])
    body = pats.reshape(n_groups, per)
    e = (body.astype(np.int64) >> 7) & 0xFF
    top = np.maximum(e, 1).max(axis=1)
    lift = rng.integers(0, 41, size=n_groups)
    lead_e = np.minimum(top + lift, 254)
    lead = ((rng.integers(0, 2, size=n_groups) << 15) | (lead_e << 7) |
            rng.integers(0, 128, size=n_groups)).astype(np.uint16)
    g = np.concatenate([lead[:, None], body], axis=1)
    return g.reshape(-1, 256)  # 8 groups per row


def test_target_closed_form_all_patterns(orc):
    w = groups_around(1)
    t = orc.mx_target(w)
    finite_group = np.repeat(((w.reshape(-1, 32) >> 7) & 0xFF).max(axis=1) < 255, 32)
    finite_group = finite_group.reshape(w.shape)
    ref = target_by_floats(w)
    got = f64(t)
    assert np.array_equal(got[finite_group], ref[finite_group])
    assert np.all(t[(got == 0)] == 0), "zero is +0"
    assert np.all(np.abs(got[finite_group]) <= np.abs(f64(w)[finite_group]))
    # groups holding Inf or NaN: the exponent-255 values are kept bit for bit
    special = ((w >> 7) & 0xFF) == 255
    assert special.any()
    assert np.array_equal(t[special], w[special])
    # the rest of those groups: multiples of 2^121, truncated
    rest = ~finite_group & ~special
    q = 2.0 ** (255 - 134)
    assert np.array_equal(got[rest], np.trunc(f64(w)[rest] / q) * q)


def test_target_idempotent_and_equal_exponent_groups_exact(orc):
    w = synth.weight(64, 512, 3, outlier_frac=0.02)
    t = orc.mx_target(w)
    assert np.array_equal(orc.mx_target(t), t)
    # a group whose values share one exponent (and no zeros) is kept exactly
    rng = np.random.default_rng(2)
    e = rng.integers(1, 254, size=(16, 8))
    same = ((rng.integers(0, 2, size=(16, 256)) << 15) | (np.repeat(e, 32, axis=1) << 7) |
            rng.integers(0, 128, size=(16, 256))).astype(np.uint16)
    assert np.array_equal(orc.mx_target(same), same)


@pytest.mark.parametrize("k,m", [(77, 3), (0, 2), (256, 7), (128, 0), (200, 4)])
def test_format3_streams(orc, k, m):
    w = groups_around(10 + m)[:128]
    R, C = w.shape
    finite = np.repeat(((w.reshape(-1, 32) >> 7) & 0xFF).max(axis=1) < 255, 32).reshape(w.shape)
    spec, verif = orc.encode(w, k, m, block=64, fmt=orc.FMT_C2T)
    tgt = orc.mx_target(w)
    assert np.array_equal(orc.reconstruct(spec, verif), tgt)
    keep = orc.select(w, k)
    # the draft: kept values of the target truncated to multiples of 2^(X-127-m), pruned +0
    draft = orc.draft_decode(spec)
    X = np.repeat(group_max_eff(w), 32, axis=1)
    qd = np.ldexp(1.0, X - 127 - m)
    want = np.where(keep, np.trunc(f64(tgt) / qd) * qd, 0.0)
    assert np.array_equal(f64(draft)[finite], want[finite])
    assert np.all((draft & ~tgt) == 0), "draft bits are a subset of the target's"
    # the speculation stream is Cassandra-2's, byte for byte
    spec2, _ = orc.encode(w, k, m, block=64, fmt=orc.FMT_C2)
    assert np.array_equal(spec[256:], spec2[256:]) and spec[8] == 3 and spec2[8] == 2
    # verification sections, unpacked with numpy
    hv = sp.parse_header(verif)
    assert hv["format"] == 3 and hv["nsec"] == 3
    lens = [n for _, n in hv["secs"]]
    assert lens == [R * C // 32, (R * k * (7 - m) + 7) // 8, (R * (C - k) * 9 + 7) // 8]
    assert np.array_equal(sp.section(verif, hv, 0), group_max_eff(w).reshape(-1).astype(np.uint8))
    e = (w.astype(np.int64) >> 7) & 0xFF
    M = np.where(e > 0, 128, 0) | (w.astype(np.int64) & 0x7F)
    d = X - np.maximum(e, 1)
    t = np.where(d >= 8, 0, M >> np.minimum(d, 7))
    low = sp.fixed_fields(sp.section(verif, hv, 1), R * k, 7 - m)
    assert np.array_equal(low, (t[keep] & ((1 << (7 - m)) - 1)))
    pr = sp.fixed_fields(sp.section(verif, hv, 2), R * (C - k), 9)
    sgn = w.astype(np.int64) >> 15
    assert np.array_equal(pr, ((sgn << 8) | t)[~keep])
    total = 256
    for n in lens:
        total = (total + n + 16 + 255) // 256 * 256
    assert verif.size == total


def test_format3_product_is_matmul_of_target(orc):
    w = synth.weight(48, 512, 9, outlier_frac=0.02)
    x = synth.activations(5, 512, 2)
    spec, verif = orc.encode(w, 150, 3, fmt=orc.FMT_C2T)
    y, absy = orc.product(spec, x, verif=verif)
    ref = f64(x) @ f64(orc.mx_target(w)).T
    assert np.all(np.abs(y - ref) <= 1e-12 * (np.abs(f64(x)) @ np.abs(f64(orc.mx_target(w))).T) + 1e-300)
    assert np.allclose(absy, np.abs(f64(x)) @ np.abs(f64(orc.mx_target(w))).T, rtol=1e-12, atol=0)


def test_format3_corrupt_group_exponent_rejected(orc):
    w = synth.weight(8, 256, 4)
    spec, verif = orc.encode(w, 80, 3, fmt=orc.FMT_C2T)
    hv = sp.parse_header(verif)
    off = hv["secs"][0][0]
    bad = verif.copy()
    bad[off] = 0  # group exponent 0: impossible
    with pytest.raises(orc.OracleError):
        orc.reconstruct(spec, bad)
    bad = verif.copy()
    bad[off + 1] ^= 1  # no longer the group's kept maximum
    with pytest.raises(orc.OracleError):
        orc.reconstruct(spec, bad)
