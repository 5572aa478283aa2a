"""An independent reader of the two-stream byte layout, written in numpy.

Test helper only: it shares nothing with the C oracle or the HIP library.  It
parses the documented layout (256-byte header, 256-aligned sections, bit i of a
bit section = bit (i & 7) of byte i >> 3) and rebuilds the draft and the
original weights, so that tests can check the encoders' bytes against the
input tensor itself rather than against another decoder.
"""
from __future__ import annotations

import struct

import numpy as np

MAGIC_SPEC, MAGIC_VERIF = 0x50535343, 0x46565343


def parse_header(buf):
    buf = bytes(np.asarray(buf, dtype=np.uint8)[:256])
    magic, version, fmt, mant = struct.unpack_from("<4I", buf, 0)
    R, C, B, k, total = struct.unpack_from("<5q", buf, 16)
    (nsec,) = struct.unpack_from("<I", buf, 56)
    secs = [struct.unpack_from("<2q", buf, 64 + 16 * s) for s in range(12)]
    return dict(magic=magic, version=version, format=fmt, m=mant, R=R, C=C, B=B, k=k,
                total=total, nsec=nsec, secs=secs[:nsec])


def section(buf, h, i):
    off, n = h["secs"][i]
    return np.asarray(buf, dtype=np.uint8)[off:off + n]


def bits_of(arr):
    return np.unpackbits(np.asarray(arr, dtype=np.uint8), bitorder="little")


def fixed_fields(sec, count, width):
    """count unsigned fields of `width` bits, packed back to back, LSB first."""
    if width == 0:
        return np.zeros(count, dtype=np.int64)
    b = bits_of(sec)[: count * width].reshape(count, width).astype(np.int64)
    return (b << np.arange(width, dtype=np.int64)).sum(axis=1)


def unary_ranks(sec, count):
    """Decode `count` unary codes (zeros then a one); returns (ranks, end bit of each)."""
    ones = np.flatnonzero(bits_of(sec))[:count]
    assert ones.size == count, "stream ends early"
    starts = np.concatenate([[0], ones[:-1] + 1]) if count else np.zeros(0, np.int64)
    return ones - starts, ones + 1


def parse_c1(spec, verif=None):
    """-> (draft [R,C] uint16, original or None, info dict)."""
    h = parse_header(spec)
    assert h["magic"] == MAGIC_SPEC and h["version"] == 1 and h["format"] == 1
    R, C, B, k, m = h["R"], h["C"], h["B"], h["k"], h["m"]
    nb = C // B
    perm = section(spec, h, 0)
    bitmap = bits_of(section(spec, h, 1))[: R * C].reshape(R, C).astype(bool)
    rowbase = section(spec, h, 2).view("<u8")
    blkoff = section(spec, h, 3).view("<u4").reshape(R, nb)
    keptb = section(spec, h, 4).view("<u2").reshape(R, nb)
    fields = fixed_fields(section(spec, h, 5), R * k, 1 + m)
    ranks, ends = unary_ranks(section(spec, h, 6), R * k)
    assert (bitmap.sum(axis=1) == k).all(), "k kept per row"
    # per-block kept-before counts and code offsets
    cnt = bitmap.reshape(R, nb, B).sum(axis=2)
    kb = np.concatenate([np.zeros((R, 1), np.int64), np.cumsum(cnt, axis=1)[:, :-1]], axis=1)
    assert (keptb == kb).all(), "kept-before"
    starts = np.concatenate([[0], ends[:-1]]) if R * k else np.zeros(0, np.int64)
    total_bits = int(ends[-1]) if R * k else 0
    for r in range(R):
        row_start = int(starts[r * k]) if k else 0
        row_end = int(ends[(r + 1) * k - 1]) if k else 0
        assert int(rowbase[r]) == row_start, "row base"
        for b in range(nb):
            i = int(kb[r, b])
            pos = int(starts[r * k + i]) if i < k else row_end
            assert int(blkoff[r, b]) == pos - row_start, "block offset"
    s = fields >> m
    ft = fields & ((1 << m) - 1)
    e = perm[ranks].astype(np.int64)
    dk = (s << 15) | (e << 7) | (ft << (7 - m))
    draft = np.zeros((R, C), dtype=np.uint16)
    draft[bitmap] = dk.astype(np.uint16)
    info = dict(h=h, code_bits=total_bits, ranks=ranks, perm=perm, bitmap=bitmap)
    if verif is None:
        return draft, None, info
    hv = parse_header(verif)
    assert hv["magic"] == MAGIC_VERIF and hv["format"] == 1
    perm_v = section(verif, hv, 0)
    vrowbase = section(verif, hv, 1).view("<u8")
    low = fixed_fields(section(verif, hv, 3), R * k, 7 - m)
    pbytes = section(verif, hv, 4).astype(np.int64)
    vranks, vends = unary_ranks(section(verif, hv, 5), R * (C - k))
    vstarts = np.concatenate([[0], vends[:-1]]) if R * (C - k) else np.zeros(0, np.int64)
    if C - k:
        assert (vrowbase == vstarts[np.arange(R) * (C - k)]).all(), "verif row base"
    ev = perm_v[vranks].astype(np.int64)
    orig = np.zeros((R, C), dtype=np.uint16)
    orig[bitmap] = (dk | low).astype(np.uint16)
    orig[~bitmap] = (((pbytes >> 7) << 15) | (ev << 7) | (pbytes & 0x7F)).astype(np.uint16)
    info.update(verif_code_bits=int(vends[-1]) if vends.size else 0, vranks=vranks, perm_v=perm_v)
    return draft, orig, info


def parse_c2(spec, verif=None):
    h = parse_header(spec)
    assert h["magic"] == MAGIC_SPEC and h["format"] == 2
    R, C, B, k, m = h["R"], h["C"], h["B"], h["k"], h["m"]
    nb = C // B
    bitmap = bits_of(section(spec, h, 0))[: R * C].reshape(R, C).astype(bool)
    shexp = section(spec, h, 1).reshape(R, C // 32).astype(np.int64)
    keptb = section(spec, h, 2).view("<u2").reshape(R, nb)
    fields = fixed_fields(section(spec, h, 3), R * k, 2 + m)
    cnt = bitmap.reshape(R, nb, B).sum(axis=2)
    kb = np.concatenate([np.zeros((R, 1), np.int64), np.cumsum(cnt, axis=1)[:, :-1]], axis=1)
    assert (keptb == kb).all()
    s = fields >> (m + 1)
    a = fields & ((1 << (m + 1)) - 1)
    rr, cc = np.nonzero(bitmap)
    E = shexp[rr, cc // 32]
    # value a * 2^(E-127-m), as an exact float32, then its top 16 bits
    val = np.ldexp(a.astype(np.float64), (E - 127 - m).astype(np.int64)).astype(np.float32)
    dk = (val.view(np.uint32) >> 16).astype(np.int64) | (s << 15)
    dk[a == 0] = 0
    draft = np.zeros((R, C), dtype=np.uint16)
    draft[bitmap] = dk.astype(np.uint16)
    if verif is None:
        return draft, None, dict(h=h, shexp=shexp)
    hv = parse_header(verif)
    perm_v = section(verif, hv, 0)
    resid_bits = bits_of(section(verif, hv, 3))
    pbytes = section(verif, hv, 4).astype(np.int64)
    vranks, _ = unary_ranks(section(verif, hv, 7), R * (C - k))
    orig = np.zeros((R, C), dtype=np.uint16)
    pos = 0
    vals = np.zeros(R * k, dtype=np.int64)
    for i in range(R * k):
        d = 0
        while resid_bits[pos + d] == 0:
            d += 1
        pos += d + 1
        w = min(8, 7 - m + d)
        L = 0
        for t in range(w):
            L |= int(resid_bits[pos + t]) << t
        pos += w
        M = (int(a[i]) << w) | L if w < 8 else L
        e = int(E[i]) - d if M >= 128 else 0
        vals[i] = (int(s[i]) << 15) | (e << 7) | (M & 0x7F)
    orig[bitmap] = vals.astype(np.uint16)
    ev = perm_v[vranks].astype(np.int64)
    orig[~bitmap] = (((pbytes >> 7) << 15) | (ev << 7) | (pbytes & 0x7F)).astype(np.uint16)
    return draft, orig, dict(h=h, shexp=shexp)
