"""Pins of the oracle's format 4: Cassandra-1 with superblock metadata
(pith.science review of the Cassandra paper, Figure 11: superblock-based data
management).  A superblock is 16 consecutive blocks of a row; its code base is
a u64 and each block's code offset a u16 from that base, in place of
Cassandra-1's u64 row base and u32 block offset.

Checked against the Cassandra-1 stream of the same tensor, read with the
independent numpy parser: every other section is byte-equal, the superblock
bases equal row base + block offset at each superblock's first block, the u16
offsets equal the differences of the u32 ones, the section sizes have their
closed forms, both decoders give Cassandra-1's results, and a superblock whose
codes run past 2^16 bits is refused.
"""
import numpy as np
import pytest

import synth
import streamparse as sp


def u64s(sec):
    return np.frombuffer(sec.tobytes(), dtype="<u8")


def u32s(sec):
    return np.frombuffer(sec.tobytes(), dtype="<u4")


def u16s(sec):
    return np.frombuffer(sec.tobytes(), dtype="<u2")


@pytest.mark.parametrize("R,C,k,m,B", [(24, 4096, 1229, 3, 256), (9, 14336, 4301, 2, 256),
                                       (5, 1024, 300, 3, 32), (3, 512, 0, 3, 64),
                                       (4, 2048, 2048, 7, 128)])
def test_superblock_stream_against_cassandra1(orc, R, C, k, m, B):
    w = synth.weight(R, C, 600 + R + C, outlier_frac=0.01)
    s1, v1 = orc.encode(w, k, m, block=B, fmt=orc.FMT_C1)
    s4, v4 = orc.encode(w, k, m, block=B, fmt=orc.FMT_C1S)
    h1, h4 = sp.parse_header(s1), sp.parse_header(s4)
    nb = C // B
    nsb = -(-nb // 16)
    assert h4["format"] == 4 and h4["nsec"] == 7
    assert int(np.frombuffer(s4[60:64].tobytes(), "<u4")[0]) == 16
    for sec in (0, 1, 4, 5, 6):
        assert np.array_equal(sp.section(s1, h1, sec), sp.section(s4, h4, sec)), sec
    assert [n for _, n in h4["secs"]][2:4] == [8 * R * nsb, 2 * R * nb]
    rowbase = u64s(sp.section(s1, h1, 2))
    blkoff = u32s(sp.section(s1, h1, 3)).reshape(R, nb).astype(np.int64)
    sbb = u64s(sp.section(s4, h4, 2)).reshape(R, nsb)
    off16 = u16s(sp.section(s4, h4, 3)).reshape(R, nb)
    first = np.arange(nsb) * 16
    assert np.array_equal(sbb, rowbase[:, None] + blkoff[:, first].astype(np.uint64))
    assert np.array_equal(off16, blkoff - np.repeat(blkoff[:, first], 16, axis=1)[:, :nb])
    # the verification stream is Cassandra-1's
    assert np.array_equal(v4[256:], v1[256:])
    assert np.array_equal(orc.draft_decode(s4), orc.draft_decode(s1))
    assert np.array_equal(orc.reconstruct(s4, v4), w)
    # metadata bits per value: closed forms
    meta1 = 64 * R + 48 * R * nb
    meta4 = 64 * R * nsb + 32 * R * nb
    assert 8 * (sum(n for _, n in h1["secs"][2:5]) - sum(n for _, n in h4["secs"][2:5])) == meta1 - meta4


def test_superblock_offsets_past_16_bits_refused(orc):
    # every exponent equally often and all kept: ranks up to 255, long codes
    rng = np.random.default_rng(1)
    e = rng.permutation(np.repeat(np.arange(256), 16))
    w = ((e << 7) | rng.integers(0, 128, size=e.size)).astype(np.uint16).reshape(1, 4096)
    with pytest.raises(orc.OracleError) as ex:
        orc.encode(w, 4096, 3, fmt=orc.FMT_C1S)
    assert ex.value.status == orc.ERR_OVERFLOW
    s1, v1 = orc.encode(w, 4096, 3, fmt=orc.FMT_C1)  # the flat layout takes it
    assert np.array_equal(orc.reconstruct(s1, v1), w)


def test_superblock_corrupt_base_rejected(orc):
    w = synth.weight(6, 8192, 5)
    s4, v4 = orc.encode(w, 2458, 3, fmt=orc.FMT_C1S)
    h4 = sp.parse_header(s4)
    off = h4["secs"][2][0]
    bad = s4.copy()
    bad[off + 8] ^= 1  # second superblock of row 0
    with pytest.raises(orc.OracleError):
        orc.reconstruct(bad, v4)
    bad = s4.copy()
    bad[60] = 8  # superblock size field
    with pytest.raises(orc.OracleError):
        orc.draft_decode(bad)
