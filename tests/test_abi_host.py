"""Host-only checks of the C-ABI library: it loads, exports every symbol the
public header declares, rejects bad arguments before launching anything, and
its host-side stream validator accepts canonical streams and rejects corrupted
ones.  No GPU is touched."""
import ctypes
import os
import re

import numpy as np
import pytest

import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def cass():
    import bit_level_weight_amd as b
    if not os.path.exists(b.LIB_PATH):
        pytest.fail("libcassandra.so is not built (python -m bit_level_weight_amd.build)")
    b.lib()
    return b


def declared_symbols():
    names = set()
    for fn in os.listdir(os.path.join(ROOT, "include")):
        if fn.endswith(".h"):
            text = open(os.path.join(ROOT, "include", fn)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names |= set(re.findall(r"\b(cass_\w+)\s*\(", text))
    return names


def test_exports_every_declared_symbol(cass):
    names = declared_symbols()
    assert len(names) >= 12
    for n in names:
        assert hasattr(cass.lib(), n), n
    assert set(cass.EXPORTED) == names


def test_debug_flags_release_and_debug_builds(cass):
    """The release library reports that its bounds checks are compiled out;
    the debug library (same sources with CASS_DEBUG) exports the same
    symbols."""
    L = cass.lib()
    v = ctypes.c_uint32(7)
    assert L.cass_debug_flags(ctypes.byref(v)) == 2 and v.value == 0  # CASS_ERR_UNSUPPORTED
    assert L.cass_debug_flags(None) == 1
    if not os.path.exists(cass.DEBUG_LIB_PATH):
        pytest.fail("libcassandra_debug.so is not built (python -m bit_level_weight_amd.build debug)")
    D = ctypes.CDLL(cass.DEBUG_LIB_PATH)
    for n in declared_symbols():
        assert hasattr(D, n), n


def test_version_and_status_strings(cass):
    L = cass.lib()
    assert L.cass_version() == 1
    assert L.cass_status_string(0) == b"ok"
    assert L.cass_status_string(4) == b"corrupt stream"


def test_ws_bytes_and_argument_errors(cass):
    L = cass.lib()
    p = cass.CassParams(1, 3, 256, 1229)
    n = ctypes.c_int64(0)
    assert L.cass_encode_ws_bytes(4096, 4096, ctypes.byref(p), ctypes.byref(n)) == 0
    assert n.value >= 4096 * 4096 // 8
    for bad in [cass.CassParams(5, 3, 256, 10), cass.CassParams(1, 8, 256, 10),
                cass.CassParams(1, 3, 100, 10), cass.CassParams(1, 3, 256, 5000),
                cass.CassParams(1, 3, 16, 10)]:
        assert L.cass_encode_ws_bytes(16, 4096, ctypes.byref(bad), ctypes.byref(n)) == \
            cass.CASS_ERR_INVALID
    assert L.cass_encode_ws_bytes(16, 131072, ctypes.byref(p), ctypes.byref(n)) == \
        cass.CASS_ERR_UNSUPPORTED
    # descriptor checks happen before any launch
    t = cass.CassTensor()
    assert L.cass_draft_gemv(None, None, 1, 0, None, 0, None) == cass.CASS_ERR_INVALID
    t.format, t.mant_bits, t.rows, t.cols, t.block, t.keep = 1, 3, 4, 256, 256, 77
    assert L.cass_draft_gemv(ctypes.byref(t), None, 1, 256, None, 4, None) == cass.CASS_ERR_INVALID
    assert L.cass_reconstruct(ctypes.byref(t), None, None) == cass.CASS_ERR_INVALID


@pytest.mark.parametrize("fmt", [1, 2])
def test_host_validator_on_oracle_streams(cass, orc, fmt):
    w = synth.weight(24, 1024, 7, outlier_frac=0.01)
    for k, m in [(307, 3), (0, 0), (1024, 7), (512, 2)]:
        spec, verif = orc.encode(w, k, m, block=256, fmt=fmt)
        assert cass.cass_tensor_validate(spec, verif) == cass.CASS_OK
        assert cass.cass_tensor_validate(spec) == cass.CASS_OK
    spec, verif = orc.encode(w, 307, 3, fmt=fmt)
    rng = np.random.default_rng(0)
    # flipping any header byte that matters, or an offset/count, is caught
    for pos in [0, 4, 8, 16, 24, 40, 48, 64, 72]:
        bad = spec.copy(); bad[pos] ^= 0x01
        assert cass.cass_tensor_validate(bad, verif) == cass.CASS_ERR_CORRUPT, pos
    h = orc.header(spec)
    kb_sec = 4 if fmt == 1 else 2
    off, n = h["sections"][kb_sec]
    for _ in range(5):
        bad = spec.copy()
        bad[off + int(rng.integers(0, n))] ^= 0x04
        assert cass.cass_tensor_validate(bad, verif) == cass.CASS_ERR_CORRUPT
    if fmt == 1:
        off, n = h["sections"][3]  # block offsets
        bad = spec.copy(); bad[off + 8] ^= 0x02
        assert cass.cass_tensor_validate(bad, verif) == cass.CASS_ERR_CORRUPT
    hv = orc.header(verif, orc.MAGIC_VERIF)
    off, n = hv["sections"][1]  # verification row bases
    bad = verif.copy(); bad[off + 8] ^= 0x10
    assert cass.cass_tensor_validate(spec, bad) == cass.CASS_ERR_CORRUPT
    assert cass.cass_tensor_validate(spec[:200]) == cass.CASS_ERR_CORRUPT


def test_describe_from_headers(cass, orc):
    w = synth.weight(8, 512, 3)
    spec, verif = orc.encode(w, 150, 3)
    t = cass.cass_tensor_describe(spec.tobytes(), FakeDev(spec.size), verif.tobytes(),
                                  FakeDev(verif.size))
    h = orc.header(spec)
    assert (t.rows, t.cols, t.keep, t.mant_bits, t.block) == (8, 512, 150, 3, 256)
    assert [t.spec_sec[i] for i in range(7)] == [o for o, _ in h["sections"]]
    with pytest.raises(cass.CassError):
        cass.cass_tensor_describe(verif.tobytes(), FakeDev(verif.size))


class FakeDev:
    """Stands in for a device buffer: describe and the argument checks only
    record pointers and sizes."""
    def __init__(self, n, ptr=0x100000):
        self.n, self.ptr = n, ptr

    def numel(self):
        return self.n

    def data_ptr(self):
        return self.ptr


@pytest.mark.parametrize("fmt", [1, 2])
def test_describe_rejects_inflated_headers(cass, orc, fmt):
    """A header whose shape asks for more bytes than its section table and
    buffers hold is refused before anything could be launched: an inflated row
    count, a section length off its closed form, a section past the buffer, a
    truncated buffer, a misaligned buffer."""
    w = synth.weight(8, 512, 3)
    spec, verif = orc.encode(w, 150, 3, fmt=fmt)
    t = cass.cass_tensor_describe(spec.tobytes(), FakeDev(spec.size), verif.tobytes(),
                                  FakeDev(verif.size))
    assert t.rows == 8

    def corrupt(buf, pos, value):
        b = bytearray(buf.tobytes())
        b[pos:pos + 8] = int(value).to_bytes(8, "little")
        return bytes(b)

    bad_cases = [
        (corrupt(spec, 16, 4096), verif.tobytes(), spec.size),            # rows 8 -> 4096
        (corrupt(spec, 72 + 16 * 1, 1 << 20), verif.tobytes(), spec.size),  # a section length
        (corrupt(spec, 64 + 16 * 1, spec.size - 256), verif.tobytes(), spec.size),  # offset
        (spec.tobytes(), verif.tobytes(), spec.size - 512),               # truncated buffer
    ]
    for sh, vh, n in bad_cases:
        with pytest.raises(cass.CassError) as e:
            cass.cass_tensor_describe(sh, FakeDev(n), vh, FakeDev(verif.size))
        assert e.value.status == cass.CASS_ERR_CORRUPT
    with pytest.raises(cass.CassError) as e:
        cass.cass_tensor_describe(spec.tobytes(), FakeDev(spec.size, 0x100008), None, None)
    assert e.value.status == cass.CASS_ERR_INVALID


def test_descriptor_sections_checked_before_launch(cass, orc):
    """A hand-made descriptor whose sections do not hold the shape's
    closed-form sizes is refused by every call before any launch."""
    L = cass.lib()
    w = synth.weight(8, 512, 3)
    spec, verif = orc.encode(w, 150, 3)
    t = cass.cass_tensor_describe(spec.tobytes(), FakeDev(spec.size), verif.tobytes(),
                                  FakeDev(verif.size))
    t.rows = 4096  # the buffers hold 8 rows
    assert L.cass_draft_gemv(ctypes.byref(t), ctypes.c_void_p(0x200000), 1, 512,
                             ctypes.c_void_p(0x300000), 4096, None) == cass.CASS_ERR_INVALID
    assert b"section" in L.cass_last_error()
    t.rows = 8
    t.spec_sec[5] = t.spec_sec[6]  # fields moved onto the codes section
    assert L.cass_draft_gemv(ctypes.byref(t), ctypes.c_void_p(0x200000), 1, 512,
                             ctypes.c_void_p(0x300000), 8, None) == cass.CASS_ERR_INVALID


def test_encode_argument_errors(cass):
    """Row stride and plan checks of the encoder, all before any launch."""
    L = cass.lib()
    p = cass.CassParams(1, 3, 256, 100)
    plan = cass.CassPlan()
    ws = ctypes.c_void_p(0x100000)
    # ld < cols
    assert L.cass_encode_plan(ctypes.c_void_p(0x200000), 4, 512, 500, ctypes.byref(p), ws,
                              1 << 30, None, ctypes.byref(plan)) == cass.CASS_ERR_INVALID
    assert b"ld" in L.cass_last_error()
    # a plan made for one stride is refused for another
    plan.rows, plan.cols, plan.ld, plan.p = 4, 512, 640, p
    assert L.cass_encode_tensor(ctypes.c_void_p(0x200000), 512, ctypes.byref(plan),
                                ctypes.c_void_p(0x300000), 1 << 20, ctypes.c_void_p(0x400000),
                                1 << 20, None, ctypes.byref(cass.CassTensor())) == \
        cass.CASS_ERR_INVALID


def test_set_option(cass):
    L = cass.lib()
    assert L.cass_set_option(b"gemv_parts", 16) == cass.CASS_OK
    assert L.cass_set_option(b"gemv_parts", 0) == cass.CASS_OK
    assert L.cass_set_option(b"gemv_parts", 65) == cass.CASS_ERR_INVALID
    assert L.cass_set_option(b"no_such_option", 1) == cass.CASS_ERR_INVALID
    assert L.cass_set_option(None, 1) == cass.CASS_ERR_INVALID
    assert L.cass_stream_read(ctypes.c_void_p(0x100008), 64, ctypes.c_void_p(0x200000),
                              None) == cass.CASS_ERR_INVALID


def test_format3_validate_and_describe(cass, orc):
    """Format 3 (MX-quantised target): oracle streams validate and describe
    with closed-form section lengths; a group exponent of 0, or one that
    differs from the shared exponent of a group that keeps values, is corrupt."""
    w = synth.weight(16, 1024, 8, outlier_frac=0.01)
    spec, verif = orc.encode(w, 307, 3, fmt=3)
    assert cass.cass_tensor_validate(spec, verif) == cass.CASS_OK
    assert cass.cass_tensor_validate(spec) == cass.CASS_OK
    t = cass.cass_tensor_describe(spec.tobytes(), FakeDev(spec.size), verif.tobytes(),
                                  FakeDev(verif.size))
    assert (t.format, t.rows, t.cols, t.keep) == (3, 16, 1024, 307)
    hv = orc.header(verif, orc.MAGIC_VERIF)
    off = hv["sections"][0][0]
    for pos, val in ((off, 0), (off + 3, int(verif[off + 3]) ^ 1)):
        bad = verif.copy()
        bad[pos] = val
        assert cass.cass_tensor_validate(spec, bad) == cass.CASS_ERR_CORRUPT
    # a length off its closed form is refused by describe
    b = bytearray(verif.tobytes())
    b[72 + 16:80 + 16] = (int(hv["sections"][1][1]) + 1).to_bytes(8, "little")
    with pytest.raises(cass.CassError):
        cass.cass_tensor_describe(spec.tobytes(), FakeDev(spec.size), bytes(b), FakeDev(verif.size))


@pytest.mark.parametrize("seed", range(6))
def test_prefix_code_tables_match_oracle(cass, orc, seed):
    """The library's host-built Huffman (package-merge, canonical values) and
    unary code tables equal the oracle's, on histograms of kept exponents and
    on random ones."""
    rng = np.random.default_rng(seed)
    if seed < 3:
        w = synth.weight(64, 1024, 40 + seed, outlier_frac=0.01)
        keep = orc.select(w, 307)
        hist = np.bincount(((w[keep] >> 7) & 0xFF).astype(np.int64), minlength=256).astype(np.uint64)
    else:
        hist = np.zeros(256, dtype=np.uint64)
        syms = rng.choice(256, size=int(rng.integers(2, 120)), replace=False)
        hist[syms] = (2.0 ** rng.uniform(0, 20, size=syms.size)).astype(np.uint64) + 1
    for L in (12, 16, 32):
        if (1 << L) < np.count_nonzero(hist):
            continue
        c = cass.cass_prefix_code_huffman(hist, L)
        ln, code = orc.huffman_code(hist, L)
        assert list(c.len) == list(ln) and list(c.code) == list(code), L
        assert c.max_len == int(ln.max())
        assert cass.cass_prefix_stream_bits(c, hist) == int((hist * ln).sum())
    u = cass.cass_prefix_code_unary(hist)
    ln, code = orc.unary_code(hist)
    short = ln <= 32
    assert np.array_equal(np.array(u.len)[short], ln[short])
    assert np.all(np.array(u.code)[short] == 1)


def test_prefix_argument_errors(cass):
    L = cass.lib()
    hist = np.zeros(256, dtype=np.uint64)
    hist[[3, 5, 9]] = [10, 3, 1]
    huff = cass.cass_prefix_code_huffman(hist, 12)
    P = ctypes.c_void_p
    # a Huffman code is not a unary code
    assert L.cass_prefix_decode(ctypes.byref(huff), P(0x100000), 4096, P(0x200000), 64, 64,
                                cass.CASS_PREFIX_UNARY_SERIAL, P(0x300000), None, 0,
                                None) == cass.CASS_ERR_INVALID
    # unknown method, misaligned output, n not a multiple of 16
    assert L.cass_prefix_decode(ctypes.byref(huff), P(0x100000), 4096, P(0x200000), 64, 64, 9,
                                P(0x300000), None, 0, None) == cass.CASS_ERR_INVALID
    assert L.cass_prefix_decode(ctypes.byref(huff), P(0x100000), 4096, P(0x200000), 64, 64,
                                cass.CASS_PREFIX_TABLE, P(0x300001), None, 0,
                                None) == cass.CASS_ERR_INVALID
    assert L.cass_prefix_decode(ctypes.byref(huff), P(0x100000), 4096, P(0x200000), 60, 64,
                                cass.CASS_PREFIX_TABLE, P(0x300000), None, 0,
                                None) == cass.CASS_ERR_INVALID
    # table decoding needs codes of at most 12 bits
    long = cass.cass_prefix_code_unary(hist)
    long.len[7], long.code[7], long.max_len = 20, 1, 20
    assert L.cass_prefix_decode(ctypes.byref(long), P(0x100000), 4096, P(0x200000), 64, 64,
                                cass.CASS_PREFIX_TABLE, P(0x300000), None, 0,
                                None) != cass.CASS_OK
    # Kraft's inequality
    bad = cass.cass_prefix_code_huffman(hist, 12)
    bad.len[100], bad.code[100] = 1, 0
    assert L.cass_prefix_encode(ctypes.byref(bad), P(0x100000), 64, 64, P(0x200000), 4096,
                                P(0x300000), None) == cass.CASS_ERR_INVALID
    # a present symbol without a code
    hist2 = hist.copy()
    hist2[200] = 1
    with pytest.raises(cass.CassError):
        cass.cass_prefix_stream_bits(huff, hist2)


def test_format4_validate_and_describe(cass, orc):
    """Format 4 (superblock metadata): oracle streams validate and describe;
    a moved superblock base, a wrong 16-bit offset or a wrong superblock-size
    field is corrupt."""
    w = synth.weight(12, 8192, 9, outlier_frac=0.01)
    spec, verif = orc.encode(w, 2458, 3, fmt=4)
    assert cass.cass_tensor_validate(spec, verif) == cass.CASS_OK
    t = cass.cass_tensor_describe(spec.tobytes(), FakeDev(spec.size), verif.tobytes(),
                                  FakeDev(verif.size))
    assert (t.format, t.rows, t.cols) == (4, 12, 8192)
    h = orc.header(spec)
    sb_off, bo_off = h["sections"][2][0], h["sections"][3][0]
    for pos in (sb_off + 8, bo_off + 2, 60):
        bad = spec.copy()
        bad[pos] ^= 1
        assert cass.cass_tensor_validate(bad, verif) == cass.CASS_ERR_CORRUPT, pos
    bad = spec.copy()
    bad[60] = 8
    with pytest.raises(cass.CassError):
        cass.cass_tensor_describe(bad.tobytes(), FakeDev(spec.size), verif.tobytes(),
                                  FakeDev(verif.size))
