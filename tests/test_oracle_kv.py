"""Pins of the KV-cache part of the oracle (online compression of keys and
values, draft and verification attention).

Sources (page title, section): Cassandra review, marsggbo.github.io, section
3.1 (the KV cache goes through the same pruning / truncation / exponent coding
as the weights), section 3.3 (KV entries are produced during inference, so the
encoder runs online).  Attention itself is the textbook softmax attention.
"""
import numpy as np
import pytest
from scipy.special import softmax

import synth

D, K_KEEP, M = 128, 38, 3


def caps(T_max, k=K_KEEP):
    return T_max * k * 8, T_max * (D - k) * 8


def parse_kv(spec, verif, T, k, m, T_max, code_cap, vcode_cap):
    """Independent numpy reader of one stream's regions (documented layout:
    256-aligned parts, each followed by >= 16 zero bytes)."""
    def parts(sizes):
        out, pos = [], 0
        for n in sizes:
            out.append(pos)
            pos = (pos + n + 16 + 255) // 256 * 256
        return out
    so = parts([256, T_max * D // 8, 4 * T_max, (T_max * k * (1 + m) + 7) // 8, (code_cap + 7) // 8])
    vo = parts([256, (T_max * k * (7 - m) + 7) // 8, T_max * (D - k), 4 * T_max, (vcode_cap + 7) // 8])
    bits = lambda a: np.unpackbits(a, bitorder="little").astype(np.int64)
    perm = spec[so[0]:so[0] + 256]
    bm = bits(spec[so[1]:so[1] + T_max * D // 8])[: T * D].reshape(T, D).astype(bool)
    offs = spec[so[2]:so[2] + 4 * T_max].view("<u4")[:T]
    fb = bits(spec[so[3]:so[4]])[: T * k * (1 + m)].reshape(T * k, 1 + m)
    fields = (fb << np.arange(1 + m)).sum(axis=1)
    cb = bits(spec[so[4]:])
    ones = np.flatnonzero(cb)[: T * k]
    starts = np.concatenate([[0], ones[:-1] + 1])
    ranks = ones - starts
    assert (offs == starts[np.arange(T) * k]).all(), "per-token code offsets"
    s, ft = fields >> m, fields & ((1 << m) - 1)
    draft = np.zeros((T, D), np.uint16)
    draft[bm] = ((s << 15) | (perm[ranks].astype(np.int64) << 7) | (ft << (7 - m))).astype(np.uint16)
    lb = bits(verif[vo[1]:vo[2]])[: T * k * (7 - m)].reshape(T * k, 7 - m) if m < 7 else np.zeros((T * k, 0), np.int64)
    low = (lb << np.arange(7 - m)).sum(axis=1) if m < 7 else np.zeros(T * k, np.int64)
    pb = verif[vo[2]:vo[2] + T * (D - k)].astype(np.int64)
    vb = bits(verif[vo[4]:])
    vones = np.flatnonzero(vb)[: T * (D - k)]
    vstarts = np.concatenate([[0], vones[:-1] + 1]) if vones.size else vones
    vr = vones - vstarts
    perm_v = verif[vo[0]:vo[0] + 256]
    orig = np.zeros((T, D), np.uint16)
    orig[bm] = (draft[bm].astype(np.int64) | low).astype(np.uint16)
    orig[~bm] = (((pb >> 7) << 15) | (perm_v[vr].astype(np.int64) << 7) | (pb & 0x7F)).astype(np.uint16)
    return draft, orig, perm, perm_v, ranks, vr


@pytest.mark.parametrize("T0", [1, 7, 64])
def test_kv_stream_roundtrip_and_layout(orc, T0):
    T, T_max = 64, 80
    vec = synth.kv_tensor(T, 1, D, 31 + T0)[:, 0, :]
    cc, vc = caps(T_max)
    spec, verif, tails = orc.kv_encode(vec, T0, K_KEEP, M, T_max, cc, vc)
    draft, orig, perm, perm_v, ranks, vranks = parse_kv(spec, verif, T, K_KEEP, M, T_max, cc, vc)
    assert (orig == vec).all(), "lossless reassembly"
    assert ((draft & ~vec) == 0).all(), "draft bits are a subset of the original bits"
    assert (orc.kv_decode(spec, T, D, K_KEEP, M, T_max, cc, vc) == draft).all()
    assert (orc.kv_decode(spec, T, D, K_KEEP, M, T_max, cc, vc, verif=verif) == vec).all()
    keep = orc.select(vec, K_KEEP)
    low = (1 << (7 - M)) - 1
    assert (draft == np.where(keep, vec & ~np.uint16(low), 0)).all()
    # the rank tables come from the first T0 tokens only
    e = (vec.astype(np.int64) >> 7) & 0xFF
    assert (perm == orc.rank_table(np.bincount(e[:T0][keep[:T0]], minlength=256))).all()
    assert (perm_v == orc.rank_table(np.bincount(e[:T0][~keep[:T0]], minlength=256))).all()
    # code bits in closed form from those tables
    rank = np.empty(256, np.int64); rank[perm] = np.arange(256)
    rank_v = np.empty(256, np.int64); rank_v[perm_v] = np.arange(256)
    assert int(tails[0]) == int((rank[e[keep]] + 1).sum())
    assert int(tails[1]) == int((rank_v[e[~keep]] + 1).sum())


def test_kv_capacity_error(orc):
    vec = synth.kv_tensor(16, 1, D, 3)[:, 0, :]
    with pytest.raises(orc.OracleError):
        orc.kv_encode(vec, 16, K_KEEP, M, 16, 10, 10)


def np_attention(q, K, V, scale, visible=None):
    qf = synth.f32_from_bf16(q).astype(np.float64)
    Kf = synth.f32_from_bf16(K).astype(np.float64)
    Vf = synth.f32_from_bf16(V).astype(np.float64)
    out = np.zeros((q.shape[0], Kf.shape[1]))
    for i in range(q.shape[0]):
        n = Kf.shape[0] if visible is None else visible[i]
        p = softmax(scale * (Kf[:n] @ qf[i]))
        out[i] = p @ Vf[:n]
    return out


def test_attention_textbook(orc):
    rng = np.random.default_rng(0)
    T = 200
    Kt = synth.kv_tensor(T, 1, D, 11)[:, 0, :]
    Vt = synth.kv_tensor(T, 1, D, 12)[:, 0, :]
    q = synth.bf16_from_f32(rng.standard_normal((6, D)).astype(np.float32))
    scale = 1 / np.sqrt(D)
    np.testing.assert_allclose(orc.attention(q, Kt, Vt, scale), np_attention(q, Kt, Vt, scale),
                               rtol=1e-12, atol=1e-12)
    vis = np.array([1, 5, 100, 199, 200, 37])
    np.testing.assert_allclose(orc.attention(q, Kt, Vt, scale, visible=vis),
                               np_attention(q, Kt, Vt, scale, visible=vis), rtol=1e-12, atol=1e-12)
    # one visible token: the output is that token's value row exactly
    one = orc.attention(q[:1], Kt, Vt, scale, visible=[1])
    assert (one[0] == synth.f32_from_bf16(Vt[0]).astype(np.float64)).all()
    # equal scores: the output is the mean of the values
    zero_q = np.zeros((1, D), np.uint16)
    np.testing.assert_allclose(orc.attention(zero_q, Kt, Vt, scale)[0],
                               synth.f32_from_bf16(Vt).astype(np.float64).mean(axis=0), rtol=1e-12)


def test_attention_keep_all_is_dense(orc):
    """keep = D with all mantissa bits: the draft KV is the KV itself."""
    T, T_max = 50, 64
    Kt = synth.kv_tensor(T, 1, D, 21)[:, 0, :]
    cc, vc = T_max * D * 16, 64
    spec, verif, _ = orc.kv_encode(Kt, T, D, 7, T_max, cc, vc)
    assert (orc.kv_decode(spec, T, D, D, 7, T_max, cc, vc) == Kt).all()


# ---------------------------------------------------------------- Cassandra-2
# OCP MX (cited by the paper; Cassandra review, section 3.2): one shared 8-bit
# exponent per 32 positions, here over the kept values of each group.

def mx_draft_reference(vec, keep, m):
    """The draft value of every position in fp64, from the definition: a kept
    value is sign * a * 2^(E - 127 - m) with E the largest max(e, 1) over the
    kept values of its 32 positions and a its significand (hidden bit
    included) shifted right by 7 - m + (E - max(e, 1)); pruned values are 0."""
    v = vec.astype(np.int64)
    s, e, f = v >> 15, (v >> 7) & 0xFF, v & 0x7F
    eff = np.maximum(e, 1)
    M = ((e > 0).astype(np.int64) << 7) | f
    T, Dd = vec.shape
    E = np.where(keep, eff, 0).reshape(T, Dd // 32, 32).max(axis=2).repeat(32, axis=1)
    shift = 7 - m + (E - eff)
    a = np.where(shift >= 8, 0, M >> np.minimum(shift, 7))
    val = np.where(s == 1, -1.0, 1.0) * a * np.exp2((E - 127 - m).astype(np.float64))
    return np.where(keep, val, 0.0), E, shift, M


def bf16_to_f64(b):
    with np.errstate(invalid="ignore"):  # NaN patterns stay NaN
        return synth.f32_from_bf16(b).astype(np.float64)


def parse_kv2(spec, verif, T, k, m, T_max, code_cap, vcode_cap):
    """Independent reader of one Cassandra-2 stream's regions (layout in the
    oracle header): returns (keep bitmap, shared exponents, fields, residue
    and pruned-code bit arrays, token offsets)."""
    def parts(sizes):
        out, pos = [], 0
        for n in sizes:
            out.append(pos)
            pos = (pos + n + 16 + 255) // 256 * 256
        return out
    so = parts([256, T_max * D // 8, T_max * D // 32, (T_max * k * (2 + m) + 7) // 8, 0])
    vo = parts([256, (code_cap + 7) // 8, T_max * (D - k), 8 * T_max, (vcode_cap + 7) // 8])
    bits = lambda a: np.unpackbits(a, bitorder="little").astype(np.int64)
    bm = bits(spec[so[1]:so[1] + T_max * D // 8])[: T * D].reshape(T, D).astype(bool)
    shexp = spec[so[2]:so[2] + T * D // 32].reshape(T, D // 32).astype(np.int64)
    fb = bits(spec[so[3]:so[3] + (T_max * k * (2 + m) + 7) // 8])[: T * k * (2 + m)].reshape(T * k, 2 + m)
    fields = (fb << np.arange(2 + m)).sum(axis=1)
    offs = verif[vo[3]:vo[3] + 8 * T_max].view("<u4")[: 2 * T].reshape(T, 2)
    return bm, shexp, fields, bits(verif[vo[1]:vo[2]]), verif[vo[2]:vo[2] + T * (D - k)], \
        bits(verif[vo[4]:]), offs, verif[vo[0]:vo[0] + 256]


@pytest.mark.parametrize("m", [0, 3, 7])
@pytest.mark.parametrize("k", [0, 38, 128])
def test_kv_c2_all_patterns(orc, m, k):
    """Every bf16 pattern (512 tokens x 128) round-trips exactly; the draft
    equals the MX value of the definition; the stream parses independently."""
    vec = synth.all_bf16_patterns(seed=5 + m + k).reshape(512, D)
    T = T_max = 512
    cc, vc = T_max * k * 264 + 64, T_max * (D - k) * 257 + 64
    spec, verif, tails = orc.kv_encode(vec, 64, k, m, T_max, cc, vc, fmt=orc.FMT_C2)
    exact = orc.kv_decode(spec, T, D, k, m, T_max, cc, vc, verif=verif, fmt=orc.FMT_C2)
    assert (exact == vec).all(), "lossless reassembly"
    draft = orc.kv_decode(spec, T, D, k, m, T_max, cc, vc, fmt=orc.FMT_C2)
    keep = orc.select(vec, k)
    ref, E, shift, M = mx_draft_reference(vec, keep, m)
    got = bf16_to_f64(draft)
    # values of 2^128 and up (shared exponent 255, the Inf/NaN binade) leave
    # the float range: there the draft keeps that binade's bit pattern (sign,
    # exponent 255), the pure-pattern reading of special values
    fin = np.abs(ref) < 2.0 ** 128
    assert np.array_equal(got[fin], ref[fin]), "draft = sign * a * 2^(E-127-m)"
    top = keep & ~fin
    assert (((draft[top] >> 7) & 0xFF) == 255).all()
    assert ((draft[top] >> 15) == (vec[top] >> 15)).all()
    assert (draft[~keep] == 0).all()
    # independent parse: bitmap, shared exponents, fields, residue bits
    bm, shexp, fields, rb, pb, vb, offs, perm_v = parse_kv2(spec, verif, T, k, m, T_max, cc, vc)
    assert (bm == keep).all()
    assert (shexp == E[:, ::32]).all()
    s = (vec.astype(np.int64) >> 15)[keep]
    a = np.where(shift >= 8, 0, M >> np.minimum(shift, 7))[keep]
    assert (fields == ((s << (m + 1)) | a)).all()
    d = (E - np.maximum((vec.astype(np.int64) >> 7) & 0xFF, 1))[keep]
    w = np.minimum(7 - m + d, 8)
    assert int(tails[0]) == int((d + 1 + w).sum()), "residue bits in closed form"
    assert int(rb[: int(tails[0])].sum()) == int(keep.sum()) + int(
        sum(bin(int(x) & ((1 << int(ww)) - 1)).count("1") for x, ww in zip(M[keep], w))), \
        "one unary terminator per kept value plus the low bits"
    # pruned side as in Cassandra-1: bytes and frozen-table codes
    e = (vec.astype(np.int64) >> 7) & 0xFF
    assert (perm_v == orc.rank_table(np.bincount(e[:64][~keep[:64]], minlength=256))).all()
    rank_v = np.empty(256, np.int64); rank_v[perm_v] = np.arange(256)
    assert int(tails[1]) == int((rank_v[e[~keep]] + 1).sum())
    pbytes = ((vec.astype(np.int64) >> 15) << 7 | (vec.astype(np.int64) & 0x7F))[~keep]
    assert (pb.astype(np.int64) == pbytes).all()
    # token offsets are prefix sums of each token's residue / code bits
    rbits = np.zeros((T, D), np.int64)
    rbits[keep] = d + 1 + w
    vbits = np.zeros((T, D), np.int64)
    vbits[~keep] = rank_v[e[~keep]] + 1
    assert (offs[:, 0] == np.concatenate([[0], np.cumsum(rbits.sum(axis=1))[:-1]])).all()
    assert (offs[:, 1] == np.concatenate([[0], np.cumsum(vbits.sum(axis=1))[:-1]])).all()


def test_kv_c2_capacity_error(orc):
    vec = synth.kv_tensor(16, 1, D, 4)[:, 0, :]
    with pytest.raises(orc.OracleError):
        orc.kv_encode(vec, 16, K_KEEP, M, 16, 10, 10_000, fmt=orc.FMT_C2)
