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
