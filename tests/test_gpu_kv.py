"""GPU parity of the compressed KV cache against the CPU oracle, through the
C ABI, for Cassandra-1 (unary exponent codes) and Cassandra-2 (shared MX
exponent per 32 positions): stream regions byte for byte (one append, and
token-at-a-time appends after a first chunk), decode bit for bit, draft and
verification attention within tolerance of the fp64 oracle.

Attention tolerance (the pages fix none): |o - o_ref| <= 2e-3 * sum_t p_t |V_t|
+ 1e-6 per element, with p the oracle's softmax weights; the sum is obtained as
the oracle's attention of the same queries over |V|.
"""
import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu

D = 128


@pytest.fixture(scope="module")
def gpu():
    import torch
    import bit_level_weight_amd as cass
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    cass.lib()
    return torch, cass


def dev(torch, a):
    a = np.ascontiguousarray(a, dtype=np.uint16)
    return torch.from_numpy(a.view(np.int16)).cuda()


def make_kv(T, H, seed):
    return synth.kv_tensor(T, H, D, seed), synth.kv_tensor(T, H, D, seed + 1)


FMTS = [1, 2]


def check_regions(torch, cache, orc, Kt, Vt, T0, k, m, fmt=1):
    """Every stream region equals the oracle's encoding of that stream."""
    H = Kt.shape[1]
    p = cache.params
    spec = cache.spec.cpu().numpy()
    verif = cache.verif.cpu().numpy()
    ss, vs = cache.kv.spec_stream_bytes, cache.kv.verif_stream_bytes
    for h in range(H):
        for kind, X in ((0, Kt), (1, Vt)):
            s = 2 * h + kind
            so, vo, tails = orc.kv_encode(X[:, h, :], T0, k, m, p.max_tokens, p.code_cap_bits,
                                          p.vcode_cap_bits, fmt=fmt)
            assert np.array_equal(spec[s * ss:(s + 1) * ss], so), f"spec stream {s}"
            assert np.array_equal(verif[s * vs:(s + 1) * vs], vo), f"verif stream {s}"


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("T,H,k,m", [(300, 8, 38, 3), (1, 2, 38, 3), (77, 3, 0, 2),
                                     (64, 2, 128, 7), (130, 4, 64, 0)])
def test_kv_append_one_call(gpu, orc, T, H, k, m, fmt):
    torch, cass = gpu
    print("case", T, H, k, m, fmt, flush=True)
    Kt, Vt = make_kv(T, H, 100 + T + k)
    cache = cass.KvCache(H, D, k, m, max_tokens=T + 16, fmt=fmt)
    cache.append(dev(torch, Kt), dev(torch, Vt))
    torch.cuda.synchronize()
    assert cass.cass_kv_status(cache.kv) == (T, cass.CASS_KV_FLAG_TABLES)
    check_regions(torch, cache, orc, Kt, Vt, T, k, m, fmt)
    out = torch.empty((2, H, T, D), dtype=torch.int16, device="cuda")
    cass.cass_kv_decode(cache.kv, True, out)
    torch.cuda.synchronize()
    o = out.cpu().numpy().view(np.uint16)
    assert np.array_equal(o[0], Kt.transpose(1, 0, 2)) and np.array_equal(o[1], Vt.transpose(1, 0, 2))


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("k", [1, 38, 127])
def test_kv_select_ties(gpu, orc, fmt, k):
    """Vectors whose magnitudes repeat (four distinct keys, mixed signs) and a
    token whose keys are all equal: the top-k keeps ties by lower index, in the
    first append and in single-token appends (the one-launch path), and the
    regions equal the oracle's encoding."""
    torch, cass = gpu
    H, m, T0, T = 2, 3, 6, 10
    rng = np.random.default_rng(900 + k + fmt)
    mags = np.array([0x3F80, 0x3F00, 0x3E80, 0x3C00], dtype=np.uint16)  # 1, 1/2, 1/4, 2^-7

    def tensor():
        X = mags[rng.integers(0, 4, size=(T, H, D))]
        X = X | (rng.integers(0, 2, size=(T, H, D)).astype(np.uint16) << 15)
        X[3, 0, :] = 0x3F80
        X[8, 1, :] = 0xBF00
        return X.astype(np.uint16)

    Kt, Vt = tensor(), tensor()
    # (exponents first kept after the tables froze take long codes: room for them)
    cache = cass.KvCache(H, D, k, m, max_tokens=T + 4, fmt=fmt, code_cap_bits=(T + 4) * D * 260,
                         vcode_cap_bits=(T + 4) * D * 260)
    cache.append(dev(torch, Kt[:T0]), dev(torch, Vt[:T0]))
    for t in range(T0, T):
        cache.append(dev(torch, Kt[t:t + 1]), dev(torch, Vt[t:t + 1]))
    torch.cuda.synchronize()
    check_regions(torch, cache, orc, Kt, Vt, T0, k, m, fmt)


@pytest.mark.parametrize("fmt", FMTS)
def test_kv_token_at_a_time_equals_one_call(gpu, orc, fmt):
    """A first chunk of T0 tokens then single-token appends gives the bytes of
    one encoding with the tables of the first chunk."""
    torch, cass = gpu
    T, T0, H, k, m = 96, 40, 8, 38, 3
    Kt, Vt = make_kv(T, H, 7)
    cache = cass.KvCache(H, D, k, m, max_tokens=128, fmt=fmt)
    cache.append(dev(torch, Kt[:T0]), dev(torch, Vt[:T0]))
    for t in range(T0, T):
        cache.append(dev(torch, Kt[t:t + 1]), dev(torch, Vt[t:t + 1]))
    torch.cuda.synchronize()
    assert cache.tokens == T
    check_regions(torch, cache, orc, Kt, Vt, T0, k, m, fmt)
    out = torch.empty((2, H, T, D), dtype=torch.int16, device="cuda")
    cass.cass_kv_decode(cache.kv, False, out)
    torch.cuda.synchronize()
    p = cache.params
    so, _, _ = orc.kv_encode(Kt[:, 3, :], T0, k, m, p.max_tokens, p.code_cap_bits, p.vcode_cap_bits,
                             fmt=fmt)
    draft_ref = orc.kv_decode(so, T, D, k, m, p.max_tokens, p.code_cap_bits, p.vcode_cap_bits,
                              fmt=fmt)
    assert np.array_equal(out.cpu().numpy().view(np.uint16)[0, 3], draft_ref)


@pytest.mark.parametrize("fmt", FMTS)
def test_kv_overflow_flag(gpu, fmt):
    torch, cass = gpu
    Kt, Vt = make_kv(32, 2, 9)
    cache = cass.KvCache(2, D, 38, 3, max_tokens=64, code_cap_bits=100, vcode_cap_bits=100, fmt=fmt)
    cache.append(dev(torch, Kt), dev(torch, Vt))
    torch.cuda.synchronize()
    t, flags = cass.cass_kv_status(cache.kv)
    assert t == 32 and flags & cass.CASS_KV_FLAG_OVERFLOW


def attn_check(got, ref, bound):
    err = np.abs(got.astype(np.float64) - ref)
    tol = 2e-3 * bound + 1e-6
    assert (err <= tol).all(), f"worst ratio {(err / tol).max():.3g}"


def oracle_attention(orc, q_rows, Kh, Vh, scale, visible=None):
    out = orc.attention(q_rows, Kh, Vh, scale, visible)
    absV = Vh & np.uint16(0x7FFF)
    bound = orc.attention(q_rows, Kh, absV, scale, visible)
    return out, bound


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("T", [1, 200, 700])
def test_draft_and_verify_attention(gpu, orc, T, fmt):
    torch, cass = gpu
    H, Hq, k, m, nq = 8, 32, 38, 3, 5
    G = Hq // H
    Kt, Vt = make_kv(T + nq, H, 50 + T)
    cache = cass.KvCache(H, D, k, m, max_tokens=T + nq + 8, fmt=fmt)
    cache.append(dev(torch, Kt[:T]), dev(torch, Vt[:T]))
    scale = 1.0 / np.sqrt(D)
    q1 = synth.activations(Hq, D, 4, t0=T)
    ws = torch.empty(cass.cass_kv_attn_ws_bytes(cache.kv, nq, Hq) + 256, dtype=torch.uint8, device="cuda")
    out = torch.empty((Hq, D), dtype=torch.float32, device="cuda")
    cass.cass_kv_draft_attn(cache.kv, dev(torch, q1), scale, out, ws)
    torch.cuda.synchronize()
    p = cache.params
    got = out.cpu().numpy()
    for h in range(H):
        caps = (p.max_tokens, p.code_cap_bits, p.vcode_cap_bits)
        sk, _, _ = orc.kv_encode(Kt[:T, h, :], T, k, m, *caps, fmt=fmt)
        sv, _, _ = orc.kv_encode(Vt[:T, h, :], T, k, m, *caps, fmt=fmt)
        Kd = orc.kv_decode(sk, T, D, k, m, *caps, fmt=fmt)
        Vd = orc.kv_decode(sv, T, D, k, m, *caps, fmt=fmt)
        ref, bound = oracle_attention(orc, q1[h * G:(h + 1) * G], Kd, Vd, scale)
        attn_check(got[h * G:(h + 1) * G], ref, bound)
    # verification: append the nq drafted tokens, then attend causally on exact KV
    if T < nq:
        return
    cache.append(dev(torch, Kt[T:T + nq]), dev(torch, Vt[T:T + nq]))
    qv = np.stack([synth.activations(Hq, D, 5, t0=T + i) for i in range(nq)])
    outv = torch.empty((nq, Hq, D), dtype=torch.float32, device="cuda")
    ws = torch.empty(cass.cass_kv_attn_ws_bytes(cache.kv, nq, Hq) + 256, dtype=torch.uint8, device="cuda")
    cass.cass_kv_verify_attn(cache.kv, dev(torch, qv), scale, outv, ws)
    torch.cuda.synchronize()
    gotv = outv.cpu().numpy()
    Ttot = T + nq
    for h in range(H):
        for g in range(G):
            rows = qv[:, h * G + g, :]
            vis = [Ttot - nq + i + 1 for i in range(nq)]
            ref, bound = oracle_attention(orc, rows, Kt[:Ttot, h, :], Vt[:Ttot, h, :], scale, vis)
            attn_check(gotv[:, h * G + g, :], ref, bound)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("G", [1, 2, 3])
def test_draft_attention_fewer_query_rows(gpu, orc, G, fmt):
    """Draft attention with fewer than four query heads per KV head (one, two
    or three rows per chunk workgroup): the rows past the last are zero in the
    matrix-core product and write no partials."""
    torch, cass = gpu
    H, k, m, T = 4, 38, 3, 300
    Hq = H * G
    Kt, Vt = make_kv(T, H, 77 + G)
    cache = cass.KvCache(H, D, k, m, max_tokens=T + 8, fmt=fmt)
    cache.append(dev(torch, Kt), dev(torch, Vt))
    scale = 1.0 / np.sqrt(D)
    q1 = synth.activations(Hq, D, 4, t0=T + G)
    ws = torch.empty(cass.cass_kv_attn_ws_bytes(cache.kv, 1, Hq) + 256, dtype=torch.uint8, device="cuda")
    out = torch.empty((Hq, D), dtype=torch.float32, device="cuda")
    cass.cass_kv_draft_attn(cache.kv, dev(torch, q1), scale, out, ws)
    torch.cuda.synchronize()
    p = cache.params
    got = out.cpu().numpy()
    caps = (p.max_tokens, p.code_cap_bits, p.vcode_cap_bits)
    for h in range(H):
        sk, _, _ = orc.kv_encode(Kt[:, h, :], T, k, m, *caps, fmt=fmt)
        sv, _, _ = orc.kv_encode(Vt[:, h, :], T, k, m, *caps, fmt=fmt)
        Kd = orc.kv_decode(sk, T, D, k, m, *caps, fmt=fmt)
        Vd = orc.kv_decode(sv, T, D, k, m, *caps, fmt=fmt)
        ref, bound = oracle_attention(orc, q1[h * G:(h + 1) * G], Kd, Vd, scale)
        attn_check(got[h * G:(h + 1) * G], ref, bound)


@pytest.mark.parametrize("fmt", FMTS)
def test_draft_attention_uneven_tokens(gpu, orc, fmt):
    """Draft attention on tokens the grouped decoders cannot take whole: a first
    chunk whose keep bitmaps leave the first 32 positions empty (channels 0-31
    scaled down) and, appended after the rank tables froze, tokens whose
    exponents the first append never saw (long codes, short code windows)."""
    torch, cass = gpu
    H, Hq, k, m, T0, T = 2, 8, 38, 3, 200, 300
    G = Hq // H
    Kt, Vt = make_kv(T, H, 4242)
    Kf, Vf = synth.f32_from_bf16(Kt).copy(), synth.f32_from_bf16(Vt).copy()
    Kf[:100, :, :32] *= np.float32(1e-4)
    Vf[:100, :, :32] *= np.float32(1e-4)
    Kf[T0:] *= np.float32(2.0 ** -30)
    Vf[T0:] *= np.float32(2.0 ** 12)
    Kt, Vt = synth.bf16_from_f32(Kf), synth.bf16_from_f32(Vf)
    cap = T + 8
    cache = cass.KvCache(H, D, k, m, max_tokens=cap, code_cap_bits=cap * k * 64,
                         vcode_cap_bits=cap * (D - k) * 64, fmt=fmt)
    cache.append(dev(torch, Kt[:T0]), dev(torch, Vt[:T0]))
    cache.append(dev(torch, Kt[T0:]), dev(torch, Vt[T0:]))
    scale = 1.0 / np.sqrt(D)
    q1 = synth.activations(Hq, D, 4, t0=T)
    ws = torch.empty(cass.cass_kv_attn_ws_bytes(cache.kv, 1, Hq) + 256, dtype=torch.uint8, device="cuda")
    out = torch.empty((Hq, D), dtype=torch.float32, device="cuda")
    cass.cass_kv_draft_attn(cache.kv, dev(torch, q1), scale, out, ws)
    torch.cuda.synchronize()
    p = cache.params
    got = out.cpu().numpy()
    caps = (p.max_tokens, p.code_cap_bits, p.vcode_cap_bits)
    for h in range(H):
        sk, _, _ = orc.kv_encode(Kt[:, h, :], T0, k, m, *caps, fmt=fmt)
        sv, _, _ = orc.kv_encode(Vt[:, h, :], T0, k, m, *caps, fmt=fmt)
        Kd = orc.kv_decode(sk, T, D, k, m, *caps, fmt=fmt)
        Vd = orc.kv_decode(sv, T, D, k, m, *caps, fmt=fmt)
        assert not (Kd[:100, :32].any() or Vd[:100, :32].any()), "first keep word not empty"
        ref, bound = oracle_attention(orc, q1[h * G:(h + 1) * G], Kd, Vd, scale)
        attn_check(got[h * G:(h + 1) * G], ref, bound)


@pytest.mark.parametrize("fmt,T", [(1, 16640), (2, 16640), (1, 33000), (2, 66000)])
def test_attention_long_context(gpu, orc, fmt, T):
    """Draft and verification attention at contexts where the chunk merge uses
    its whole structure: 16640 tokens are 130 chunks of 128 (past 64 chunks,
    every merge wave carries chunk maxima and sums); past 512 chunks the
    merge's strided loop runs a second pass: 66000 + 5 tokens in chunks of 128,
    33000 + 5 in the 64-token chunks of the Cassandra-1 verification kernel.
    All 32 query heads are checked against the oracle's decode plus fp64
    attention."""
    torch, cass = gpu
    H, Hq, k, m, nq = 8, 32, 38, 3, 5
    G = Hq // H
    print("case", fmt, T, flush=True)
    Kt, Vt = make_kv(T + nq, H, 9000 + T + fmt)
    cache = cass.KvCache(H, D, k, m, max_tokens=T + nq + 8, fmt=fmt)
    cache.append(dev(torch, Kt[:T]), dev(torch, Vt[:T]))
    scale = 1.0 / np.sqrt(D)
    q1 = synth.activations(Hq, D, 4, t0=T)
    ws = torch.empty(cass.cass_kv_attn_ws_bytes(cache.kv, nq, Hq) + 256, dtype=torch.uint8,
                     device="cuda")
    out = torch.empty((Hq, D), dtype=torch.float32, device="cuda")
    cass.cass_kv_draft_attn(cache.kv, dev(torch, q1), scale, out, ws)
    cache.append(dev(torch, Kt[T:T + nq]), dev(torch, Vt[T:T + nq]))
    qv = np.stack([synth.activations(Hq, D, 5, t0=T + i) for i in range(nq)])
    outv = torch.empty((nq, Hq, D), dtype=torch.float32, device="cuda")
    wsv = torch.empty(cass.cass_kv_attn_ws_bytes(cache.kv, nq, Hq) + 256, dtype=torch.uint8,
                      device="cuda")
    cass.cass_kv_verify_attn(cache.kv, dev(torch, qv), scale, outv, wsv)
    torch.cuda.synchronize()
    got, gotv = out.cpu().numpy(), outv.cpu().numpy()
    # the same call again gives the same bits (workgroups that share a CU
    # with another one included: more than 256 workgroups here)
    for _ in range(2):
        again = torch.empty_like(outv)
        cass.cass_kv_verify_attn(cache.kv, dev(torch, qv), scale, again, wsv)
        torch.cuda.synchronize()
        assert np.array_equal(again.cpu().numpy(), gotv), "verification attention not deterministic"
    p = cache.params
    caps = (p.max_tokens, p.code_cap_bits, p.vcode_cap_bits)
    Ttot = T + nq
    for h in range(H):
        sk, _, _ = orc.kv_encode(Kt[:T, h, :], T, k, m, *caps, fmt=fmt)
        sv, _, _ = orc.kv_encode(Vt[:T, h, :], T, k, m, *caps, fmt=fmt)
        Kd = orc.kv_decode(sk, T, D, k, m, *caps, fmt=fmt)
        Vd = orc.kv_decode(sv, T, D, k, m, *caps, fmt=fmt)
        ref, bound = oracle_attention(orc, q1[h * G:(h + 1) * G], Kd, Vd, scale)
        attn_check(got[h * G:(h + 1) * G], ref, bound)
        # the G x nq verification rows of this KV head in one oracle call
        rows = np.concatenate([qv[:, h * G + g, :] for g in range(G)])
        vis = [Ttot - nq + i + 1 for i in range(nq)] * G
        ref, bound = oracle_attention(orc, rows, Kt[:Ttot, h, :], Vt[:Ttot, h, :], scale, vis)
        gv = np.concatenate([gotv[:, h * G + g, :] for g in range(G)])
        attn_check(gv, ref, bound)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("caps", [None, (2600, 2600)])
def test_kv_append_few_tokens_one_launch(gpu, orc, fmt, caps):
    """Appends of up to 16 tokens run as one launch (one wave per stream); the
    regions, tails, flags and token counts equal those of the five-launch path
    step by step, with and without code capacities that overflow; and the
    result equals the oracle's encoding."""
    torch, cass = gpu
    H, k, m, T0 = 4, 38, 3, 40
    sizes = [1, 5, 3, 16, 17, 2]
    T = T0 + sum(sizes)
    Kt, Vt = make_kv(T, H, 321 + fmt)
    kw = {} if caps is None else dict(code_cap_bits=caps[0], vcode_cap_bits=caps[1])
    a = cass.KvCache(H, D, k, m, max_tokens=T + 8, fmt=fmt, **kw)
    b = cass.KvCache(H, D, k, m, max_tokens=T + 8, fmt=fmt, **kw)
    a.append(dev(torch, Kt[:T0]), dev(torch, Vt[:T0]))
    b.append(dev(torch, Kt[:T0]), dev(torch, Vt[:T0]))
    t = T0
    for n in sizes:
        a.append(dev(torch, Kt[t:t + n]), dev(torch, Vt[t:t + n]))
        cass.cass_set_option("kv_append_path", 1)
        try:
            b.append(dev(torch, Kt[t:t + n]), dev(torch, Vt[t:t + n]))
        finally:
            cass.cass_set_option("kv_append_path", 0)
        t += n
        torch.cuda.synchronize()
        assert torch.equal(a.spec, b.spec) and torch.equal(a.verif, b.verif), n
        assert torch.equal(a.state, b.state), n
    if caps is None:
        check_regions(torch, a, orc, Kt, Vt, T0, k, m, fmt)
    else:
        assert cass.cass_kv_status(a.kv)[1] & cass.CASS_KV_FLAG_OVERFLOW
