"""The self-speculative step (k = 4 draft passes, rollback of the drafted
tokens, one verification pass of k + 1 tokens, acceptance) on a two-layer
stack, against the CPU oracle through the C ABI; and truncation of the
compressed KV cache, which the step's rollback and acceptance use.

What is checked after a step: every layer's cache holds exactly the oracle's
encoding of the prefix plus the verified tokens the acceptance keeps (byte for
byte, both streams); every draft GEMV and verification GEMM output is within
1e-3 * sum|W||x| of the fp64 oracle product; the last draft pass's attention
matches the oracle over the zero-filled draft K, V of the prefix and the four
drafted tokens, and the verification attention the oracle over the exact K, V
of the prefix and the five verified tokens (causal), both within
2e-3 * sum_t p_t |V_t| + 1e-6.  The step captured in a HIP graph gives the
eager step's outputs on every replay (bit for bit, but for the last bits of
the verification GEMM, whose column splits meet in float atomics) and leaves
the caches as it found them.
"""
import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu

D = 128
TOL = 1e-3


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


def host16(t):
    return t.cpu().numpy().view(np.uint16)


def regions_equal(cache, orc, Kt, Vt, T0, k, m, fmt):
    """Every stream region of the cache equals the oracle's encoding of the
    tokens Kt, Vt [T, H, D] with rank tables from the first T0."""
    H = Kt.shape[1]
    p = cache.params
    spec, verif = cache.spec.cpu().numpy(), cache.verif.cpu().numpy()
    ss, vs = cache.kv.spec_stream_bytes, cache.kv.verif_stream_bytes
    st = cache.state.cpu().numpy().view(np.uint64)
    for h in range(H):
        for kind, X in ((0, Kt), (1, Vt)):
            s = 2 * h + kind
            so, vo, tails = orc.kv_encode(X[:, h, :], T0, k, m, p.max_tokens, p.code_cap_bits,
                                          p.vcode_cap_bits, fmt=fmt)
            assert np.array_equal(spec[s * ss:(s + 1) * ss], so), f"spec stream {s}"
            assert np.array_equal(verif[s * vs:(s + 1) * vs], vo), f"verif stream {s}"
            assert tuple(st[2 + 2 * s:4 + 2 * s]) == tuple(tails), f"tails of stream {s}"
    assert int(st[0]) == Kt.shape[0]


# ----------------------------------------------------------------- truncation


@pytest.mark.parametrize("fmt", [1, 2])
def test_truncate_then_append_equals_appending_kept(gpu, orc, fmt):
    """Tokens appended and then dropped leave no trace: the cache equals the
    oracle's encoding of the kept tokens only, whether the dropped tokens came
    in one call or one at a time, and whether the cut falls inside a call."""
    torch, cass = gpu
    T, T0, H, k, m = 90, 40, 4, 38, 3
    Kt, Vt = synth.kv_tensor(T, H, D, 21), synth.kv_tensor(T, H, D, 22)
    Jk, Jv = synth.kv_tensor(12, H, D, 77), synth.kv_tensor(12, H, D, 78)
    cache = cass.KvCache(H, D, k, m, max_tokens=128, fmt=fmt)
    cache.append(dev(torch, Kt[:T0]), dev(torch, Vt[:T0]))
    cache.append(dev(torch, np.concatenate([Kt[T0:T0 + 2], Jk[:5]])),
                 dev(torch, np.concatenate([Vt[T0:T0 + 2], Jv[:5]])))
    cache.truncate(T0 + 2)  # the cut inside the last call
    for t in range(T0 + 2, T0 + 6):
        cache.append(dev(torch, Kt[t:t + 1]), dev(torch, Vt[t:t + 1]))
    for i in range(5, 9):
        cache.append(dev(torch, Jk[i:i + 1]), dev(torch, Jv[i:i + 1]))
    cache.truncate(T0 + 6)
    torch.cuda.synchronize()
    regions_equal(cache, orc, Kt[:T0 + 6], Vt[:T0 + 6], T0, k, m, fmt)
    cache.append(dev(torch, Kt[T0 + 6:]), dev(torch, Vt[T0 + 6:]))
    torch.cuda.synchronize()
    assert cass.cass_kv_status(cache.kv) == (T, cass.CASS_KV_FLAG_TABLES)
    regions_equal(cache, orc, Kt, Vt, T0, k, m, fmt)
    # no-op and out-of-range requests
    cache.truncate(T)
    with pytest.raises(cass.CassError):
        cache.truncate(T + 1)
    with pytest.raises(cass.CassError):
        cache.truncate(-1)


@pytest.mark.parametrize("fmt", [1, 2])
def test_truncate_reopens_overflowed_stream(gpu, orc, fmt):
    """Code capacities that hold the kept tokens but not the dropped ones
    (past the first): the overflow closes the streams, truncation to the
    prefix reopens them, and the kept
    tokens' bytes equal the oracle's with the same capacities (the overflow
    flag stays raised)."""
    torch, cass = gpu
    T, T0, H, k, m = 60, 40, 2, 38, 3
    Kt, Vt = synth.kv_tensor(T, H, D, 31), synth.kv_tensor(T, H, D, 32)
    Jk, Jv = synth.kv_tensor(64, H, D, 33), synth.kv_tensor(64, H, D, 34)
    big = cass.KvCache(H, D, k, m, max_tokens=T + 64, fmt=fmt)
    # capacities that hold the kept tokens, and the first dropped token after
    # the prefix, in every stream
    caps_s, caps_v = 0, 0
    for h in range(H):
        for X, J in ((Kt, Jk), (Vt, Jv)):
            for toks in (X, np.concatenate([X[:T0], J[:1]])):
                _, _, tails = orc.kv_encode(toks[:, h, :], T0, k, m, big.params.max_tokens,
                                            big.params.code_cap_bits, big.params.vcode_cap_bits,
                                            fmt=fmt)
                caps_s, caps_v = max(caps_s, int(tails[0])), max(caps_v, int(tails[1]))
    del big
    cache = cass.KvCache(H, D, k, m, max_tokens=T + 64, code_cap_bits=caps_s,
                         vcode_cap_bits=caps_v, fmt=fmt)
    cache.append(dev(torch, Kt[:T0]), dev(torch, Vt[:T0]))
    cache.append(dev(torch, Jk), dev(torch, Jv))  # far past the capacities
    torch.cuda.synchronize()
    _, flags = cass.cass_kv_status(cache.kv)
    assert flags & cass.CASS_KV_FLAG_OVERFLOW
    cache.truncate(T0)
    cache.append(dev(torch, Kt[T0:]), dev(torch, Vt[T0:]))
    torch.cuda.synchronize()
    regions_equal(cache, orc, Kt, Vt, T0, k, m, fmt)
    _, flags = cass.cass_kv_status(cache.kv)
    assert flags & cass.CASS_KV_FLAG_OVERFLOW


# ---------------------------------------------------------- the composed step


HIDDEN, FFN, H, HQ = 1024, 2048, 2, 8
SHAPES = {"qkv": ((HQ + 2 * H) * D, HIDDEN), "o": (HIDDEN, HQ * D), "gu": (2 * FFN, HIDDEN),
          "down": (HIDDEN, FFN)}
MATS = ("qkv", "o", "gu", "down")


def stack_inputs(nl, T0, fmt, keep=0.3, mant=3):
    layers = [{m: synth.weight(*SHAPES[m], seed=9000 + 10 * li + j, outlier_frac=0.01)
               for j, m in enumerate(MATS)} for li in range(nl)]
    kvs = [(synth.kv_tensor(T0, H, D, 9500 + 2 * li), synth.kv_tensor(T0, H, D, 9501 + 2 * li))
           for li in range(nl)]
    k4 = 4
    ins = {"x": {m: synth.activations(k4 + 1, SHAPES[m][1], 2, t0=50 + j) for j, m in enumerate(MATS)},
           "q": synth.activations((k4 + 1) * HQ, D, 4, t0=70).reshape(k4 + 1, HQ, D),
           "k_new": synth.kv_tensor(k4 + 1, H, D, 9601), "v_new": synth.kv_tensor(k4 + 1, H, D, 9602),
           "k_draft": synth.kv_tensor(k4, H, D, 9603), "v_draft": synth.kv_tensor(k4, H, D, 9604)}
    return layers, kvs, ins


def build_step(torch, cass, layers, kvs, ins, T0, fmt, kkeep=38, mant=3, max_tokens=None):
    from bit_level_weight_amd.spec_step import SpecStep
    enc = [{m: cass.encode(dev(torch, w[m]), synth.keep_count(0.3, w[m].shape[1]), 3, fmt=fmt)
            for m in MATS} for w in layers]
    caches = []
    for K, V in kvs:
        c = cass.KvCache(H, D, kkeep, mant, max_tokens=max_tokens or T0 + 16, fmt=fmt)
        c.append(dev(torch, K), dev(torch, V))
        caches.append(c)
    dins = {"x": {m: dev(torch, ins["x"][m]) for m in MATS}}
    for n in ("q", "k_new", "v_new", "k_draft", "v_draft"):
        dins[n] = dev(torch, ins[n])
    return SpecStep(enc, caches, HQ, k=4, inputs=dins), enc, caches


@pytest.mark.parametrize("fmt", [1, 2])
def test_spec_step_against_oracle(gpu, orc, fmt):
    torch, cass = gpu
    nl, T0, accepted, kk, mant = 2, 300, 2, 38, 3
    layers, kvs, ins = stack_inputs(nl, T0, fmt)
    step, enc, caches = build_step(torch, cass, layers, kvs, ins, T0, fmt)
    assert step.step(accepted) == accepted + 1
    torch.cuda.synchronize()
    assert step.tokens() == T0 + 1 + accepted
    scale = 1.0 / np.sqrt(D)
    G = HQ // H
    for li in range(nl):
        print("layer", li, flush=True)
        K, V = kvs[li]
        # the cache: prefix + the verified tokens the acceptance keeps
        keepK = np.concatenate([K, ins["k_new"][:accepted + 1]])
        keepV = np.concatenate([V, ins["v_new"][:accepted + 1]])
        regions_equal(caches[li], orc, keepK, keepV, T0, kk, mant, fmt)
        # products
        for m in MATS:
            kept = synth.keep_count(0.3, SHAPES[m][1])
            spec_o, verif_o = orc.encode(layers[li][m], kept, 3, fmt=fmt)
            y, absy = orc.product(spec_o, ins["x"][m][:4], threads=8)
            got = step.y_draft[li][m].cpu().numpy()
            assert (np.abs(got - y) <= TOL * absy).all(), f"draft {m}"
            Y, absY = orc.product(spec_o, ins["x"][m], verif=verif_o, threads=8)
            got = step.y_ver[li][m].cpu().numpy()
            assert (np.abs(got - Y) <= TOL * absY).all(), f"verify {m}"
        # attention of the last draft pass: prefix + the four drafted tokens, draft data
        p = caches[li].params
        caps = (p.max_tokens, p.code_cap_bits, p.vcode_cap_bits)
        Kd_all = np.concatenate([K, ins["k_draft"]])
        Vd_all = np.concatenate([V, ins["v_draft"]])
        Tn = T0 + 4
        got_d = step.a_draft[li].cpu().numpy()[3]
        got_v = step.a_ver[li].cpu().numpy()
        Ke = np.concatenate([K, ins["k_new"]])
        Ve = np.concatenate([V, ins["v_new"]])
        for h in range(H):
            sk, _, _ = orc.kv_encode(Kd_all[:, h, :], T0, kk, mant, *caps, fmt=fmt)
            sv, _, _ = orc.kv_encode(Vd_all[:, h, :], T0, kk, mant, *caps, fmt=fmt)
            Kd = orc.kv_decode(sk, Tn, D, kk, mant, *caps, fmt=fmt)
            Vd = orc.kv_decode(sv, Tn, D, kk, mant, *caps, fmt=fmt)
            q = ins["q"][3, h * G:(h + 1) * G]
            ref = orc.attention(q, Kd, Vd, scale)
            bound = orc.attention(q, Kd, Vd & np.uint16(0x7FFF), scale)
            assert (np.abs(got_d[h * G:(h + 1) * G] - ref) <= 2e-3 * bound + 1e-6).all(), \
                f"draft attention layer {li} head {h}"
            Tv = T0 + 5
            vis = [Tv - 5 + i + 1 for i in range(5)]
            for g in range(G):
                rows = ins["q"][:, h * G + g, :]
                ref = orc.attention(rows, Ke[:, h, :], Ve[:, h, :], scale, vis)
                bound = orc.attention(rows, Ke[:, h, :], Ve[:, h, :] & np.uint16(0x7FFF), scale, vis)
                assert (np.abs(got_v[:, h * G + g] - ref) <= 2e-3 * bound + 1e-6).all(), \
                    f"verify attention layer {li} head {h}"


def test_spec_step_graph_replays_eager(gpu):
    """The step in a HIP graph: every replay gives the eager outputs (bit for
    bit where the kernels are deterministic) and returns the caches to their
    starting bytes; eager work runs between the replays."""
    torch, cass = gpu
    nl, T0, fmt = 2, 700, 1
    layers, kvs, ins = stack_inputs(nl, T0, fmt)
    step, enc, caches = build_step(torch, cass, layers, kvs, ins, T0, fmt)
    torch.cuda.synchronize()
    start = [(c.spec.clone(), c.verif.clone(), c.state.clone()) for c in caches]

    def outputs():
        # (outputs of deterministic kernels, verification GEMM outputs)
        out, ver = [], []
        for li in range(nl):
            out += [step.y_draft[li][m].clone() for m in MATS]
            ver += [step.y_ver[li][m].clone() for m in MATS]
            out += [step.a_draft[li].clone(), step.a_ver[li].clone()]
        return out, ver

    step.step(0, keep=False)
    torch.cuda.synchronize()
    ref = outputs()
    for c, (s0, v0, t0) in zip(caches, start):
        assert torch.equal(c.spec, s0) and torch.equal(c.verif, v0) and torch.equal(c.state, t0)
    g = step.capture()
    assert step.tokens() == T0
    for r in range(3):
        for li in range(nl):  # eager work between replays: the outputs poisoned
            for m in MATS:
                step.y_draft[li][m].fill_(float("nan"))
                step.y_ver[li][m].fill_(float("nan"))
            step.a_draft[li].fill_(float("nan"))
            step.a_ver[li].fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = outputs()
        assert all(torch.equal(a, b) for a, b in zip(got[0], ref[0])), f"replay {r}"
        # the verification GEMM adds the partial sums of its column splits with
        # float atomics, so its last bits follow the order they land in
        for a, b in zip(got[1], ref[1]):
            assert ((a - b).abs() <= 1e-5 * (a.abs() + b.abs()) + 1e-6).all(), f"replay {r}"
        for c, (s0, v0, t0) in zip(caches, start):
            assert torch.equal(c.spec, s0) and torch.equal(c.verif, v0) and \
                torch.equal(c.state, t0), f"caches after replay {r}"
