"""The allocation-free draft attention (cass_kv_draft_attn_static) against the
workspace entry point (cass_kv_draft_attn) through the C ABI: two calls in a
row, the second over a smaller cache, each bit-equal to the workspace call on
the same inputs (the two share their kernels), and the size limit refused
before any launch."""
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


def cache_of(torch, cass, T, H, fmt, seed):
    Kt, Vt = synth.kv_tensor(T, H, D, seed), synth.kv_tensor(T, H, D, seed + 1)
    cache = cass.KvCache(H, D, 38, 3, max_tokens=T + 8, fmt=fmt)
    cache.append(dev(torch, Kt), dev(torch, Vt))
    return cache


def test_static_draft_attention_matches_workspace_call(gpu):
    torch, cass = gpu
    cases = [(9000, 8, 32, 1, 11), (700, 4, 8, 2, 12)]  # second: fewer tokens and heads
    for T, H, Hq, fmt, seed in cases:
        print("case", T, H, Hq, fmt, flush=True)
        cache = cache_of(torch, cass, T, H, fmt, 500 + seed)
        q = dev(torch, synth.activations(Hq, D, 4, t0=seed))
        ws = torch.empty(cass.cass_kv_attn_ws_bytes(cache.kv, 1, Hq), dtype=torch.uint8,
                         device="cuda")
        o_ws = torch.full((Hq, D), float("nan"), dtype=torch.float32, device="cuda")
        o_st = torch.full((Hq, D), float("nan"), dtype=torch.float32, device="cuda")
        cass.cass_kv_draft_attn(cache.kv, q, 1 / np.sqrt(D), o_ws, ws)
        cass.cass_kv_draft_attn_static(cache.kv, q, 1 / np.sqrt(D), o_st)
        torch.cuda.synchronize()
        assert torch.isfinite(o_ws).all()
        assert torch.equal(o_ws, o_st), (T, H, Hq, fmt)


def test_static_draft_attention_refuses_oversize(gpu):
    torch, cass = gpu
    # a cache whose partials would need more than the fixed scratch holds
    p = cass.CassKvParams(8, D, 38, 3, 300_000, 300_000 * 38 * 8, 300_000 * 90 * 8, 1)
    kv = cass.CassKv()
    kv.p = p
    kv.spec, kv.verif, kv.state = 0x100000, 0x200000, 0x300000
    kv.tokens = 300_000
    q = torch.zeros((32, D), dtype=torch.int16, device="cuda")
    o = torch.zeros((32, D), dtype=torch.float32, device="cuda")
    with pytest.raises(cass.CassError) as e:
        cass.cass_kv_draft_attn_static(kv, q, 1.0, o)
    assert e.value.status == cass.CASS_ERR_CAPACITY
