"""The debug library (the same sources compiled with CASS_DEBUG: device bounds
checks on shared-memory staging, DMA alignment, tile writes and staged bit
positions) on the GPU: every hot-path call over valid inputs of several
shapes and formats leaves the check flags clear, and its results equal the
release library's bit for bit."""
import os

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


def run_path(torch, cass):
    """Weights (formats 1, 2, 4; a tall and a wide matrix) and a Cassandra-1
    KV cache through every hot-path call; returns the outputs on the host."""
    out = []
    for fmt in (1, 2, 4):
        for R, C in ((300, 4096), (40, 14336)):
            w = synth.weight(R, C, 70 + fmt + R, outlier_frac=0.01)
            k = synth.keep_count(0.3, C)
            enc = cass.encode(dev(torch, w), k, 3, fmt=fmt)
            x = dev(torch, synth.activations(1, C, 2, t0=fmt))
            X = dev(torch, synth.activations(5, C, 2, t0=fmt + 1))
            y = torch.empty((1, R), dtype=torch.float32, device="cuda")
            Y = torch.empty((5, R), dtype=torch.float32, device="cuda")
            o = torch.empty((R, C), dtype=torch.int16, device="cuda")
            cass.cass_draft_gemv(enc.desc, x, y)
            out.append(y.cpu().numpy())
            if fmt != 2:  # (format 2's verification sums partial products with atomics)
                cass.cass_verify_gemm(enc.desc, X, Y)
                out.append(Y.cpu().numpy())
            cass.cass_reconstruct(enc.desc, o)
            out.append(o.cpu().numpy())
            cass.cass_draft_decode(enc.desc, o)
            out.append(o.cpu().numpy())
    H, Hq, T = 8, 32, 3000
    Kt, Vt = synth.kv_tensor(T + 5, H, D, 77), synth.kv_tensor(T + 5, H, D, 78)
    cache = cass.KvCache(H, D, 38, 3, max_tokens=T + 16)
    cache.append(dev(torch, Kt[:T - 3]), dev(torch, Vt[:T - 3]))
    for t in range(T - 3, T):
        cache.append(dev(torch, Kt[t:t + 1]), dev(torch, Vt[t:t + 1]))
    q = dev(torch, synth.activations(Hq, D, 4, t0=T))
    ws = torch.empty(cass.cass_kv_attn_ws_bytes(cache.kv, 5, Hq) + 4096, dtype=torch.uint8,
                     device="cuda")
    o1 = torch.empty((Hq, D), dtype=torch.float32, device="cuda")
    cass.cass_kv_draft_attn(cache.kv, q, 1 / np.sqrt(D), o1, ws)
    out.append(o1.cpu().numpy())
    cache.append(dev(torch, Kt[T:T + 5]), dev(torch, Vt[T:T + 5]))
    qv = dev(torch, np.stack([synth.activations(Hq, D, 5, t0=T + i) for i in range(5)]))
    ov = torch.empty((5, Hq, D), dtype=torch.float32, device="cuda")
    cass.cass_kv_verify_attn(cache.kv, qv, 1 / np.sqrt(D), ov, ws)
    out.append(ov.cpu().numpy())
    out.append(cache.spec.cpu().numpy())
    out.append(cache.verif.cpu().numpy())
    torch.cuda.synchronize()
    return out


def test_debug_build_checks_stay_clear(gpu):
    torch, cass = gpu
    if not os.path.exists(cass.DEBUG_LIB_PATH):
        pytest.fail("libcassandra_debug.so is not built (python -m bit_level_weight_amd.build debug)")
    release = run_path(torch, cass)
    saved = (cass._lib, cass.LIB_PATH)
    try:
        cass._lib, cass.LIB_PATH = None, cass.DEBUG_LIB_PATH
        cass.lib()
        assert cass.cass_debug_flags() == 0  # (clears anything left over)
        debug = run_path(torch, cass)
        assert cass.cass_debug_flags() == 0
    finally:
        cass._lib, cass.LIB_PATH = saved
    assert len(debug) == len(release)
    for i, (a, b) in enumerate(zip(release, debug)):
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), i
