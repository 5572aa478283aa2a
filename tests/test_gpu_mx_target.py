"""Format 3 (Cassandra-2 with an MX-quantised target) on the GPU against the
CPU oracle, through the C ABI: both streams byte for byte, the reconstructed
target bit for bit (and equal to the oracle's definition of the target), the
draft bit for bit, and the draft GEMV and verification GEMM within
1e-3 * sum|W||x| of the fp64 oracle products (the verification GEMM's weights
being the quantised target)."""
import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu

TOL = 1e-3
FMT = 3


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


def host_u8(t):
    return t.cpu().numpy().view(np.uint8)


def host_u16(t):
    return t.cpu().numpy().view(np.uint16)


def within(y_gpu, y_ref, absy):
    err = np.abs(y_gpu.astype(np.float64) - y_ref)
    bad = err > TOL * absy
    assert not bad.any(), f"{bad.sum()} outputs outside tolerance"


CASES = [
    # rows, cols, keep, mant, block
    (1024, 2560, 768, 3, 256),   # Qwen3-4B width, keep 0.3
    (37, 4096, 1229, 3, 256),    # ragged rows
    (33, 1024, 307, 0, 256),     # sign only in the draft
    (8, 512, 512, 7, 256),       # keep everything
    (7, 1024, 0, 5, 128),        # keep nothing
    (16, 512, 205, 4, 32),       # smallest block
]


@pytest.mark.parametrize("case", CASES, ids=[str(c) for c in CASES])
def test_format3_against_oracle(gpu, orc, case):
    torch, cass = gpu
    R, C, k, m, B = case
    print("case", case, flush=True)
    w = synth.weight(R, C, 4000 + R + C + k, outlier_frac=0.01)
    spec_o, verif_o = orc.encode(w, k, m, block=B, fmt=FMT)
    enc = cass.encode(dev(torch, w), k, m, block=B, fmt=FMT)
    out = torch.empty((R, C), dtype=torch.int16, device="cuda")
    cass.cass_reconstruct(enc.desc, out)
    torch.cuda.synchronize()
    assert np.array_equal(host_u8(enc.spec), spec_o), "speculation stream"
    assert np.array_equal(host_u8(enc.verif), verif_o), "verification stream"
    assert np.array_equal(host_u16(out), orc.mx_target(w)), "target"
    cass.cass_draft_decode(enc.desc, out)
    torch.cuda.synchronize()
    assert np.array_equal(host_u16(out), orc.draft_decode(spec_o)), "draft"
    for batch in (1, 2):
        x = synth.activations(batch, C, 5, t0=batch)
        y = torch.full((batch, R), float("nan"), dtype=torch.float32, device="cuda")
        cass.cass_draft_gemv(enc.desc, dev(torch, x), y)
        torch.cuda.synchronize()
        within(y.cpu().numpy(), *orc.product(spec_o, x, threads=8))
    X = synth.activations(5, C, 5, t0=9)
    Y = torch.full((5, R), float("nan"), dtype=torch.float32, device="cuda")
    cass.cass_verify_gemm(enc.desc, dev(torch, X), Y)
    torch.cuda.synchronize()
    within(Y.cpu().numpy(), *orc.product(spec_o, X, verif=verif_o, threads=8))


def test_format3_all_bf16_patterns(gpu, orc):
    torch, cass = gpu
    w = synth.all_bf16_patterns(seed=17)
    for k, m in [(77, 3), (256, 7), (0, 0), (200, 5)]:
        spec_o, verif_o = orc.encode(w, k, m, block=64, fmt=FMT)
        enc = cass.encode(dev(torch, w), k, m, block=64, fmt=FMT)
        out = torch.empty((256, 256), dtype=torch.int16, device="cuda")
        cass.cass_reconstruct(enc.desc, out)
        torch.cuda.synchronize()
        assert np.array_equal(host_u8(enc.spec), spec_o), (k, m)
        assert np.array_equal(host_u8(enc.verif), verif_o), (k, m)
        assert np.array_equal(host_u16(out), orc.mx_target(w)), (k, m)


def test_format3_qwen3_4b_gate_up_full_size(gpu, orc):
    """The Qwen3-4B-shaped gate|up matrix (19456 x 2560) at keep 0.3, m = 3:
    every byte of both streams, the target, and every output of the batch-2
    draft GEMV and the N = 5 verification GEMM."""
    torch, cass = gpu
    w = np.concatenate([synth.weight(9728, 2560, 77_001), synth.weight(9728, 2560, 77_002)])
    R, C = w.shape
    k = synth.keep_count(0.3, C)
    enc = cass.encode(dev(torch, w), k, 3, fmt=FMT)
    out = torch.empty((R, C), dtype=torch.int16, device="cuda")
    cass.cass_reconstruct(enc.desc, out)
    x = synth.activations(2, C, 5, t0=3)
    y = torch.full((2, R), float("nan"), dtype=torch.float32, device="cuda")
    cass.cass_draft_gemv(enc.desc, dev(torch, x), y)
    X = synth.activations(5, C, 5, t0=11)
    Y = torch.full((5, R), float("nan"), dtype=torch.float32, device="cuda")
    cass.cass_verify_gemm(enc.desc, dev(torch, X), Y)
    torch.cuda.synchronize()
    spec_o, verif_o = orc.encode(w, k, 3, fmt=FMT)
    assert np.array_equal(host_u8(enc.spec), spec_o)
    assert np.array_equal(host_u8(enc.verif), verif_o)
    assert np.array_equal(host_u16(out), orc.mx_target(w))
    within(y.cpu().numpy(), *orc.product(spec_o, x, threads=8))
    within(Y.cpu().numpy(), *orc.product(spec_o, X, verif=verif_o, threads=8))
