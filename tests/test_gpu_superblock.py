"""Format 4 (Cassandra-1 with superblock metadata) on the GPU against the CPU
oracle, through the C ABI: both streams byte for byte, exact reconstruction,
the draft bit for bit, the draft GEMV and verification GEMM within
1e-3 * sum|W||x| of the fp64 oracle; a tensor whose superblock offsets need
more than 16 bits is refused by the encoder."""
import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu

TOL = 1e-3
FMT = 4


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


def within(y_gpu, y_ref, absy):
    err = np.abs(y_gpu.astype(np.float64) - y_ref)
    bad = err > TOL * absy
    assert not bad.any(), f"{bad.sum()} outputs outside tolerance"


CASES = [
    # rows, cols, keep, mant, block
    (37, 4096, 1229, 3, 256),    # one superblock per row
    (24, 14336, 4301, 2, 256),   # 3.5 superblocks per row
    (64, 8192, 2458, 4, 128),    # 4 superblocks per row
    (5, 1024, 0, 3, 32),         # keep nothing
    (4, 2048, 2048, 7, 64),      # keep everything
    (3, 256, 77, 3, 256),        # one block
]


@pytest.mark.parametrize("case", CASES, ids=[str(c) for c in CASES])
def test_format4_against_oracle(gpu, orc, case):
    torch, cass = gpu
    R, C, k, m, B = case
    print("case", case, flush=True)
    w = synth.weight(R, C, 8000 + R + C + k, outlier_frac=0.01)
    spec_o, verif_o = orc.encode(w, k, m, block=B, fmt=FMT)
    enc = cass.encode(dev(torch, w), k, m, block=B, fmt=FMT)
    torch.cuda.synchronize()
    assert np.array_equal(enc.spec.cpu().numpy(), spec_o), "speculation stream"
    assert np.array_equal(enc.verif.cpu().numpy(), verif_o), "verification stream"
    X = synth.activations(5, C, 2, t0=9)
    Yr = orc.product(spec_o, X, verif=verif_o, threads=8)
    # the staged exact kernel (default) and the per-thread readers (option exact_path 1)
    for ep in (0, 1):
        cass.cass_set_option("exact_path", ep)
        try:
            out = torch.empty((R, C), dtype=torch.int16, device="cuda")
            cass.cass_reconstruct(enc.desc, out)
            torch.cuda.synchronize()
            assert np.array_equal(out.cpu().numpy().view(np.uint16), w), ("reconstruction", ep)
            cass.cass_draft_decode(enc.desc, out)
            torch.cuda.synchronize()
            assert np.array_equal(out.cpu().numpy().view(np.uint16), orc.draft_decode(spec_o)), \
                ("draft", ep)
            Y = torch.full((5, R), float("nan"), dtype=torch.float32, device="cuda")
            cass.cass_verify_gemm(enc.desc, dev(torch, X), Y)
            torch.cuda.synchronize()
            within(Y.cpu().numpy(), *Yr)
        finally:
            cass.cass_set_option("exact_path", 0)
    # the balanced kernel (default) and the per-thread one (option gemv_path 2)
    for path in (0, 2):
        cass.cass_set_option("gemv_path", path)
        try:
            for batch in (1, 2):
                x = synth.activations(batch, C, 2, t0=batch)
                y = torch.full((batch, R), float("nan"), dtype=torch.float32, device="cuda")
                cass.cass_draft_gemv(enc.desc, dev(torch, x), y)
                torch.cuda.synchronize()
                within(y.cpu().numpy(), *orc.product(spec_o, x, threads=8))
        finally:
            cass.cass_set_option("gemv_path", 0)


def test_format4_llama8b_gate_up_full_size(gpu, orc):
    """The Llama-3-8B-shaped gate|up matrix (28672 x 4096) at keep 0.3, m = 3:
    every byte of both streams, the exact reconstruction, and sampled rows of
    the draft GEMV and of the verification GEMM."""
    torch, cass = gpu
    w = np.concatenate([synth.weight(14336, 4096, 91_001, outlier_frac=0.01),
                        synth.weight(14336, 4096, 91_002, outlier_frac=0.01)])
    R, C = w.shape
    k = synth.keep_count(0.3, C)
    wd = dev(torch, w)
    enc = cass.encode(wd, k, 3, fmt=FMT)
    out = torch.empty_like(wd)
    cass.cass_reconstruct(enc.desc, out)
    X = synth.activations(5, C, 2, t0=6)
    Y = torch.full((5, R), float("nan"), dtype=torch.float32, device="cuda")
    cass.cass_verify_gemm(enc.desc, dev(torch, X), Y)
    torch.cuda.synchronize()
    assert torch.equal(out, wd)
    del out
    x = synth.activations(1, C, 2, t0=4)
    y = torch.full((1, R), float("nan"), dtype=torch.float32, device="cuda")
    cass.cass_draft_gemv(enc.desc, dev(torch, x), y)
    torch.cuda.synchronize()
    spec_o, verif_o = orc.encode(w, k, 3, fmt=FMT)
    assert np.array_equal(enc.spec.cpu().numpy(), spec_o)
    assert np.array_equal(enc.verif.cpu().numpy(), verif_o)
    rows = np.random.default_rng(0).choice(R, size=512, replace=False)
    yr, ar = orc.product_rows(spec_o, x, rows)
    within(y.cpu().numpy()[:, rows], yr, ar)
    Yr, Ar = orc.product_rows(spec_o, X, rows, verif=verif_o)
    within(Y.cpu().numpy()[:, rows], Yr, Ar)


def test_format4_offsets_past_16_bits_refused(gpu):
    torch, cass = gpu
    rng = np.random.default_rng(1)
    e = rng.permutation(np.repeat(np.arange(256), 16))
    w = ((e << 7) | rng.integers(0, 128, size=e.size)).astype(np.uint16).reshape(1, 4096)
    with pytest.raises(cass.CassError) as ex:
        cass.encode(dev(torch, w), 4096, 3, fmt=FMT)
    assert ex.value.status == cass.CASS_ERR_OVERFLOW
