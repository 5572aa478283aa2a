"""GPU parity: the HIP library against the CPU oracle, through the C ABI.

  * encoded streams: byte for byte;
  * draft decode and reconstruction: bit for bit;
  * draft GEMV and verification GEMM (fp32 accumulation) against the oracle's
    fp64 products: |y - y_ref| <= 1e-3 * sum_j |W'[n][j]| |x[j]| per element.
Inputs are the seeded synthetic tensors of the workloads.
"""
import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu

TOL = 1e-3


@pytest.fixture(scope="module")
def gpu():
    import torch
    import bit_level_weight_amd as cass
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    cass.lib()
    return torch, cass


@pytest.fixture
def opt(gpu):
    """Sets library code-path options for one test and restores the defaults."""
    torch, cass = gpu
    names = []

    def set_option(name, value):
        cass.cass_set_option(name, value)
        names.append(name)
    yield set_option
    for n in names:
        cass.cass_set_option(n, 0)


def dev(torch, a):
    a = np.ascontiguousarray(a, dtype=np.uint16)
    return torch.from_numpy(a.view(np.int16)).cuda()


def host_u8(t):
    return t.cpu().numpy().view(np.uint8)


def host_u16(t):
    return t.cpu().numpy().view(np.uint16)


def check_product(y_gpu, y_ref, absy):
    err = np.abs(y_gpu.astype(np.float64) - y_ref)
    bound = TOL * absy
    bad = err > bound
    assert not bad.any(), (f"{bad.sum()} outputs outside tolerance; worst ratio "
                           f"{(err / np.maximum(bound, 1e-300)).max():.3g}")


CASES = [
    # rows, cols, keep, mant, block, format
    (1024, 1024, 512, 3, 256, 1),   # the small worked configuration
    (37, 4096, 1229, 3, 256, 1),    # ragged row count, keep 0.3
    (64, 14336, 4301, 2, 256, 1),   # long rows
    (5, 1024, 0, 3, 256, 1),        # keep nothing
    (5, 1024, 1024, 7, 256, 1),     # keep everything, full mantissa
    (16, 512, 205, 0, 32, 1),       # sign only, smallest block
    (16, 512, 205, 7, 64, 1),
    (1, 32, 1, 4, 32, 1),           # single word
    (1024, 2560, 768, 3, 256, 2),   # Cassandra-2
    (33, 1024, 307, 0, 256, 2),
    (8, 512, 512, 7, 256, 2),
    (7, 1024, 0, 5, 128, 2),
]


def make_w(R, C, seed):
    w = synth.weight(R, C, seed, outlier_frac=0.01)
    if R > 2 and C >= 64:
        w[:, C // 2: C // 2 + 16] = w[:, 0:16]  # ties at many thresholds
    return w


@pytest.mark.parametrize("case", CASES, ids=[str(c) for c in CASES])
def test_encode_decode_bit_exact(gpu, orc, case):
    torch, cass = gpu
    R, C, k, m, B, fmt = case
    print("case", case, flush=True)
    w = make_w(R, C, 1000 + R + C + k)
    spec_o, verif_o = orc.encode(w, k, m, block=B, fmt=fmt)
    wd = dev(torch, w)
    enc = cass.encode(wd, k, m, block=B, fmt=fmt)
    torch.cuda.synchronize()
    spec_g, verif_g = host_u8(enc.spec), host_u8(enc.verif)
    assert spec_g.size == spec_o.size and verif_g.size == verif_o.size
    assert np.array_equal(spec_g, spec_o), f"spec differs at {np.flatnonzero(spec_g != spec_o)[:8]}"
    assert np.array_equal(verif_g, verif_o), f"verif differs at {np.flatnonzero(verif_g != verif_o)[:8]}"
    out = torch.empty((R, C), dtype=torch.int16, device="cuda")
    cass.cass_reconstruct(enc.desc, out)
    torch.cuda.synchronize()
    assert np.array_equal(host_u16(out), w)
    cass.cass_draft_decode(enc.desc, out)
    torch.cuda.synchronize()
    assert np.array_equal(host_u16(out), orc.draft_decode(spec_o))


def test_all_bf16_patterns_gpu(gpu, orc):
    torch, cass = gpu
    w = synth.all_bf16_patterns(seed=3)
    for fmt in (1, 2):
        for k, m in [(77, 3), (256, 7), (0, 0), (200, 5)]:
            spec_o, verif_o = orc.encode(w, k, m, block=64, fmt=fmt)
            enc = cass.encode(dev(torch, w), k, m, block=64, fmt=fmt)
            out = torch.empty((256, 256), dtype=torch.int16, device="cuda")
            cass.cass_reconstruct(enc.desc, out)
            torch.cuda.synchronize()
            assert np.array_equal(host_u8(enc.spec), spec_o), (fmt, k, m)
            assert np.array_equal(host_u8(enc.verif), verif_o), (fmt, k, m)
            assert np.array_equal(host_u16(out), w), (fmt, k, m)
            cass.cass_draft_decode(enc.desc, out)
            torch.cuda.synchronize()
            assert np.array_equal(host_u16(out), orc.draft_decode(spec_o)), (fmt, k, m)


def test_encode_is_deterministic(gpu):
    torch, cass = gpu
    w = dev(torch, make_w(300, 4096, 5))
    a = cass.encode(w, 1229, 3)
    b = cass.encode(w, 1229, 3)
    torch.cuda.synchronize()
    assert torch.equal(a.spec, b.spec) and torch.equal(a.verif, b.verif)


PRODUCT_CASES = [
    (1024, 1024, 512, 3, 256, 1),
    (37, 4096, 1229, 3, 256, 1),
    (64, 14336, 4301, 4, 256, 1),
    (5, 1024, 0, 3, 256, 1),
    (96, 2560, 768, 3, 256, 2),
    (21, 9728, 2918, 3, 256, 2),
    (40, 1024, 1024, 7, 256, 2),
]


@pytest.mark.parametrize("case", PRODUCT_CASES, ids=[str(c) for c in PRODUCT_CASES])
def test_draft_gemv_and_verify_gemm(gpu, orc, case):
    torch, cass = gpu
    R, C, k, m, B, fmt = case
    print("case", case, flush=True)
    w = make_w(R, C, 77 + R + C)
    spec_o, verif_o = orc.encode(w, k, m, block=B, fmt=fmt)
    enc = cass.encode(dev(torch, w), k, m, block=B, fmt=fmt)
    for batch in (1, 2, 3):
        x = synth.activations(batch, C, 2, t0=batch)
        y = torch.full((batch, R), float("nan"), dtype=torch.float32, device="cuda")
        cass.cass_draft_gemv(enc.desc, dev(torch, x), y)
        torch.cuda.synchronize()
        y_ref, absy = orc.product(spec_o, x, threads=4)
        check_product(y.cpu().numpy(), y_ref, absy)
        if k == 0:
            assert (y.cpu().numpy() == 0).all()
    for ntok in (1, 5, 16):
        X = synth.activations(ntok, C, 3, t0=ntok)
        Y = torch.full((ntok, R), float("nan"), dtype=torch.float32, device="cuda")
        cass.cass_verify_gemm(enc.desc, dev(torch, X), Y)
        torch.cuda.synchronize()
        Y_ref, absY = orc.product(spec_o, X, verif=verif_o, threads=4)
        check_product(Y.cpu().numpy(), Y_ref, absY)


EXACT_CASES = [
    # rows, cols, keep, mant, block, weights
    (37, 4096, 1229, 3, 256, "normal"),
    (16, 512, 205, 0, 32, "normal"),
    (20, 14336, 4301, 2, 256, "normal"),
    (9, 1024, 0, 3, 128, "normal"),
    (9, 1024, 1024, 7, 64, "normal"),
    (33, 2048, 614, 3, 256, "wide"),   # long codes: past the LDS code share
    (19, 1280, 384, 5, 256, "normal"),  # odd block count, mantissa without the value table
    (40, 1024, 307, 1, 64, "normal"),
    # even rows keep their first positions, odd rows their last: in the first
    # and last blocks the rows' runs differ so much (full fields and low
    # mantissas against full pruned bytes) that the staged kernel packs them
    # back to back instead of giving every row an equal slot
    (32, 4096, 1229, 3, 256, "split"),
]


def exact_weights(R, C, kind, seed, keep=0):
    if kind == "wide":
        return synth.weight_wide(R, C, seed)
    w = make_w(R, C, seed)
    if kind == "split":
        # magnitudes at least 1 in each row's chosen range, below 1 elsewhere
        a = synth.f32_from_bf16(w)
        k = keep
        big = np.zeros_like(a, dtype=bool)
        big[0::2, :k] = True
        big[1::2, C - k:] = True
        a = np.where(big, np.sign(a) * (1.0 + np.abs(a)), a * np.float32(1e-3)).astype(np.float32)
        w = synth.bf16_from_f32(a)
    return w


@pytest.mark.parametrize("path", ["default", "blocks1", "blocks2", "direct"])
def test_exact_paths(gpu, orc, opt, path):
    """Reconstruction, draft decode and verification GEMM (Cassandra-1) through
    each decoder: the staged kernel with its default stage width, with stages
    of one or two blocks (option exact_blocks), and the per-thread stream readers
    (option exact_path)."""
    torch, cass = gpu
    if path == "blocks1":
        opt("exact_blocks", 1)
    elif path == "blocks2":
        opt("exact_blocks", 2)
    elif path == "direct":
        opt("exact_path", 1)
    for case in EXACT_CASES:
        R, C, k, m, B, kind = case
        print("case", path, case, flush=True)
        w = exact_weights(R, C, kind, 31 + R if kind == "wide" else 41 + R + C, keep=k)
        spec_o, verif_o = orc.encode(w, k, m, block=B)
        enc = cass.encode(dev(torch, w), k, m, block=B)
        out = torch.empty((R, C), dtype=torch.int16, device="cuda")
        cass.cass_reconstruct(enc.desc, out)
        torch.cuda.synchronize()
        assert np.array_equal(host_u16(out), w), case
        cass.cass_draft_decode(enc.desc, out)
        torch.cuda.synchronize()
        assert np.array_equal(host_u16(out), orc.draft_decode(spec_o)), case
        X = synth.activations(5, C, 3, t0=R)
        Y = torch.full((5, R), float("nan"), dtype=torch.float32, device="cuda")
        cass.cass_verify_gemm(enc.desc, dev(torch, X), Y)
        torch.cuda.synchronize()
        Y_ref, absY = orc.product(spec_o, X, verif=verif_o, threads=4)
        check_product(Y.cpu().numpy(), Y_ref, absY)


def test_verify_gemm_repeatable(gpu, orc):
    """The staged verification GEMM (Cassandra-1) splits a row's columns over
    the waves of one workgroup and adds their partial sums in wave order, so
    repeated calls give bit-identical outputs, within the product tolerance of
    the oracle."""
    torch, cass = gpu
    fmt = 1
    R, C, k, m, B = 200, 4096, 1229, 3, 256
    w = make_w(R, C, 77 + fmt)
    spec_o, verif_o = orc.encode(w, k, m, block=B, fmt=fmt)
    enc = cass.encode(dev(torch, w), k, m, block=B, fmt=fmt)
    X = dev(torch, synth.activations(5, C, 3, t0=fmt))
    outs = []
    for _ in range(3):
        Y = torch.full((5, R), float("nan"), dtype=torch.float32, device="cuda")
        cass.cass_verify_gemm(enc.desc, X, Y)
        torch.cuda.synchronize()
        outs.append(Y.cpu().numpy())
    assert all(np.array_equal(outs[0].view(np.uint32), o.view(np.uint32)) for o in outs[1:])
    Y_ref, absY = orc.product(spec_o, synth.activations(5, C, 3, t0=fmt), verif=verif_o, threads=4)
    check_product(outs[0], Y_ref, absY)


@pytest.mark.parametrize("fmt", [1, 2])
def test_direct_gemv_path(gpu, orc, opt, fmt):
    """The direct (non-staged) GEMV kernels, selected with the gemv_path option."""
    torch, cass = gpu
    R, C, k, m = 70, 4096, 1229, 3
    w = make_w(R, C, 606)
    spec_o, _ = orc.encode(w, k, m, fmt=fmt)
    enc = cass.encode(dev(torch, w), k, m, fmt=fmt)
    opt("gemv_path", 2)
    for batch in (1, 2):
        x = synth.activations(batch, C, 5)
        y = torch.full((batch, R), float("nan"), dtype=torch.float32, device="cuda")
        cass.cass_draft_gemv(enc.desc, dev(torch, x), y)
        torch.cuda.synchronize()
        y_ref, absy = orc.product(spec_o, x)
        check_product(y.cpu().numpy(), y_ref, absy)


BAL_CASES = [
    # rows, cols, keep, mant, block, parts (gemv_parts option; 0 = default), weights
    (64, 4096, 1229, 3, 256, 0, "normal"),    # q=0.3, 8 values per group
    (67, 4096, 819, 3, 256, 0, "normal"),     # q=0.2, 4 per group, ragged last round
    (48, 4096, 1024, 4, 256, 0, "normal"),    # q=0.25, m=4: 6 per group
    (33, 2048, 1024, 2, 128, 64, "normal"),   # 64 parts of 16, block 128
    (40, 1024, 307, 3, 32, 1, "normal"),      # one lane per row, block 32
    (16, 1024, 40, 3, 64, 64, "normal"),      # parts smaller than a group
    (20, 512, 30, 3, 256, 64, "normal"),      # k < parts: lanes without values
    (64, 4096, 1229, 3, 256, 16, "wide"),     # codes of 32+ bits: per-value steps
    (64, 4096, 2048, 5, 256, 8, "onewide"),   # one row's codes exceed the LDS share
    (64, 4096, 1229, 3, 256, 0, "ramp"),      # kept values pile up in the last blocks
    (64, 4096, 1229, 3, 256, 16, "clustered"),  # two full blocks: block estimates 2+ off
    (37, 4096, 1229, 3, 256, 0, "clustered"),
]


BAL_C2_CASES = [
    # rows, cols, keep, mant, block, parts (gemv_parts option; 0 = default), weights
    (64, 2560, 768, 3, 256, 0, "normal"),     # Qwen3-4B width, 6 fields per group
    (67, 4096, 819, 3, 256, 0, "normal"),     # ragged last round
    (33, 2048, 1024, 0, 128, 64, "normal"),   # sign-only significand: 8 per group
    (40, 1024, 307, 7, 32, 1, "normal"),      # 9-bit fields: 3 per group, one lane per row
    (20, 512, 30, 3, 256, 64, "normal"),      # k < parts
    (64, 4096, 1229, 3, 256, 16, "wide"),     # wide exponents (large shared-exponent offsets)
    (8, 1024, 1024, 5, 256, 0, "normal"),     # keep everything
    (64, 2560, 768, 3, 256, 0, "clustered"),  # two full blocks, most others sparse
]


@pytest.mark.parametrize("case", BAL_C2_CASES, ids=[str(c) for c in BAL_C2_CASES])
def test_balanced_gemv_c2(gpu, orc, opt, case):
    """The balanced draft GEMV for Cassandra-2 (shared exponent per 32
    positions) across part counts, mantissa widths and batches."""
    torch, cass = gpu
    R, C, k, m, B, parts, kind = case
    print("case", case, flush=True)
    w = bal_weights(R, C, kind, 2000 + R + k)
    spec_o, _ = orc.encode(w, k, m, block=B, fmt=2)
    enc = cass.encode(dev(torch, w), k, m, block=B, fmt=2)
    if parts:
        opt("gemv_parts", parts)
    for batch in (1, 2, 3):
        x = synth.activations(batch, C, 7, t0=batch)
        y = torch.full((batch, R), float("nan"), dtype=torch.float32, device="cuda")
        cass.cass_draft_gemv(enc.desc, dev(torch, x), y)
        torch.cuda.synchronize()
        y_ref, absy = orc.product(spec_o, x, threads=4)
        check_product(y.cpu().numpy(), y_ref, absy)


def bal_weights(R, C, kind, seed):
    if kind == "normal":
        return make_w(R, C, seed)
    if kind == "wide":
        return synth.weight_wide(R, C, seed)
    if kind in ("ramp", "clustered"):
        # the per-row kept values are far from uniform over the blocks, so a
        # lane's block estimate (kept count / blocks) misses by several blocks
        # and many blocks keep nothing
        rng = np.random.default_rng(seed)
        a = rng.standard_normal((R, C), dtype=np.float32) * np.float32(0.02)
        if kind == "ramp":
            a *= np.exp2(np.linspace(0.0, 12.0, C, dtype=np.float32))[None, :]
        else:
            for b in (2, 9):
                a[:, b * 256:(b + 1) * 256] *= np.float32(100.0)
        return synth.bf16_from_f32(a)
    w = make_w(R, C, seed)
    w[5] = synth.weight_wide(1, C, seed + 1, binades=120)[0]
    return w


@pytest.mark.parametrize("case", BAL_CASES, ids=[str(c) for c in BAL_CASES])
def test_balanced_gemv_variants(gpu, orc, opt, case):
    """The balanced draft GEMV (default Cassandra-1 path) across part counts,
    keep ratios, blocks, long codes and the global-code fallback."""
    torch, cass = gpu
    R, C, k, m, B, parts, kind = case
    print("case", case, flush=True)
    w = bal_weights(R, C, kind, 1000 + R + k)
    spec_o, _ = orc.encode(w, k, m, block=B)
    enc = cass.encode(dev(torch, w), k, m, block=B)
    if parts:
        opt("gemv_parts", parts)
    for batch in (1, 3):
        x = synth.activations(batch, C, 6, t0=batch)
        y = torch.full((batch, R), float("nan"), dtype=torch.float32, device="cuda")
        cass.cass_draft_gemv(enc.desc, dev(torch, x), y)
        torch.cuda.synchronize()
        y_ref, absy = orc.product(spec_o, x, threads=4)
        check_product(y.cpu().numpy(), y_ref, absy)


@pytest.mark.parametrize("path", ["staged", "direct"])
def test_other_gemv_paths(gpu, orc, opt, path):
    """The staged and direct kernels, which serve shapes the balanced kernel
    does not take (selected here by environment)."""
    torch, cass = gpu
    R, C, k, m = 45, 4096, 1229, 3
    w = make_w(R, C, 808)
    spec_o, _ = orc.encode(w, k, m)
    enc = cass.encode(dev(torch, w), k, m)
    if path == "staged":
        opt("gemv_path", 1)
    else:
        opt("gemv_path", 2)
    x = synth.activations(2, C, 7)
    y = torch.full((2, R), float("nan"), dtype=torch.float32, device="cuda")
    cass.cass_draft_gemv(enc.desc, dev(torch, x), y)
    torch.cuda.synchronize()
    y_ref, absy = orc.product(spec_o, x)
    check_product(y.cpu().numpy(), y_ref, absy)


def test_strided_operands(gpu, orc):
    """ldx > cols and ldy > rows are honoured (padding untouched)."""
    torch, cass = gpu
    R, C = 100, 2048
    w = make_w(R, C, 9)
    spec_o, verif_o = orc.encode(w, 614, 3)
    enc = cass.encode(dev(torch, w), 614, 3)
    x = synth.activations(2, C, 4)
    xpad = np.zeros((2, C + 64), dtype=np.uint16)
    xpad[:, :C] = x
    y = torch.full((2, R + 3), 7.0, dtype=torch.float32, device="cuda")
    cass.cass_draft_gemv(enc.desc, dev(torch, xpad)[:, :C], y[:, :R])
    torch.cuda.synchronize()
    yh = y.cpu().numpy()
    assert (yh[:, R:] == 7.0).all()
    y_ref, absy = orc.product(spec_o, x)
    check_product(yh[:, :R], y_ref, absy)


def test_empty_tensor(gpu):
    torch, cass = gpu
    w = torch.empty((0, 1024), dtype=torch.int16, device="cuda")
    enc = cass.encode(w, 300, 3)
    torch.cuda.synchronize()
    assert enc.rows == 0
    y = torch.empty((1, 0), dtype=torch.float32, device="cuda")
    cass.cass_draft_gemv(enc.desc, torch.zeros((1, 1024), dtype=torch.int16, device="cuda"), y)
    torch.cuda.synchronize()


LLAMA_MATS = ["qkv", "o", "gu", "down"]


@pytest.fixture(scope="module")
def llama_layer():
    return synth.fused_layer(synth.LLAMA3_8B, config=2, layer=0, outlier_frac=0.01)


@pytest.fixture(scope="module")
def qwen_layer():
    return synth.fused_layer(synth.QWEN3_4B, config=5, layer=0, outlier_frac=0.0)


def full_size_check(torch, cass, orc, w, k, m, fmt, batch):
    """One matrix at its full shape, encoded by the library as the benchmark
    does: both streams byte for byte against the oracle's encoding of the whole
    matrix, exact reconstruction, and every output of the draft GEMV (the
    benchmark's launch configuration) and of the N = 5 verification GEMM."""
    R, C = w.shape
    wd = dev(torch, w)
    enc = cass.encode(wd, k, m, fmt=fmt)
    out = torch.empty_like(wd)
    cass.cass_reconstruct(enc.desc, out)
    x = synth.activations(batch, C, 2)
    y = torch.full((batch, R), float("nan"), dtype=torch.float32, device="cuda")
    cass.cass_draft_gemv(enc.desc, dev(torch, x), y)
    X = synth.activations(5, C, 2, t0=10)
    Y = torch.full((5, R), float("nan"), dtype=torch.float32, device="cuda")
    cass.cass_verify_gemm(enc.desc, dev(torch, X), Y)
    torch.cuda.synchronize()
    assert torch.equal(out, wd), "reconstruction"
    spec_g, verif_g = host_u8(enc.spec), host_u8(enc.verif)
    del enc, out, wd
    spec_o, verif_o = orc.encode(w, k, m, fmt=fmt)
    assert np.array_equal(spec_g, spec_o), "speculation stream"
    assert np.array_equal(verif_g, verif_o), "verification stream"
    y_ref, absy = orc.product(spec_o, x, threads=8)
    check_product(y.cpu().numpy(), y_ref, absy)
    Y_ref, absY = orc.product(spec_o, X, verif=verif_o, threads=8)
    check_product(Y.cpu().numpy(), Y_ref, absY)


@pytest.mark.parametrize("name", LLAMA_MATS)
def test_llama8b_layer_full_size(gpu, orc, llama_layer, name):
    """The Llama-3-8B-shaped layer (q|k|v, o, gate|up, down) at keep 0.3, 3
    mantissa bits, Cassandra-1, batch 1: the benchmark's workload, every byte
    and every output."""
    torch, cass = gpu
    w = llama_layer[name]
    print("matrix", name, w.shape, flush=True)
    full_size_check(torch, cass, orc, w, synth.keep_count(0.3, w.shape[1]), 3, 1, 1)


@pytest.mark.parametrize("name", LLAMA_MATS)
def test_qwen3_4b_c2_full_size(gpu, orc, qwen_layer, name):
    """The Qwen3-4B-shaped layer at keep 0.3, 3 mantissa bits, Cassandra-2
    (shared exponent per 32 positions), batch 2: the benchmark's 36-layer
    stack's shapes, every byte and every output."""
    torch, cass = gpu
    w = qwen_layer[name]
    print("matrix", name, w.shape, flush=True)
    full_size_check(torch, cass, orc, w, synth.keep_count(0.3, w.shape[1]), 3, 2, 2)


@pytest.mark.parametrize("fmt", [1, 2])
def test_strided_encode(gpu, orc, fmt):
    """Rows of the input spaced ld > cols elements apart (a column slice of a
    wider matrix) encode to the same bytes as the contiguous rows."""
    torch, cass = gpu
    R, C, ld = 37, 1024, 1536
    wide = synth.weight(R, ld, 91 + fmt, outlier_frac=0.01)
    wd = dev(torch, wide)[:, 256:256 + C]
    assert wd.stride(0) == ld
    enc = cass.encode(wd, 307, 3, fmt=fmt)
    torch.cuda.synchronize()
    spec_o, verif_o = orc.encode(wide[:, 256:256 + C], 307, 3, fmt=fmt)
    assert np.array_equal(host_u8(enc.spec), spec_o)
    assert np.array_equal(host_u8(enc.verif), verif_o)
