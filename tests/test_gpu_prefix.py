"""The comparison exponent codecs on the GPU against the CPU oracle, through
the C ABI: streams and block offsets of the canonical Huffman and the unary
code byte for byte equal to the oracle's encoding (with the same code tables,
which the host tests check equal), and every decoder giving back the symbols
exactly."""
import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def gpu():
    import torch
    import bit_level_weight_amd as cass
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    cass.lib()
    return torch, cass


def kept_exponents(orc, R, C, k, seed):
    w = synth.weight(R, C, seed, outlier_frac=0.01)
    keep = orc.select(w, k)
    return ((w[keep] >> 7) & 0xFF).astype(np.uint8)


def run_codec(torch, cass, orc, sym, block, code, ln, cv, methods):
    n = sym.size
    bits = int(ln[sym].astype(np.int64).sum())
    stream_bytes = ((bits + 7) // 8 + 15) // 16 * 16 + 16
    stream = torch.full((stream_bytes,), 0xAB, dtype=torch.uint8, device="cuda")
    blkoff = torch.zeros(((n + block - 1) // block,), dtype=torch.int32, device="cuda")
    d_sym = torch.from_numpy(sym).cuda()
    cass.cass_prefix_encode(code, d_sym, block, stream, blkoff)
    torch.cuda.synchronize()
    s_o, b_o, bits_o = orc.prefix_encode(sym, block, ln, cv)
    assert bits_o == bits
    got = stream.cpu().numpy()
    assert np.array_equal(got[:stream_bytes], np.pad(s_o, (0, max(0, stream_bytes - s_o.size)))[:stream_bytes])
    assert np.array_equal(blkoff.cpu().numpy().view(np.uint32), b_o)
    ws = torch.empty((cass.cass_prefix_decode_ws_bytes(stream_bytes),), dtype=torch.uint8,
                     device="cuda")
    for method in methods:
        out = torch.full((n,), 0xCD, dtype=torch.uint8, device="cuda")
        cass.cass_prefix_decode(code, stream, blkoff, n, block, method, out, ws)
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy(), sym), method


@pytest.mark.parametrize("R,C,k,block", [(64, 1024, 307, 256), (16, 4096, 1229, 64),
                                         (3, 512, 160, 16), (200, 1024, 1024, 256)])
def test_codecs_round_trip(gpu, orc, R, C, k, block):
    torch, cass = gpu
    print("case", R, C, k, block, flush=True)
    sym = kept_exponents(orc, R, C, k, 7000 + R + C)
    sym = sym[: sym.size // 16 * 16]
    hist = np.bincount(sym, minlength=256).astype(np.uint64)
    huff = cass.cass_prefix_code_huffman(hist, 12)
    ln, cv = orc.huffman_code(hist, 12)
    run_codec(torch, cass, orc, sym, block, huff, ln, cv, [cass.CASS_PREFIX_TABLE])
    if np.count_nonzero(hist) > 32:
        return  # the unary codes of ranks past 31 are longer than 32 bits
    un = cass.cass_prefix_code_unary(hist)
    ln, cv = orc.unary_code(hist)
    methods = [cass.CASS_PREFIX_UNARY_SERIAL, cass.CASS_PREFIX_UNARY_PARALLEL]
    if un.max_len <= 12:
        methods.append(cass.CASS_PREFIX_TABLE)
    run_codec(torch, cass, orc, sym, block, un, ln, cv, methods)


def test_codecs_edge_cases(gpu, orc):
    torch, cass = gpu
    # one symbol only (1-bit Huffman code, 1-bit unary code), sixteen symbols
    sym = np.full(16, 121, dtype=np.uint8)
    hist = np.bincount(sym, minlength=256).astype(np.uint64)
    ln, cv = orc.huffman_code(hist, 12)
    run_codec(torch, cass, orc, sym, 16, cass.cass_prefix_code_huffman(hist, 12), ln, cv,
              [cass.CASS_PREFIX_TABLE])
    ln, cv = orc.unary_code(hist)
    run_codec(torch, cass, orc, sym, 16, cass.cass_prefix_code_unary(hist), ln, cv,
              [cass.CASS_PREFIX_UNARY_SERIAL, cass.CASS_PREFIX_UNARY_PARALLEL])
    # the parallel decoder over many workgroups: long runs of rare symbols (long codes)
    rng = np.random.default_rng(3)
    p = np.array([0.5, 0.2, 0.1, 0.08, 0.05, 0.03, 0.02, 0.01, 0.005, 0.005])
    sym = (110 + rng.choice(10, size=300_000, p=p)).astype(np.uint8)
    sym[1000:3000] = 119  # rarest symbol, in one run
    hist = np.bincount(sym, minlength=256).astype(np.uint64)
    ln, cv = orc.unary_code(hist)
    run_codec(torch, cass, orc, sym, 256, cass.cass_prefix_code_unary(hist), ln, cv,
              [cass.CASS_PREFIX_UNARY_SERIAL, cass.CASS_PREFIX_UNARY_PARALLEL])
    ln, cv = orc.huffman_code(hist, 12)
    run_codec(torch, cass, orc, sym, 256, cass.cass_prefix_code_huffman(hist, 12), ln, cv,
              [cass.CASS_PREFIX_TABLE])
