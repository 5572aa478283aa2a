"""CPU oracle for the Cassandra bit-level weight format -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The HIP library never calls it and the
two share no code.  The arithmetic lives in ``cass_oracle.c`` (plain scalar C,
one function per step of the method, each citing the passage it follows); this
module only builds it with gcc and marshals numpy arrays through ctypes.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "cass_oracle.c")
_LIB = os.path.join(_HERE, "libcass_oracle.so")

OK, ERR_INVALID, ERR_UNSUPPORTED, ERR_OVERFLOW, ERR_CORRUPT, ERR_CAPACITY = range(6)
FMT_C1, FMT_C2, FMT_C2T, FMT_C1S = 1, 2, 3, 4
SUPERBLOCK_BLOCKS = 16
MAGIC_SPEC, MAGIC_VERIF = 0x50535343, 0x46565343


class OracleError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"oracle {what} failed with status {status}")
        self.status = status


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (plain -O2, no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB):
        cmd = ["gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fopenmp", "-fPIC",
               "-shared", "-Wall", "-Wextra", "-o", _LIB + ".tmp", _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(_LIB + ".tmp", _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        L = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        L.orc_select.argtypes = [P, I64, I64, I64, P]
        L.orc_histograms.argtypes = [P, P, I64, P, P]
        L.orc_rank_table.argtypes = [P, P]
        L.orc_rank_table.restype = None
        L.orc_encode.argtypes = [P, I64, I64, I64, ctypes.c_int, I64, ctypes.c_int, P, I64,
                                 P, I64, ctypes.POINTER(I64), ctypes.POINTER(I64)]
        L.orc_draft_decode.argtypes = [P, I64, P]
        L.orc_reconstruct.argtypes = [P, I64, P, I64, P]
        L.orc_product.argtypes = [P, I64, P, I64, P, I64, P, P, ctypes.c_int]
        L.orc_product_rows.argtypes = [P, I64, P, I64, P, I64, P, I64, P, P]
        L.orc_header.argtypes = [P, I64, ctypes.c_uint32, P, P, P]
        L.orc_mx_target.argtypes = [P, I64, I64, P]
        L.orc_huffman_lengths.argtypes = [P, ctypes.c_int, P]
        L.orc_canonical_codes.argtypes = [P, P]
        L.orc_unary_code.argtypes = [P, P, P]
        L.orc_prefix_encode.argtypes = [P, I64, I64, P, P, P, I64, P, ctypes.POINTER(I64)]
        L.orc_prefix_decode.argtypes = [P, I64, I64, P, P, P]
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _check(st, what):
    if st != OK:
        raise OracleError(st, what)


def _u16(w):
    return np.ascontiguousarray(w, dtype=np.uint16)


def select(w, k: int) -> np.ndarray:
    """Boolean keep-mask [R, C]: exactly k per row by |w|, ties to the lower column."""
    w = _u16(w)
    R, C = w.shape
    keep = np.zeros((R, C), dtype=np.uint8)
    _check(lib().orc_select(_p(w), R, C, k, _p(keep)), "select")
    return keep.astype(bool)


def histograms(w, keep):
    w = _u16(w)
    keep = np.ascontiguousarray(keep, dtype=np.uint8)
    hk = np.zeros(256, dtype=np.uint64)
    hp = np.zeros(256, dtype=np.uint64)
    _check(lib().orc_histograms(_p(w), _p(keep), w.size, _p(hk), _p(hp)), "histograms")
    return hk, hp


def rank_table(hist) -> np.ndarray:
    """perm[r] = symbol of rank r (count descending, symbol ascending)."""
    h = np.ascontiguousarray(hist, dtype=np.uint64)
    perm = np.zeros(256, dtype=np.uint8)
    lib().orc_rank_table(_p(h), _p(perm))
    return perm


def encode(w, k: int, m: int, block: int = 256, fmt: int = FMT_C1):
    """Encode bf16 bit patterns w[R, C] -> (spec bytes, verif bytes) as uint8 arrays."""
    w = _u16(w)
    R, C = w.shape
    sb, vb = ctypes.c_int64(0), ctypes.c_int64(0)
    L = lib()
    _check(L.orc_encode(_p(w), R, C, k, m, block, fmt, None, 0, None, 0,
                        ctypes.byref(sb), ctypes.byref(vb)), "encode sizes")
    spec = np.zeros(sb.value, dtype=np.uint8)
    verif = np.zeros(vb.value, dtype=np.uint8)
    _check(L.orc_encode(_p(w), R, C, k, m, block, fmt, _p(spec), spec.size, _p(verif),
                        verif.size, ctypes.byref(sb), ctypes.byref(vb)), "encode")
    return spec, verif


def mx_target(w) -> np.ndarray:
    """Target weights of format 3 (Cassandra-2 with an MX-quantised target):
    per 32 positions of a row, every value's significand aligned to the
    group's largest exponent and chopped to 8 bits (orc_mx_target)."""
    w = _u16(w)
    R, C = w.shape
    out = np.zeros((R, C), dtype=np.uint16)
    _check(lib().orc_mx_target(_p(w), R, C, _p(out)), "mx_target")
    return out


def huffman_code(hist, max_len: int = 32):
    """(lengths u8[256], canonical codes u32[256]) of a length-limited Huffman code."""
    h = np.ascontiguousarray(hist, dtype=np.uint64)
    ln = np.zeros(256, dtype=np.uint8)
    code = np.zeros(256, dtype=np.uint32)
    _check(lib().orc_huffman_lengths(_p(h), max_len, _p(ln)), "huffman_lengths")
    _check(lib().orc_canonical_codes(_p(ln), _p(code)), "canonical_codes")
    return ln, code


def unary_code(hist):
    """(lengths, codes) of Cassandra-1's frequency-ranked unary code."""
    h = np.ascontiguousarray(hist, dtype=np.uint64)
    ln = np.zeros(256, dtype=np.uint8)
    code = np.zeros(256, dtype=np.uint32)
    _check(lib().orc_unary_code(_p(h), _p(ln), _p(code)), "unary_code")
    return ln, code


def prefix_encode(sym, block, ln, code):
    """-> (stream bytes (zero padded to a multiple of 16, plus 16), block offsets, bits)."""
    sym = np.ascontiguousarray(sym, dtype=np.uint8)
    ln = np.ascontiguousarray(ln, dtype=np.uint8)
    code = np.ascontiguousarray(code, dtype=np.uint32)
    bits = ctypes.c_int64(0)
    _check(lib().orc_prefix_encode(_p(sym), sym.size, block, _p(ln), _p(code), None, 0, None,
                                   ctypes.byref(bits)), "prefix_encode sizes")
    nbytes = (bits.value + 7) // 8
    stream = np.zeros((nbytes + 15) // 16 * 16 + 16, dtype=np.uint8)
    blkoff = np.zeros(max(1, (sym.size + block - 1) // block), dtype=np.uint32)
    _check(lib().orc_prefix_encode(_p(sym), sym.size, block, _p(ln), _p(code), _p(stream),
                                   stream.size, _p(blkoff), ctypes.byref(bits)), "prefix_encode")
    return stream, blkoff, bits.value


def prefix_decode(stream, n, ln, code):
    stream = np.ascontiguousarray(stream, dtype=np.uint8)
    out = np.zeros(n, dtype=np.uint8)
    _check(lib().orc_prefix_decode(_p(stream), stream.size, n,
                                   _p(np.ascontiguousarray(ln, dtype=np.uint8)),
                                   _p(np.ascontiguousarray(code, dtype=np.uint32)), _p(out)),
           "prefix_decode")
    return out


def header(buf, magic: int = MAGIC_SPEC):
    buf = np.ascontiguousarray(buf, dtype=np.uint8)
    out = np.zeros(8, dtype=np.int64)
    off = np.zeros(12, dtype=np.int64)
    ln = np.zeros(12, dtype=np.int64)
    _check(lib().orc_header(_p(buf), buf.size, magic, _p(out), _p(off), _p(ln)), "header")
    keys = ("format", "mant_bits", "rows", "cols", "block", "keep", "total_bytes", "n_sections")
    h = dict(zip(keys, (int(v) for v in out)))
    h["sections"] = [(int(o), int(n)) for o, n in zip(off, ln)][: h["n_sections"]]
    return h


def draft_decode(spec) -> np.ndarray:
    spec = np.ascontiguousarray(spec, dtype=np.uint8)
    h = header(spec)
    out = np.zeros((h["rows"], h["cols"]), dtype=np.uint16)
    _check(lib().orc_draft_decode(_p(spec), spec.size, _p(out)), "draft_decode")
    return out


def reconstruct(spec, verif) -> np.ndarray:
    spec = np.ascontiguousarray(spec, dtype=np.uint8)
    verif = np.ascontiguousarray(verif, dtype=np.uint8)
    h = header(spec)
    out = np.zeros((h["rows"], h["cols"]), dtype=np.uint16)
    _check(lib().orc_reconstruct(_p(spec), spec.size, _p(verif), verif.size, _p(out)),
           "reconstruct")
    return out


def product(spec, x, verif=None, threads: int = 1):
    """(y, absy) in float64, shape [ntok, R]: draft product when verif is None,
    else the product with the exact reconstructed weights."""
    spec = np.ascontiguousarray(spec, dtype=np.uint8)
    x = _u16(np.atleast_2d(x))
    h = header(spec)
    assert x.shape[1] == h["cols"]
    ntok = x.shape[0]
    y = np.zeros((ntok, h["rows"]), dtype=np.float64)
    absy = np.zeros_like(y)
    if verif is not None:
        verif = np.ascontiguousarray(verif, dtype=np.uint8)
    _check(lib().orc_product(_p(spec), spec.size, _p(verif),
                             0 if verif is None else verif.size, _p(x), ntok, _p(y),
                             _p(absy), threads), "product")
    return y, absy


def product_rows(spec, x, rows, verif=None):
    """orc_product for the listed rows only -> (y, absy), shape [ntok, len(rows)]."""
    spec = np.ascontiguousarray(spec, dtype=np.uint8)
    x = _u16(np.atleast_2d(x))
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    ntok = x.shape[0]
    y = np.zeros((ntok, rows.size), dtype=np.float64)
    absy = np.zeros_like(y)
    if verif is not None:
        verif = np.ascontiguousarray(verif, dtype=np.uint8)
    _check(lib().orc_product_rows(_p(spec), spec.size, _p(verif),
                                  0 if verif is None else verif.size, _p(x), ntok, _p(rows),
                                  rows.size, _p(y), _p(absy)), "product_rows")
    return y, absy


# ------------------------------------------------------------------ KV cache

def _kv_lib():
    L = lib()
    if not getattr(L, "_kv_ready", False):
        P, I64 = ctypes.c_void_p, ctypes.c_int64
        L.orc_kv_layout.argtypes = [ctypes.c_int, I64, I64, ctypes.c_int, I64, I64, I64, P, P,
                                    ctypes.POINTER(I64), ctypes.POINTER(I64)]
        L.orc_kv_encode.argtypes = [ctypes.c_int, P, I64, I64, I64, I64, ctypes.c_int, I64, I64,
                                    I64, P, P, P]
        L.orc_kv_decode.argtypes = [ctypes.c_int, P, P, I64, I64, I64, ctypes.c_int, I64, I64,
                                    I64, P]
        L.orc_attention.argtypes = [P, I64, P, P, I64, I64, ctypes.c_double, P, P]
        L._kv_ready = True
    return L


def kv_layout(D, k, m, T_max, code_cap, vcode_cap, fmt=FMT_C1):
    """(spec part offsets[5], verif part offsets[5], spec bytes, verif bytes) of one stream."""
    so = np.zeros(5, dtype=np.int64)
    vo = np.zeros(5, dtype=np.int64)
    sb, vb = ctypes.c_int64(0), ctypes.c_int64(0)
    _check(_kv_lib().orc_kv_layout(fmt, D, k, m, T_max, code_cap, vcode_cap, _p(so), _p(vo),
                                   ctypes.byref(sb), ctypes.byref(vb)), "kv_layout")
    return so, vo, sb.value, vb.value


def kv_encode(vec, T0, k, m, T_max, code_cap, vcode_cap, fmt=FMT_C1):
    """One (head, K|V) stream of all tokens of vec[T, D] -> (spec, verif, tails)."""
    vec = _u16(vec)
    T, D = vec.shape
    _, _, sb, vb = kv_layout(D, k, m, T_max, code_cap, vcode_cap, fmt)
    spec = np.zeros(sb, dtype=np.uint8)
    verif = np.zeros(vb, dtype=np.uint8)
    tails = np.zeros(2, dtype=np.uint64)
    _check(_kv_lib().orc_kv_encode(fmt, _p(vec), T, T0, D, k, m, T_max, code_cap, vcode_cap,
                                   _p(spec), _p(verif), _p(tails)), "kv_encode")
    return spec, verif, tails


def kv_decode(spec, T, D, k, m, T_max, code_cap, vcode_cap, verif=None, fmt=FMT_C1):
    spec = np.ascontiguousarray(spec, dtype=np.uint8)
    if verif is not None:
        verif = np.ascontiguousarray(verif, dtype=np.uint8)
    out = np.zeros((T, D), dtype=np.uint16)
    _check(_kv_lib().orc_kv_decode(fmt, _p(spec), _p(verif), T, D, k, m, T_max, code_cap,
                                   vcode_cap, _p(out)), "kv_decode")
    return out


def attention(q, K, V, scale, visible=None):
    """fp64 softmax attention of q[nq, D] over K, V [T, D] (bf16 patterns)."""
    q = _u16(np.atleast_2d(q))
    K = _u16(K)
    V = _u16(V)
    nq, D = q.shape
    T = K.shape[0]
    out = np.zeros((nq, D), dtype=np.float64)
    vis = None if visible is None else np.ascontiguousarray(visible, dtype=np.int64)
    _check(_kv_lib().orc_attention(_p(q), nq, _p(K), _p(V), T, D, float(scale), _p(vis),
                                   _p(out)), "attention")
    return out
