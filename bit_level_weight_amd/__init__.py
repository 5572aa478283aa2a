"""Python binding of libcassandra (the Cassandra bit-level weight format on
MI355X).  Argument marshalling only: every step runs in the HIP library.

The functions carry the C names (see include/cassandra.h) and take torch
tensors for device buffers; PyTorch provides device memory and streams.
``encode()`` is a convenience wrapper that sizes and allocates the buffers
with torch and runs the two encoder passes.

Importing this package does not touch the GPU.  Loading the library fails
loudly when it has not been built (``python -m bit_level_weight_amd.build``).
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libcassandra.so")
DEBUG_LIB_PATH = os.path.join(_HERE, "libcassandra_debug.so")

CASS_OK, CASS_ERR_INVALID, CASS_ERR_UNSUPPORTED, CASS_ERR_OVERFLOW, CASS_ERR_CORRUPT, \
    CASS_ERR_CAPACITY, CASS_ERR_HIP = range(7)
CASS_FMT_C1_UNARY, CASS_FMT_C2_MX32, CASS_FMT_C2_MX_TARGET, CASS_FMT_C1_SUPERBLOCK = 1, 2, 3, 4
MAX_SECTIONS = 12

# symbols include/cassandra.h declares
EXPORTED = (
    "cass_encode_ws_bytes", "cass_encode_plan", "cass_encode_tensor", "cass_tensor_describe",
    "cass_draft_gemv", "cass_verify_gemm", "cass_reconstruct", "cass_draft_decode",
    "cass_tensor_validate", "cass_status_string", "cass_last_error", "cass_version",
    "cass_kv_bytes", "cass_kv_init", "cass_kv_append_ws_bytes", "cass_kv_append_encode",
    "cass_kv_status", "cass_kv_decode", "cass_kv_attn_ws_bytes", "cass_kv_draft_attn",
    "cass_kv_verify_attn", "cass_set_option", "cass_stream_read", "cass_kv_draft_attn_static",
    "cass_kv_truncate", "cass_prefix_code_huffman", "cass_prefix_code_unary",
    "cass_prefix_stream_bits", "cass_prefix_encode", "cass_prefix_decode_ws_bytes",
    "cass_prefix_decode", "cass_debug_flags",
)
CASS_DBG_STAGE, CASS_DBG_ALIGN, CASS_DBG_TILE, CASS_DBG_WINDOW = 1, 2, 4, 8
# the same sources built with CASS_DEBUG (device bounds checks); load it in
# place of the release library by pointing LIB_PATH here before lib()
CASS_PREFIX_TABLE, CASS_PREFIX_UNARY_SERIAL, CASS_PREFIX_UNARY_PARALLEL = 1, 2, 3
CASS_STREAM_READ_BLOCKS = 2048
CASS_KV_STATE_BYTES = 4096
CASS_KV_STATIC_SCRATCH_BYTES = 32 << 20
CASS_KV_FLAG_TABLES, CASS_KV_FLAG_OVERFLOW = 1, 2


class CassParams(ctypes.Structure):
    _fields_ = [("format", ctypes.c_int32), ("mant_bits", ctypes.c_int32),
                ("block", ctypes.c_int64), ("keep", ctypes.c_int64)]


class CassTensor(ctypes.Structure):
    _fields_ = [("format", ctypes.c_int32), ("mant_bits", ctypes.c_int32),
                ("rows", ctypes.c_int64), ("cols", ctypes.c_int64), ("block", ctypes.c_int64),
                ("keep", ctypes.c_int64),
                ("spec", ctypes.c_void_p), ("spec_bytes", ctypes.c_int64),
                ("verif", ctypes.c_void_p), ("verif_bytes", ctypes.c_int64),
                ("spec_sec", ctypes.c_int64 * MAX_SECTIONS),
                ("verif_sec", ctypes.c_int64 * MAX_SECTIONS)]


class CassPlan(ctypes.Structure):
    _fields_ = [("rows", ctypes.c_int64), ("cols", ctypes.c_int64), ("ld", ctypes.c_int64),
                ("p", CassParams),
                ("spec_bytes", ctypes.c_int64), ("verif_bytes", ctypes.c_int64),
                ("spec_sec", ctypes.c_int64 * MAX_SECTIONS),
                ("spec_len", ctypes.c_int64 * MAX_SECTIONS),
                ("verif_sec", ctypes.c_int64 * MAX_SECTIONS),
                ("verif_len", ctypes.c_int64 * MAX_SECTIONS),
                ("hist_kept", ctypes.c_uint64 * 256), ("hist_pruned", ctypes.c_uint64 * 256),
                ("perm_spec", ctypes.c_uint8 * 256), ("perm_verif", ctypes.c_uint8 * 256),
                ("spec_code_bits", ctypes.c_uint64), ("verif_code_bits", ctypes.c_uint64),
                ("resid_bits", ctypes.c_uint64),
                ("ws", ctypes.c_void_p), ("ws_bytes", ctypes.c_int64)]


class CassKvParams(ctypes.Structure):
    _fields_ = [("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("keep", ctypes.c_int32), ("mant_bits", ctypes.c_int32),
                ("max_tokens", ctypes.c_int64), ("code_cap_bits", ctypes.c_int64),
                ("vcode_cap_bits", ctypes.c_int64), ("format", ctypes.c_int32)]


class CassKv(ctypes.Structure):
    _fields_ = [("p", CassKvParams), ("spec", ctypes.c_void_p), ("verif", ctypes.c_void_p),
                ("state", ctypes.c_void_p), ("spec_stream_bytes", ctypes.c_int64),
                ("verif_stream_bytes", ctypes.c_int64), ("spec_part", ctypes.c_int64 * 5),
                ("verif_part", ctypes.c_int64 * 5), ("tokens", ctypes.c_int64)]


class CassPrefixCode(ctypes.Structure):
    _fields_ = [("max_len", ctypes.c_int32), ("len", ctypes.c_uint8 * 256),
                ("code", ctypes.c_uint32 * 256)]


class CassError(RuntimeError):
    def __init__(self, status, detail):
        super().__init__(f"libcassandra status {status}: {detail}")
        self.status = status


_lib = None


def lib():
    """Load libcassandra.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"HIP library missing: {LIB_PATH}; build it with "
                               "`python -m bit_level_weight_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P, I64, I32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        L.cass_encode_ws_bytes.argtypes = [I64, I64, ctypes.POINTER(CassParams),
                                           ctypes.POINTER(I64)]
        L.cass_encode_plan.argtypes = [P, I64, I64, I64, ctypes.POINTER(CassParams), P, I64, P,
                                       ctypes.POINTER(CassPlan)]
        L.cass_encode_tensor.argtypes = [P, I64, ctypes.POINTER(CassPlan), P, I64, P, I64, P,
                                         ctypes.POINTER(CassTensor)]
        L.cass_tensor_describe.argtypes = [P, P, I64, P, P, I64, ctypes.POINTER(CassTensor)]
        L.cass_draft_gemv.argtypes = [ctypes.POINTER(CassTensor), P, I32, I64, P, I64, P]
        L.cass_verify_gemm.argtypes = [ctypes.POINTER(CassTensor), P, I32, I64, P, I64, P]
        L.cass_reconstruct.argtypes = [ctypes.POINTER(CassTensor), P, P]
        L.cass_draft_decode.argtypes = [ctypes.POINTER(CassTensor), P, P]
        L.cass_tensor_validate.argtypes = [P, I64, P, I64]
        L.cass_status_string.argtypes = [I32]
        L.cass_status_string.restype = ctypes.c_char_p
        L.cass_last_error.argtypes = []
        L.cass_last_error.restype = ctypes.c_char_p
        L.cass_version.argtypes = []
        L.cass_debug_flags.argtypes = [ctypes.POINTER(ctypes.c_uint32)]
        L.cass_set_option.argtypes = [ctypes.c_char_p, I64]
        L.cass_stream_read.argtypes = [P, I64, P, P]
        KP, KV = ctypes.POINTER(CassKvParams), ctypes.POINTER(CassKv)
        L.cass_kv_bytes.argtypes = [KP, ctypes.POINTER(I64), ctypes.POINTER(I64),
                                    ctypes.POINTER(I64)]
        L.cass_kv_init.argtypes = [KV, KP, P, P, P, P]
        L.cass_kv_append_ws_bytes.argtypes = [KV, I32, ctypes.POINTER(I64)]
        L.cass_kv_append_encode.argtypes = [KV, P, P, I32, P, I64, P]
        L.cass_kv_status.argtypes = [KV, ctypes.POINTER(I64), ctypes.POINTER(ctypes.c_uint32), P]
        L.cass_kv_decode.argtypes = [KV, I32, P, P]
        L.cass_kv_attn_ws_bytes.argtypes = [KV, I32, I32, ctypes.POINTER(I64)]
        L.cass_kv_draft_attn.argtypes = [KV, P, I32, ctypes.c_float, P, P, I64, P]
        L.cass_kv_verify_attn.argtypes = [KV, P, I32, I32, ctypes.c_float, P, P, I64, P]
        L.cass_kv_draft_attn_static.argtypes = [KV, P, I32, ctypes.c_float, P, P]
        L.cass_kv_truncate.argtypes = [KV, I64, P]
        PC = ctypes.POINTER(CassPrefixCode)
        L.cass_prefix_code_huffman.argtypes = [P, I32, PC]
        L.cass_prefix_code_unary.argtypes = [P, PC]
        L.cass_prefix_stream_bits.argtypes = [PC, P, ctypes.POINTER(I64)]
        L.cass_prefix_encode.argtypes = [PC, P, I64, I64, P, I64, P, P]
        L.cass_prefix_decode_ws_bytes.argtypes = [I64, ctypes.POINTER(I64)]
        L.cass_prefix_decode.argtypes = [PC, P, I64, P, I64, I64, I32, P, P, I64, P]
        _lib = L
    return _lib


def _check(status):
    if status != CASS_OK:
        raise CassError(status, lib().cass_last_error().decode())


def _stream(stream):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _params(fmt, mant_bits, block, keep):
    return CassParams(int(fmt), int(mant_bits), int(block), int(keep))


# ------------------------------------------------------------ C-named calls


def cass_encode_ws_bytes(rows, cols, params: CassParams) -> int:
    n = ctypes.c_int64(0)
    _check(lib().cass_encode_ws_bytes(rows, cols, ctypes.byref(params), ctypes.byref(n)))
    return n.value


def _ld(w):
    assert w.dim() == 2 and w.stride(1) == 1, "rows must be contiguous"
    return w.stride(0)


def cass_encode_plan(w, params: CassParams, ws, stream=None) -> CassPlan:
    """w: [rows, cols] bf16 patterns with unit column stride (any row stride)."""
    rows, cols = w.shape
    plan = CassPlan()
    _check(lib().cass_encode_plan(_ptr(w), rows, cols, _ld(w), ctypes.byref(params), _ptr(ws),
                                  ws.numel() * ws.element_size(), _stream(stream),
                                  ctypes.byref(plan)))
    return plan


def cass_encode_tensor(w, plan: CassPlan, spec, verif, stream=None) -> CassTensor:
    t = CassTensor()
    _check(lib().cass_encode_tensor(_ptr(w), _ld(w), ctypes.byref(plan), _ptr(spec),
                                    spec.numel(), _ptr(verif), verif.numel(), _stream(stream),
                                    ctypes.byref(t)))
    return t


def cass_tensor_describe(spec_header: bytes, spec, verif_header: bytes | None = None,
                         verif=None) -> CassTensor:
    t = CassTensor()
    sh = ctypes.create_string_buffer(bytes(spec_header[:256]), 256)
    vh = ctypes.create_string_buffer(bytes(verif_header[:256]), 256) if verif_header else None
    _check(lib().cass_tensor_describe(sh, _ptr(spec), spec.numel(), vh, _ptr(verif),
                                      0 if verif is None else verif.numel(), ctypes.byref(t)))
    return t


def cass_draft_gemv(W: CassTensor, x, y, stream=None):
    """x: [batch, >=cols] bf16 patterns on the GPU; y: [batch, >=rows] float32."""
    assert x.dim() == 2 and y.dim() == 2 and x.shape[0] == y.shape[0]
    _check(lib().cass_draft_gemv(ctypes.byref(W), _ptr(x), x.shape[0], x.stride(0), _ptr(y),
                                 y.stride(0), _stream(stream)))


def cass_verify_gemm(W: CassTensor, X, Y, stream=None):
    assert X.dim() == 2 and Y.dim() == 2 and X.shape[0] == Y.shape[0]
    _check(lib().cass_verify_gemm(ctypes.byref(W), _ptr(X), X.shape[0], X.stride(0), _ptr(Y),
                                  Y.stride(0), _stream(stream)))


def cass_reconstruct(W: CassTensor, out, stream=None):
    _check(lib().cass_reconstruct(ctypes.byref(W), _ptr(out), _stream(stream)))


def cass_draft_decode(W: CassTensor, out, stream=None):
    _check(lib().cass_draft_decode(ctypes.byref(W), _ptr(out), _stream(stream)))


def cass_tensor_validate(spec: np.ndarray, verif: np.ndarray | None = None) -> int:
    spec = np.ascontiguousarray(spec, dtype=np.uint8)
    vp = None
    if verif is not None:
        verif = np.ascontiguousarray(verif, dtype=np.uint8)
        vp = verif.ctypes.data_as(ctypes.c_void_p)
    return lib().cass_tensor_validate(spec.ctypes.data_as(ctypes.c_void_p), spec.size, vp,
                                      0 if verif is None else verif.size)


def cass_version() -> int:
    return lib().cass_version()


def cass_debug_flags() -> int:
    """CASS_DBG_* bits the debug library's device bounds checks raised since
    the previous call (then cleared); raises CassError on the release library."""
    v = ctypes.c_uint32(0)
    _check(lib().cass_debug_flags(ctypes.byref(v)))
    return int(v.value)


def cass_set_option(name: str, value: int):
    """Select an internal code path (tests and benchmarks; 0 = default)."""
    _check(lib().cass_set_option(name.encode(), int(value)))


def cass_stream_read(buf, out, stream=None):
    """Streaming read of every byte of buf (device, 16-byte multiple) into a
    fold of CASS_STREAM_READ_BLOCKS words in out: the read-bandwidth ceiling."""
    _check(lib().cass_stream_read(_ptr(buf), buf.numel() * buf.element_size(), _ptr(out),
                                  _stream(stream)))


# ------------------------------------------------------------ convenience


class Encoded:
    """Device buffers of one encoded tensor plus its descriptor."""

    def __init__(self, desc: CassTensor, spec, verif, plan: CassPlan):
        self.desc, self.spec, self.verif, self.plan = desc, spec, verif, plan

    @property
    def rows(self):
        return self.desc.rows

    @property
    def cols(self):
        return self.desc.cols

    @property
    def spec_bytes(self):
        return self.desc.spec_bytes

    @property
    def verif_bytes(self):
        return self.desc.verif_bytes


def encode(w, keep: int, mant_bits: int, block: int = 256, fmt: int = CASS_FMT_C1_UNARY,
           stream=None, ws=None) -> Encoded:
    """Encode a [rows, cols] bf16-pattern tensor on the GPU (int16/uint16/bfloat16)."""
    import torch
    rows, cols = w.shape
    p = _params(fmt, mant_bits, block, keep)
    need = cass_encode_ws_bytes(rows, cols, p)
    if ws is None or ws.numel() < need:
        ws = torch.empty(need, dtype=torch.uint8, device=w.device)
    plan = cass_encode_plan(w, p, ws, stream)
    spec = torch.empty(plan.spec_bytes, dtype=torch.uint8, device=w.device)
    verif = torch.empty(plan.verif_bytes, dtype=torch.uint8, device=w.device)
    desc = cass_encode_tensor(w, plan, spec, verif, stream)
    enc = Encoded(desc, spec, verif, plan)
    enc._ws = ws  # the workspace must outlive the packing pass
    return enc


# ------------------------------------------------- comparison exponent codecs


def _hist_arg(hist):
    h = np.ascontiguousarray(hist, dtype=np.uint64)
    assert h.size == 256
    return h, h.ctypes.data_as(ctypes.c_void_p)


def cass_prefix_code_huffman(hist, max_len: int) -> CassPrefixCode:
    c = CassPrefixCode()
    h, hp = _hist_arg(hist)
    _check(lib().cass_prefix_code_huffman(hp, max_len, ctypes.byref(c)))
    return c


def cass_prefix_code_unary(hist) -> CassPrefixCode:
    c = CassPrefixCode()
    h, hp = _hist_arg(hist)
    _check(lib().cass_prefix_code_unary(hp, ctypes.byref(c)))
    return c


def cass_prefix_stream_bits(code: CassPrefixCode, hist) -> int:
    n = ctypes.c_int64(0)
    h, hp = _hist_arg(hist)
    _check(lib().cass_prefix_stream_bits(ctypes.byref(code), hp, ctypes.byref(n)))
    return n.value


def cass_prefix_encode(code: CassPrefixCode, sym, block, stream, blkoff, stream_h=None):
    _check(lib().cass_prefix_encode(ctypes.byref(code), _ptr(sym), sym.numel(), block, _ptr(stream),
                                    stream.numel() * stream.element_size(), _ptr(blkoff),
                                    _stream(stream_h)))


def cass_prefix_decode_ws_bytes(stream_bytes: int) -> int:
    n = ctypes.c_int64(0)
    _check(lib().cass_prefix_decode_ws_bytes(stream_bytes, ctypes.byref(n)))
    return n.value


def cass_prefix_decode(code: CassPrefixCode, stream, blkoff, n, block, method, out, ws=None,
                       stream_h=None):
    _check(lib().cass_prefix_decode(ctypes.byref(code), _ptr(stream),
                                    stream.numel() * stream.element_size(), _ptr(blkoff), n, block,
                                    method, _ptr(out), _ptr(ws),
                                    0 if ws is None else ws.numel() * ws.element_size(),
                                    _stream(stream_h)))


# ------------------------------------------------------------------ KV cache


def cass_kv_bytes(params: CassKvParams):
    sb, vb, tb = ctypes.c_int64(0), ctypes.c_int64(0), ctypes.c_int64(0)
    _check(lib().cass_kv_bytes(ctypes.byref(params), ctypes.byref(sb), ctypes.byref(vb),
                               ctypes.byref(tb)))
    return sb.value, vb.value, tb.value


def cass_kv_init(params: CassKvParams, spec, verif, state, stream=None) -> CassKv:
    kv = CassKv()
    _check(lib().cass_kv_init(ctypes.byref(kv), ctypes.byref(params), _ptr(spec), _ptr(verif),
                              _ptr(state), _stream(stream)))
    return kv


def cass_kv_append_ws_bytes(kv: CassKv, ntok: int) -> int:
    n = ctypes.c_int64(0)
    _check(lib().cass_kv_append_ws_bytes(ctypes.byref(kv), ntok, ctypes.byref(n)))
    return n.value


def cass_kv_append_encode(kv: CassKv, k, v, ws, stream=None):
    """k, v: [ntok, n_kv_heads, head_dim] bf16 patterns on the GPU."""
    ntok = k.shape[0]
    _check(lib().cass_kv_append_encode(ctypes.byref(kv), _ptr(k), _ptr(v), ntok, _ptr(ws),
                                       ws.numel() * ws.element_size(), _stream(stream)))


def cass_kv_truncate(kv: CassKv, tokens: int, stream=None):
    _check(lib().cass_kv_truncate(ctypes.byref(kv), int(tokens), _stream(stream)))


def cass_kv_status(kv: CassKv, stream=None):
    t, f = ctypes.c_int64(0), ctypes.c_uint32(0)
    _check(lib().cass_kv_status(ctypes.byref(kv), ctypes.byref(t), ctypes.byref(f),
                                _stream(stream)))
    return t.value, f.value


def cass_kv_decode(kv: CassKv, exact: bool, out, stream=None):
    _check(lib().cass_kv_decode(ctypes.byref(kv), int(bool(exact)), _ptr(out), _stream(stream)))


def cass_kv_attn_ws_bytes(kv: CassKv, nq: int, n_q_heads: int) -> int:
    n = ctypes.c_int64(0)
    _check(lib().cass_kv_attn_ws_bytes(ctypes.byref(kv), nq, n_q_heads, ctypes.byref(n)))
    return n.value


def cass_kv_draft_attn(kv: CassKv, q, scale, out, ws, stream=None):
    """q: [n_q_heads, head_dim] bf16; out: [n_q_heads, head_dim] float32."""
    _check(lib().cass_kv_draft_attn(ctypes.byref(kv), _ptr(q), q.shape[0], float(scale),
                                    _ptr(out), _ptr(ws), ws.numel() * ws.element_size(),
                                    _stream(stream)))


def cass_kv_draft_attn_static(kv: CassKv, q, scale, out, stream=None):
    """cass_kv_draft_attn with the library's fixed device scratch instead of a
    workspace (allocates nothing; calls on one device must not overlap)."""
    _check(lib().cass_kv_draft_attn_static(ctypes.byref(kv), _ptr(q), q.shape[0], float(scale),
                                           _ptr(out), _stream(stream)))


def cass_kv_verify_attn(kv: CassKv, q, scale, out, ws, stream=None):
    """q: [nq, n_q_heads, head_dim] bf16; out: same shape, float32."""
    _check(lib().cass_kv_verify_attn(ctypes.byref(kv), _ptr(q), q.shape[0], q.shape[1],
                                     float(scale), _ptr(out), _ptr(ws),
                                     ws.numel() * ws.element_size(), _stream(stream)))


class KvCache:
    """Device buffers (torch) of one layer's compressed KV cache and its descriptor."""

    def __init__(self, n_kv_heads, head_dim, keep, mant_bits, max_tokens, code_cap_bits=None,
                 vcode_cap_bits=None, device="cuda", stream=None, fmt=CASS_FMT_C1_UNARY):
        import torch
        # default capacities: 8 bits per kept (C-1 codes) or 24 per kept
        # (C-2 residues), 8 per pruned value
        code_cap_bits = code_cap_bits or max_tokens * keep * (8 if fmt == CASS_FMT_C1_UNARY else 24)
        vcode_cap_bits = vcode_cap_bits or max_tokens * (head_dim - keep) * 8
        self.params = CassKvParams(n_kv_heads, head_dim, keep, mant_bits, max_tokens,
                                   code_cap_bits, vcode_cap_bits, fmt)
        sb, vb, tb = cass_kv_bytes(self.params)
        self.spec = torch.empty(sb, dtype=torch.uint8, device=device)
        self.verif = torch.empty(vb, dtype=torch.uint8, device=device)
        self.state = torch.empty(tb, dtype=torch.uint8, device=device)
        self.kv = cass_kv_init(self.params, self.spec, self.verif, self.state, stream)
        self._ws = None

    def append(self, k, v, stream=None):
        import torch
        need = cass_kv_append_ws_bytes(self.kv, k.shape[0])
        if self._ws is None or self._ws.numel() < need:
            self._ws = torch.empty(max(need, 1), dtype=torch.uint8, device=k.device)
        cass_kv_append_encode(self.kv, k, v, self._ws, stream)

    def truncate(self, tokens, stream=None):
        cass_kv_truncate(self.kv, tokens, stream)

    @property
    def tokens(self):
        return self.kv.tokens
