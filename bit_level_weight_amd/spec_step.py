"""One self-speculative decoding step over compressed layers (a timing shell).

Cassandra review (marsggbo.github.io), section 1: the draft model guesses k
tokens one after another and the target checks all of them in one parallel
pass; section 3.1: the draft reads only the speculation data of every weight
and KV tensor (zero-filled), the target reads both streams; section 4 quotes
acceptance rates of 0.74 to 0.91.

Per decoder layer (its linear maps fused as q|k|v, o, gate|up and down, plus
the layer's compressed KV cache) one step runs, all in the library's kernels
through its C ABI (this module prepares arguments once and orders the calls):

  k draft passes, each for one token, per layer:
      q|k|v draft GEMV -> append the token's keys and values to the cache
      (online encoder) -> draft attention over the cache -> o, gate|up, down
      draft GEMVs
  per layer, the verification pass for the k+1 tokens (the step's input token
  and the k drafts):
      the k drafted tokens leave the cache (their keys and values came from the
      draft) -> q|k|v verification GEMM -> append the k+1 tokens' keys and
      values -> verification attention (causal over the block) -> o, gate|up,
      down verification GEMMs
  acceptance: each cache keeps the input token and the accepted drafts.

Synthetic parts: the activations between the linear maps (norms, rotary
embedding, the gated activation and residual adds are elementwise work outside
this path) are resident bf16 inputs made up front, and so are the queries and
the new tokens' keys and values; acceptance is a seeded run of Bernoulli(alpha)
successes, at most k (greedy acceptance needs trained weights).
"""
from __future__ import annotations

import ctypes

import numpy as np

from . import CassKv, CassError, lib

MATS = ("qkv", "o", "gu", "down")


def expected_tokens(alpha: float, k: int) -> float:
    """Mean tokens one step yields when each draft is accepted with
    probability alpha until the first rejection: the accepted run plus the
    target's own token, sum_{i=0..k} alpha^i."""
    return float(sum(alpha ** i for i in range(k + 1)))


def draw_accepted(rng: np.random.Generator, alpha: float, k: int) -> int:
    """Accepted drafts of one step: leading successes of k Bernoulli(alpha) trials."""
    a = 0
    while a < k and rng.random() < alpha:
        a += 1
    return a


class SpecStep:
    """Buffers and call sequence of one speculative step.

    layers: one dict per layer, MATS -> Encoded (q|k|v rows = (Hq + 2 H) * D);
    caches: one KvCache per layer (same parameters); n_q_heads: query heads.
    inputs: device bf16 patterns (int16) to use instead of the random ones:
    "x" (MATS -> [k+1, cols], row i = token i's input), "q" [k+1, Hq, D],
    "k_new"/"v_new" [k+1, H, D] (the verified tokens), "k_draft"/"v_draft"
    [k, H, D] (the draft's keys and values of tokens 0..k-1).
    """

    def __init__(self, layers, caches, n_q_heads: int, k: int = 4, seed: int = 0,
                 scale: float | None = None, inputs: dict | None = None):
        import torch
        self.torch = torch
        self.L = lib()
        self.layers, self.caches, self.k = layers, caches, k
        p = caches[0].params
        self.H, self.D, self.Hq = p.n_kv_heads, p.head_dim, n_q_heads
        self.scale = float(scale if scale is not None else 1.0 / np.sqrt(self.D))
        n = k + 1
        g = torch.Generator(device="cuda")
        g.manual_seed(seed)

        def bf16(*shape):
            return torch.randn(shape, generator=g, device="cuda").to(torch.bfloat16).view(torch.int16)

        cols = {m: layers[0][m].cols for m in MATS}
        rows = {m: layers[0][m].rows for m in MATS}
        for lay in layers:
            for m in MATS:
                if (lay[m].rows, lay[m].cols) != (rows[m], cols[m]):
                    raise ValueError("layers differ in shape")
        inputs = inputs or {}
        self.x = inputs.get("x") or {m: bf16(n, cols[m]) for m in MATS}
        self.q = inputs.get("q", None)
        self.q = self.q if self.q is not None else bf16(n, n_q_heads, self.D)
        for name, t in (("k_new", n), ("v_new", n), ("k_draft", k), ("v_draft", k)):
            v = inputs.get(name, None)
            setattr(self, name, v if v is not None else bf16(t, self.H, self.D))
        shapes = {"q": (n, n_q_heads, self.D), "k_new": (n, self.H, self.D),
                  "v_new": (n, self.H, self.D), "k_draft": (k, self.H, self.D),
                  "v_draft": (k, self.H, self.D)}
        for name, shp in shapes.items():
            t = getattr(self, name)
            if tuple(t.shape) != shp or not t.is_contiguous() or t.element_size() != 2:
                raise ValueError(f"{name}: expected contiguous 16-bit {shp}")
        for m in MATS:
            t = self.x[m]
            if tuple(t.shape) != (n, cols[m]) or not t.is_contiguous() or t.element_size() != 2:
                raise ValueError(f"x[{m}]: expected contiguous 16-bit {(n, cols[m])}")
        f32 = dict(dtype=torch.float32, device="cuda")
        nl = len(layers)
        self.y_draft = [{m: torch.empty((k, rows[m]), **f32) for m in MATS} for _ in range(nl)]
        self.y_ver = [{m: torch.empty((n, rows[m]), **f32) for m in MATS} for _ in range(nl)]
        self.a_draft = [torch.empty((k, n_q_heads, self.D), **f32) for _ in range(nl)]
        self.a_ver = [torch.empty((n, n_q_heads, self.D), **f32) for _ in range(nl)]
        # workspaces sized for the fullest cache the step can see
        full = CassKv.from_buffer_copy(caches[0].kv)
        full.tokens = p.max_tokens
        need = ctypes.c_int64(0)
        self._check(self.L.cass_kv_append_ws_bytes(ctypes.byref(full), n, ctypes.byref(need)))
        self.app_ws = torch.empty(max(need.value, 1), dtype=torch.uint8, device="cuda")
        self._check(self.L.cass_kv_attn_ws_bytes(ctypes.byref(full), n, n_q_heads,
                                                 ctypes.byref(need)))
        self.attn_ws = torch.empty(max(need.value, 1), dtype=torch.uint8, device="cuda")
        self._desc = [{m: ctypes.byref(lay[m].desc) for m in MATS} for lay in layers]
        self._kv = [ctypes.byref(c.kv) for c in caches]
        self._ldx = {m: cols[m] for m in MATS}
        self._ldy = {m: rows[m] for m in MATS}

    def _check(self, status):
        if status != 0:
            raise CassError(status, self.L.cass_last_error().decode())

    @staticmethod
    def _p(t, offset_elems=0):
        return ctypes.c_void_p(t.data_ptr() + offset_elems * t.element_size())

    def tokens(self) -> int:
        return int(self.caches[0].kv.tokens)

    def draft_pass(self, i: int, stream) -> None:
        """Draft pass i (0-based): one token through every layer on draft data."""
        L, c, P, s = self.L, self._check, self._p, stream
        kvb = self.H * self.D
        for li in range(len(self.layers)):
            d, y, kv = self._desc[li], self.y_draft[li], self._kv[li]

            def gemv(m):
                c(L.cass_draft_gemv(d[m], P(self.x[m], i * self._ldx[m]), 1, self._ldx[m],
                                    P(y[m], i * self._ldy[m]), self._ldy[m], s))

            gemv("qkv")
            c(L.cass_kv_append_encode(kv, P(self.k_draft, i * kvb), P(self.v_draft, i * kvb), 1,
                                      P(self.app_ws), self.app_ws.numel(), s))
            c(L.cass_kv_draft_attn(kv, P(self.q, i * self.Hq * self.D), self.Hq, self.scale,
                                   P(self.a_draft[li], i * self.Hq * self.D), P(self.attn_ws),
                                   self.attn_ws.numel(), s))
            for m in ("o", "gu", "down"):
                gemv(m)

    def verify_pass(self, t0: int, stream) -> None:
        """The k+1 tokens through every layer on exact data; each cache first
        drops everything past t0 (the drafted tokens)."""
        L, c, P, s = self.L, self._check, self._p, stream
        n = self.k + 1
        for li in range(len(self.layers)):
            d, y, kv = self._desc[li], self.y_ver[li], self._kv[li]

            def gemm(m):
                c(L.cass_verify_gemm(d[m], P(self.x[m]), n, self._ldx[m], P(y[m]), self._ldy[m], s))

            c(L.cass_kv_truncate(kv, t0, s))
            gemm("qkv")
            c(L.cass_kv_append_encode(kv, P(self.k_new), P(self.v_new), n, P(self.app_ws),
                                      self.app_ws.numel(), s))
            c(L.cass_kv_verify_attn(kv, P(self.q), n, self.Hq, self.scale, P(self.a_ver[li]),
                                    P(self.attn_ws), self.attn_ws.numel(), s))
            for m in ("o", "gu", "down"):
                gemm(m)

    def step(self, accepted: int, stream=None, keep: bool = True) -> int:
        """One step; the caches then hold the input token and `accepted`
        drafts (keep=False: back to the step's start, for fixed-size timing).
        Returns the tokens the step yields (accepted + 1)."""
        if not 0 <= accepted <= self.k:
            raise ValueError("accepted must be in 0..k")
        s = ctypes.c_void_p((stream or self.torch.cuda.current_stream()).cuda_stream)
        t0 = self.tokens()
        if t0 + self.k + 1 > self.caches[0].params.max_tokens:
            raise CassError(3, "cache full")
        for i in range(self.k):
            self.draft_pass(i, s)
        self.verify_pass(t0, s)
        end = t0 + 1 + accepted if keep else t0
        for kv in self._kv:
            self._check(self.L.cass_kv_truncate(kv, end, s))
        return accepted + 1

    def run(self, phase: str, stream=None) -> None:
        """One phase at a fixed context, the caches left as found: "step"
        (the whole step), "draft" (the k draft passes) or "verify" (the
        verification pass of the k+1 tokens)."""
        if phase == "step":
            self.step(0, stream, keep=False)
            return
        s = ctypes.c_void_p((stream or self.torch.cuda.current_stream()).cuda_stream)
        t0 = self.tokens()
        if phase == "draft":
            for i in range(self.k):
                self.draft_pass(i, s)
        elif phase == "verify":
            self.verify_pass(t0, s)
        else:
            raise ValueError(phase)
        for kv in self._kv:
            self._check(self.L.cass_kv_truncate(kv, t0, s))

    def capture(self, phase: str = "step"):
        """A HIP graph of one phase (see run) that leaves the caches as it
        found them; replaying it repeats the phase at the same context."""
        torch = self.torch
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            self.run(phase, side)  # warm: kernel attributes, lazy module loads
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            self.run(phase, torch.cuda.current_stream())
        torch.cuda.synchronize()
        return g
