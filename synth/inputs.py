"""Seeded synthetic tensors with the shapes and value mix of the workloads.

Recipe (the same for every consumer):
  * values: ``numpy.random.default_rng(seed).standard_normal(dtype=float32)``
    scaled by sigma, then rounded to bfloat16 with round-to-nearest-even;
  * seed = 1_000_000*config + 1000*layer + matrix_id, with matrix ids
    q=0 k=1 v=2 o=3 gate=4 up=5 down=6 and KV keys=7 values=8;
  * activations / queries: N(0,1) bf16 with seed 1_000_000*config + 999_000 + t;
  * weight outliers: round(0.01*C) input columns, drawn by a permutation from the
    same generator after the values, are multiplied by 10 before rounding;
  * KV outliers: 4 channels of the 128 per head, fixed over tokens, drawn
    separately for keys and values, multiplied by 8 before rounding.

Shapes follow the Llama-3-8B and Qwen3-4B decoder layers named by the pages
(Cassandra review, marsggbo.github.io, section 4: the evaluated models).  Trained
weights are not available; these Gaussian tensors stand in for them.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "bf16_from_f32", "f32_from_bf16", "seed_for", "act_seed", "keep_count",
    "weight", "activations", "kv_tensor", "all_bf16_patterns",
    "LLAMA3_8B", "QWEN3_4B", "weight_wide", "layer_matrices", "fused_layer",
]

MATRIX_ID = {"q": 0, "k": 1, "v": 2, "o": 3, "gate": 4, "up": 5, "down": 6,
             "kv_k": 7, "kv_v": 8}

# (rows, cols) = (out_features, in_features) of each projection.
LLAMA3_8B = {
    "q": (4096, 4096), "k": (1024, 4096), "v": (1024, 4096), "o": (4096, 4096),
    "gate": (14336, 4096), "up": (14336, 4096), "down": (4096, 14336),
}
QWEN3_4B = {
    "q": (4096, 2560), "k": (1024, 2560), "v": (1024, 2560), "o": (2560, 4096),
    "gate": (9728, 2560), "up": (9728, 2560), "down": (2560, 9728),
}


def bf16_from_f32(a) -> np.ndarray:
    """Round float32 to bfloat16 bit patterns (uint16), nearest-even; NaN stays NaN."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    out = r.astype(np.uint16)
    nan = np.isnan(a)
    if nan.any():
        out[nan] = ((u[nan] >> 16) | 0x40).astype(np.uint16)
    return out


def f32_from_bf16(b) -> np.ndarray:
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def seed_for(config: int, layer: int, matrix: str) -> int:
    return 1_000_000 * config + 1000 * layer + MATRIX_ID[matrix]


def act_seed(config: int, t: int) -> int:
    return 1_000_000 * config + 999_000 + t


def keep_count(keep_ratio: float, group: int) -> int:
    """Number of values kept per group of ``group`` values: floor(ratio*group + 1/2)."""
    return int(np.floor(keep_ratio * group + 0.5))


def weight(rows: int, cols: int, seed: int, sigma: float = 0.02,
           outlier_frac: float = 0.0, outlier_scale: float = 10.0) -> np.ndarray:
    """bf16 [rows, cols] ~ N(0, sigma^2), with round(outlier_frac*cols) input columns x scale."""
    rng = np.random.default_rng(seed)
    a = rng.standard_normal((rows, cols), dtype=np.float32)
    a *= np.float32(sigma)
    n_out = int(round(outlier_frac * cols))
    if n_out:
        cols_sel = rng.permutation(cols)[:n_out]
        a[:, cols_sel] *= np.float32(outlier_scale)
    return bf16_from_f32(a)


def activations(n: int, cols: int, config: int, t0: int = 0) -> np.ndarray:
    """bf16 [n, cols] ~ N(0,1); row t uses seed act_seed(config, t0 + t)."""
    out = np.empty((n, cols), dtype=np.uint16)
    for t in range(n):
        rng = np.random.default_rng(act_seed(config, t0 + t))
        out[t] = bf16_from_f32(rng.standard_normal(cols, dtype=np.float32))
    return out


def weight_wide(rows: int, cols: int, seed: int, binades: int = 48) -> np.ndarray:
    """bf16 [rows, cols]: N(0,1) times 2^-u with u uniform in [0, binades),
    so exponents spread over ~binades values (long exponent codes)."""
    rng = np.random.default_rng(seed)
    a = rng.standard_normal((rows, cols), dtype=np.float32)
    a *= np.exp2(-rng.uniform(0.0, binades, size=(rows, cols))).astype(np.float32)
    return bf16_from_f32(a)


def kv_tensor(tokens: int, heads: int, dim: int, seed: int,
              n_outlier: int = 4, outlier_scale: float = 8.0) -> np.ndarray:
    """bf16 [tokens, heads, dim] ~ N(0,1) with n_outlier fixed channels per head x scale."""
    rng = np.random.default_rng(seed)
    a = rng.standard_normal((tokens, heads, dim), dtype=np.float32)
    for h in range(heads):
        ch = rng.permutation(dim)[:n_outlier]
        a[:, h, ch] *= np.float32(outlier_scale)
    return bf16_from_f32(a)


def all_bf16_patterns(seed: int | None = None) -> np.ndarray:
    """A 256x256 uint16 array holding each of the 65536 bit patterns exactly once."""
    p = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    if seed is not None:
        p = np.random.default_rng(seed).permutation(p)
    return p.reshape(256, 256)


def layer_matrices(shapes: dict, config: int, layer: int, outlier_frac: float,
                   sigma: float = 0.02, names=None) -> dict:
    """Generate the named projection matrices of one decoder layer."""
    names = names or list(shapes)
    return {n: weight(*shapes[n], seed_for(config, layer, n), sigma, outlier_frac)
            for n in names}


def fused_layer(shapes: dict, config: int, layer: int, outlier_frac: float,
                sigma: float = 0.02) -> dict:
    """The layer as the four GEMV operands of a decode step: qkv (q|k|v rows
    stacked), o, gu (gate|up rows stacked) and down."""
    m = layer_matrices(shapes, config, layer, outlier_frac, sigma)
    return {
        "qkv": np.concatenate([m["q"], m["k"], m["v"]], axis=0),
        "o": m["o"],
        "gu": np.concatenate([m["gate"], m["up"]], axis=0),
        "down": m["down"],
    }
