"""Seeded synthetic inputs for the compressed-MLP matmul workloads.

This module only draws numbers.  It holds none of the codec's or the matmul's
arithmetic, so both the CPU oracle (``oracle/``) and the HIP path
(``mlp_matmul_amd``) may take their inputs from it without sharing any of the
method between them.

The Unweight page (Cloudflare, "Unweight: how we compressed an LLM 22% without
sacrificing quality", section "Why compression is harder than you'd think" and
the introduction) measures on trained Llama-3.1-8B MLP weights.  Those weights
are not available here, so every input is synthetic with Llama-3.1-8B's MLP
shapes: gate and up are 14336x4096 (out x in), down is 4096x14336.

Recipe (fixed order, numpy ``default_rng``):
  1. weights ~ standard_normal(float32) * sigma   (sigma per row for workload 4)
  2. outlier mask = random() < p
  3. outlier values ~ standard_normal(float32) * s at the masked positions
  4. round float32 -> bfloat16, round-to-nearest-even
  5. activations ~ standard_normal(float32) -> bfloat16 RNE (own stream)

Seeds: the small single-matrix workload uses ``default_rng(0)`` for weights
then activations.  Every other workload ``c`` uses
``default_rng([c, layer, m, k])`` with m = 0 gate, 1 up, 2 down and k = 0 for
weights, 1 for activations.  The 32-layer stack draws each layer's outlier rate
from ``default_rng([5, layer, 9, 0])``.
"""
from __future__ import annotations

import numpy as np

LLAMA_HIDDEN = 4096
LLAMA_FFN = 14336

# (rows, cols) of each MLP matrix, stored as torch Linear.weight [out, in].
MLP_SHAPES = {
    0: (LLAMA_FFN, LLAMA_HIDDEN),   # gate
    1: (LLAMA_FFN, LLAMA_HIDDEN),   # up
    2: (LLAMA_HIDDEN, LLAMA_FFN),   # down
}
MATRIX_NAMES = {0: "gate", 1: "up", 2: "down"}

# Outlier rate of the 32-layer stack is uniform in [0.01%, 0.2%].
STACK_P_LO = 1e-4
STACK_P_HI = 2e-3


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest even.

    NaNs stay NaN (quiet bit forced), infinities stay infinite.  The rounding
    add is done in 32-bit arithmetic: for every non-NaN pattern the sum stays
    below 2^32 (the largest finite magnitude 0x7F7FFFFF plus 0x8000, with the
    sign bit at most 0xFF807FFF), and NaNs are replaced afterwards.
    """
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    with np.errstate(over="ignore"):
        r = ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(a)
    if nan.any():
        r[nan] = ((u[nan] >> np.uint32(16)) | np.uint32(0x40)).astype(np.uint16)
    return r


def gaussian_weights(rng: np.random.Generator, rows: int, cols: int,
                     sigma: float = 0.02, p_out: float = 0.0,
                     s_out: float = 0.0, row_sigma=None) -> np.ndarray:
    """bf16 bits [rows, cols]: N(0, sigma) plus Bernoulli(p_out) N(0, s_out) outliers."""
    w = rng.standard_normal((rows, cols), dtype=np.float32)
    if row_sigma is not None:
        w *= np.asarray(row_sigma, dtype=np.float32)[:, None]
    else:
        w *= np.float32(sigma)
    if p_out > 0.0:
        mask = rng.random((rows, cols)) < p_out
        n = int(mask.sum())
        w[mask] = rng.standard_normal(n, dtype=np.float32) * np.float32(s_out)
    return f32_to_bf16_bits(w)


def gaussian_activations(rng: np.random.Generator, batch: int, cols: int) -> np.ndarray:
    """bf16 bits [batch, cols] drawn N(0, 1)."""
    return f32_to_bf16_bits(rng.standard_normal((batch, cols), dtype=np.float32))


# ---------------------------------------------------------------- workload 1
def small_matrix(batch: int = 1):
    """512x1024 bf16 N(0,0.02) with 0.1% N(0,1) outliers and a 1x1024 N(0,1)
    activation, both from default_rng(0).  Returns (W bits, X bits)."""
    rng = np.random.default_rng(0)
    w = gaussian_weights(rng, 512, 1024, sigma=0.02, p_out=1e-3, s_out=1.0)
    x = gaussian_activations(rng, batch, 1024)
    return w, x


# ------------------------------------------------------- workloads 2, 3, 4, 5
def stack_outlier_rate(layer: int) -> float:
    u = np.random.default_rng([5, layer, 9, 0]).random()
    return STACK_P_LO + u * (STACK_P_HI - STACK_P_LO)


def layer_weight(workload: int, layer: int, m: int, shape=None) -> np.ndarray:
    """bf16 bits of MLP matrix m (0 gate, 1 up, 2 down) of one layer.

    workload 2 and 3: N(0,0.02) + 0.05% N(0,0.5) outliers.
    workload 4: per-row sigma_r log-uniform in [0.005, 0.05], no outliers.
    workload 5: N(0,0.02) + per-layer outlier rate in [0.01%, 0.2%] of N(0,0.5).
    ``shape`` overrides Llama's (rows, cols) for reduced-size tests.
    """
    rows, cols = shape if shape is not None else MLP_SHAPES[m]
    rng = np.random.default_rng([workload, layer, m, 0])
    if workload in (2, 3):
        return gaussian_weights(rng, rows, cols, 0.02, 5e-4, 0.5)
    if workload == 4:
        u = rng.random(rows)
        lo, hi = np.log(0.005), np.log(0.05)
        row_sigma = np.exp(lo + u * (hi - lo)).astype(np.float32)
        return gaussian_weights(rng, rows, cols, row_sigma=row_sigma)
    if workload == 5:
        return gaussian_weights(rng, rows, cols, 0.02, stack_outlier_rate(layer), 0.5)
    raise ValueError(f"no layer weights for workload {workload}")


def layer_activation(workload: int, layer: int, m: int, batch: int, cols=None) -> np.ndarray:
    """bf16 bits [batch, cols] of the activation fed to matrix m."""
    if cols is None:
        cols = MLP_SHAPES[m][1]
    rng = np.random.default_rng([workload, layer, m, 1])
    return gaussian_activations(rng, batch, cols)


def random_bf16_bits(seed: int, n: int) -> np.ndarray:
    """Uniformly random 16-bit patterns: every exponent, NaNs and subnormals."""
    return np.random.default_rng(seed).integers(0, 1 << 16, size=n, dtype=np.uint16)


def geometric_exponent_matrix(rows: int = 1024, cols: int = 4096, long_tile: int = 3, seed: int = 12):
    """bf16 bits whose 16 exponents (110..125) occur with counts N/2, N/4, ...,
    N/2^15, N/2^15 (N = rows*cols, a power of two), so every exponent is in
    the top-16 palette and no group is verbatim, and the frequencies are
    geometric.  Tile ``long_tile`` (4096 consecutive elements) holds only
    exponents of the ten rarest classes, in proportion to their counts; the
    rest are shuffled over the other tiles.  Sign and mantissa are uniform.
    A stress input for stream layout: the rarest classes are the longest
    codewords, so that tile's stream is much longer than the average tile."""
    n = rows * cols
    assert n & (n - 1) == 0 and n >= 1 << 16
    rng = np.random.default_rng(seed)
    exps = np.arange(110, 126, dtype=np.int64)
    counts = np.array([n >> k for k in range(1, 16)] + [n >> 15], dtype=np.int64)
    rare = np.arange(7, 16)                                   # the nine rarest classes
    # 4096 elements of the rare classes, drawn without replacement
    pool = np.repeat(exps[rare], counts[rare])
    pick = rng.permutation(pool.size)[:4096]
    tile_e = pool[pick]
    left = np.concatenate([np.repeat(exps, counts)[np.repeat(np.arange(16), counts) < 7],
                           np.delete(pool, pick)])
    left = left[rng.permutation(left.size)]
    t0 = long_tile * 4096
    e = np.concatenate([left[:t0], tile_e, left[t0:]])
    sm = rng.integers(0, 256, size=n, dtype=np.int64)
    bits = ((sm & 0x80) << 8) | (e << 7) | (sm & 0x7F)
    return bits.astype(np.uint16).reshape(rows, cols)


# ------------------------------------------------------------- attention
# Llama-3.1-8B attention projections (grouped-query: 8 KV heads of 128), the
# second workload on the same codec.  The page compresses only the MLP
# weights; no statistics of the attention weights are given, so they are
# drawn like the MLP's (N(0,0.02) with 0.05 % N(0,0.5) outliers).
ATTN_SHAPES = {
    "q": (4096, 4096),
    "k": (1024, 4096),
    "v": (1024, 4096),
    "o": (4096, 4096),
}
ATTN_IDS = {"q": 0, "k": 1, "v": 2, "o": 3}


def attention_weight(layer: int, name: str, shape=None) -> np.ndarray:
    """bf16 bits of one attention projection, default_rng([6, layer, id, 0])."""
    rows, cols = shape if shape is not None else ATTN_SHAPES[name]
    rng = np.random.default_rng([6, layer, ATTN_IDS[name], 0])
    return gaussian_weights(rng, rows, cols, 0.02, 5e-4, 0.5)


def attention_activation(layer: int, name: str, batch: int) -> np.ndarray:
    """bf16 bits [batch, cols] fed to one attention projection."""
    rng = np.random.default_rng([6, layer, ATTN_IDS[name], 1])
    return gaussian_activations(rng, batch, ATTN_SHAPES[name][1])


# Llama-3.1-8B's output projection (the unembedding matrix, vocabulary x
# hidden), the embedding-sized matmul of the model.
LM_HEAD_SHAPE = (128256, 4096)


def lm_head_weight(shape=None) -> np.ndarray:
    """bf16 bits of the output projection, default_rng([7, 0, 0, 0]):
    N(0, 0.02) with Binomial(N, 5e-4) outliers N(0, 0.5) at uniformly drawn
    positions (the same distribution as the other weights, drawn without a
    per-element mask so that a 525M-element matrix generates in seconds)."""
    rows, cols = shape if shape is not None else LM_HEAD_SHAPE
    rng = np.random.default_rng([7, 0, 0, 0])
    w = rng.standard_normal((rows, cols), dtype=np.float32)
    w *= np.float32(0.02)
    n = int(rng.binomial(rows * cols, 5e-4))
    pos = rng.integers(0, rows * cols, n)
    w.reshape(-1)[pos] = rng.standard_normal(n, dtype=np.float32) * np.float32(0.5)
    # round to nearest even as f32_to_bf16_bits does, in 32-bit arithmetic:
    # the draws are finite, so the sum cannot carry out of 32 bits
    u = w.view(np.uint32)
    return ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)


def lm_head_activation(batch: int, cols: int = LM_HEAD_SHAPE[1]) -> np.ndarray:
    """bf16 bits [batch, cols] N(0, 1) fed to the output projection."""
    return gaussian_activations(np.random.default_rng([7, 0, 0, 1]), batch, cols)
