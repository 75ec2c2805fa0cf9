"""Oracle numerics: bf16 values, the fp64 matmul and the SiLU chain.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The Unweight page (Cloudflare, "How the reconstructive matmul works") says the
fused kernel rebuilds bf16 weights on chip and multiplies them; since the codec
is lossless, the product it must reach is the plain definition
Y[b, r] = sum_c W[r, c] * X[b, c].  bf16 values convert exactly to fp64 and a
bf16 x bf16 product is exact in fp64, so the only rounding here is fp64
summation (relative error ~K * 2^-53).
"""
from __future__ import annotations

import numpy as np


def bf16_to_f64(bits) -> np.ndarray:
    """Exact value of bf16 bit patterns: the upper half of an fp32."""
    b = np.asarray(bits, dtype=np.uint16)
    with np.errstate(invalid="ignore"):
        return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def matmul(w_bits, x_bits) -> np.ndarray:
    """Y = X . W^T in fp64.  W is [R, C] bf16 bits, X is [B, C] bf16 bits."""
    W = bf16_to_f64(w_bits)
    X = bf16_to_f64(x_bits)
    return X @ W.T


def abs_bound(w_bits, x_bits) -> np.ndarray:
    """S[b, r] = sum_c |W[r, c] * X[b, c]|, the scale of the error tolerance."""
    W = np.abs(bf16_to_f64(w_bits))
    X = np.abs(bf16_to_f64(x_bits))
    return X @ W.T


def matmul_rows(w_bits, x_bits, rows) -> tuple:
    """Y and S restricted to the given output rows (for sampled checks)."""
    Wr = np.asarray(w_bits)[np.asarray(rows)]
    return matmul(Wr, x_bits), abs_bound(Wr, x_bits)


def silu(z: np.ndarray) -> np.ndarray:
    """SiLU(z) = z / (1 + exp(-z)) in fp64."""
    z = np.asarray(z, dtype=np.float64)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def f64_to_bf16_bits(v) -> np.ndarray:
    """Round fp64 values to the nearest bf16, ties to even.

    A finite nonzero |v| with binary exponent k (2^k <= |v| < 2^(k+1)) is
    scaled exactly by 2^(7-k) into [128, 256) and rounded half-to-even there
    (numpy's rint); below the normal range the quantum is fixed at 2^-133.
    A carry to 256 moves to the next binade; overflow gives infinity.
    """
    v = np.asarray(v, dtype=np.float64)
    sign = np.where(np.signbit(v), 0x8000, 0).astype(np.int64)
    a = np.abs(v)
    out = np.zeros(v.shape, dtype=np.int64)
    finite = np.isfinite(a) & (a > 0)
    with np.errstate(all="ignore"):
        _, k = np.frexp(np.where(finite, a, 1.0))
    k = k.astype(np.int64) - 1                       # a = 1.f * 2^k
    sub = finite & (k < -126)
    nrm = finite & ~sub
    # normal range
    a = np.where(finite, a, 0.0)
    q = np.rint(np.ldexp(a, np.where(nrm, 7 - k, 0)))
    carry = nrm & (q == 256)
    q = np.where(carry, 128, q)
    E = np.where(carry, k + 1, k) + 127
    big = nrm & (E >= 255)
    out = np.where(nrm, (E << 7) | (q.astype(np.int64) - 128), out)
    out = np.where(big, 0x7F80, out)
    # subnormal range: multiples of 2^-133 (a carry to 128 is the smallest normal)
    qs = np.rint(np.ldexp(a, np.where(sub, 133, 0))).astype(np.int64)
    out = np.where(sub, qs, out)
    out = np.where(np.isinf(v), 0x7F80, out)
    out = out | sign
    out = np.where(np.isnan(v), 0x7FC0, out)
    return out.astype(np.uint16)


def silu_mul(g, u) -> np.ndarray:
    """h = SiLU(g) * u in fp64 (inputs are the fp32 gate and up projections)."""
    return silu(np.asarray(g, dtype=np.float64)) * np.asarray(u, dtype=np.float64)
