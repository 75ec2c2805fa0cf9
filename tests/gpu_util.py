"""Helpers for the GPU parity tests: host<->device copies and the tolerance
check.  Expected values always come from the oracle or from the seeded
inputs themselves, never from the HIP path."""
import numpy as np

from oracle import numerics

# Matmul tolerance: |Y_gpu - Y_ref| <= TOL * sum_c |W[r,c] X[b,c]| per output.
TOL = 2e-3


def to_dev_bf16(bits):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def from_dev_bits(t):
    import torch
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def from_dev_u8(t):
    return t.cpu().numpy().view(np.uint8)


def assert_matmul_close(Y_gpu, w_bits, x_bits, rows=None, what=""):
    """Y_gpu: [B, R] (or [B, len(rows)]) float32 numpy; compares to the fp64 oracle."""
    if rows is None:
        ref = numerics.matmul(w_bits, x_bits)
        S = numerics.abs_bound(w_bits, x_bits)
    else:
        ref, S = numerics.matmul_rows(w_bits, x_bits, rows)
    Y = np.asarray(Y_gpu, dtype=np.float64)
    assert Y.shape == ref.shape, (Y.shape, ref.shape)
    err = np.abs(Y - ref)
    bad = err > TOL * S
    zero = S == 0
    bad |= zero & (Y != 0)
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(f"{what}: {int(bad.sum())} outputs out of tolerance; first {tuple(i)} "
                             f"gpu={Y[tuple(i)]!r} ref={ref[tuple(i)]!r} S={S[tuple(i)]!r}")
    return float((err / np.where(S > 0, S, 1)).max())


def print_case(msg):
    print(msg, flush=True)


def bf16_order_key(b):
    """bf16 bit patterns as integers ordered like their values (so that one
    ulp apart means a difference of 1)."""
    b = np.asarray(b).astype(np.int64)
    return np.where(b & 0x8000, -(b & 0x7FFF), b & 0x7FFF)


def check_silu_product(h_bits, g, u, what=""):
    """h within one bf16 ulp of bf16(SiLU(g)*u) computed in fp64 on the same g, u."""
    href = numerics.f64_to_bf16_bits(numerics.silu_mul(g, u))
    d = np.abs(bf16_order_key(h_bits) - bf16_order_key(href)).max() if href.size else 0
    assert d <= 1, f"{what}: h off by {d} bf16 ulps"
