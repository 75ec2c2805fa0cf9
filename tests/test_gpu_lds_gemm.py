"""GPU parity of the tiled MFMA kernel that rebuilds each weight once per
workgroup into a shared LDS tile (above batch 64 by default for single
matrices, above batch 32 for the fused gate/up pair).

Every tile configuration, prefetch depth and workgroup order sums each
output over the same K order (the tiling only moves rows and batch columns
between waves and workgroups), so they must agree bit for bit at one split;
the rebuilt weights are bit-exact, so the palette, exponent and bf16 sources
must agree bit for bit too.  Against the fp64 oracle every output is within
2e-3 of sum |w*x|; one-hot activations pin the rebuilt weights exactly.
"""
import itertools

import numpy as np
import pytest

import mlp_matmul_amd as uw
from oracle import codec, numerics
import workloads
from tests.gpu_util import assert_matmul_close, print_case, to_dev_bf16

pytestmark = pytest.mark.gpu

# (config, prefetch depth, workgroup order) the kernel is instantiated with
# (prefetch 4 and 6 run as 3 with 256 columns):
# configs 0/1/2 are 128 rows x 64/128/256 batch columns
_VARIANTS = list(itertools.product((0, 1, 2), (2, 3, 4, 6), (0, 1)))


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    uw.lib()
    return torch


def _force(monkeypatch, cfg, p, order):
    monkeypatch.setenv("UW_MFMA_LDS", "1")
    monkeypatch.setenv("UW_LDS_CFG", str(cfg))
    monkeypatch.setenv("UW_LDS_P", str(p))
    monkeypatch.setenv("UW_LDS_ORDER", str(order))


def _three_sources(dm, W, exps, X, split, scr):
    return [f().cpu().numpy().view(np.uint32) for f in (
        lambda: uw.gemm_recon_pal(dm, None, X, kernel=uw.UW_KERNEL_MFMA, split_k=split, scratch=scr),
        lambda: uw.gemm_recon_exp(dm, exps, X, kernel=uw.UW_KERNEL_MFMA, split_k=split, scratch=scr),
        lambda: uw.gemm_bf16(W, X, kernel=uw.UW_KERNEL_MFMA, split_k=split, scratch=scr))]


@pytest.mark.parametrize("R,C,B,split", [(300, 4096 + 1024, 70, 1), (300, 4096 + 1024, 300, 3),
                                         (129, 2048, 64, 2), (257, 1024, 130, 1)])
def test_lds_gemm_all_variants(torch_cuda, monkeypatch, R, C, B, split):
    """Row bands past R (300 = 2 x 128 + 44), batch tiles past B, K-slices of
    uneven length whose row segments straddle 4096-weight tiles: every
    variant bit-identical, the three sources bit-identical, and within
    tolerance of the oracle."""
    import torch
    rng = np.random.default_rng(R * 7 + C + B + split)
    w = workloads.gaussian_weights(rng, R, C, 0.02, 0.004, 1.0)
    x = workloads.gaussian_activations(np.random.default_rng(C + B), B, C)
    dm = uw.compress(w).to_device()
    X, W = to_dev_bf16(x), to_dev_bf16(w)
    exps = uw.decode_exponents(dm)
    scr = torch.empty(split * 4 * B * R + 256, dtype=torch.uint8, device="cuda")
    ref = None
    for cfg, p, order in _VARIANTS:
        print_case(f"lds gemm R={R} C={C} B={B} split={split} cfg={cfg} p={p} order={order}")
        _force(monkeypatch, cfg, p, order)
        pal, exp, bf = _three_sources(dm, W, exps, X, split, scr)
        assert np.array_equal(pal, exp), f"exp source cfg={cfg} p={p} order={order}"
        assert np.array_equal(pal, bf), f"bf16 source cfg={cfg} p={p} order={order}"
        if ref is None:
            ref = pal
            assert_matmul_close(pal.view(np.float32), w, x, what=f"lds gemm R={R} C={C} B={B} split={split}")
        else:
            assert np.array_equal(pal, ref), f"cfg={cfg} p={p} order={order} differs from cfg=0 p=2 order=0"


@pytest.mark.parametrize("cfg", [0, 1, 2])
def test_lds_gemm_one_hot(torch_cuda, monkeypatch, cfg):
    """X = 70 rows of the identity: Y[b, r] = W[r, c_b] exactly, including
    columns inside groups that are verbatim in many rows, for every tile
    configuration and with split-K (partial sums of zeros are exact)."""
    w, _ = workloads.small_matrix()
    dm = uw.compress(w).to_device()
    vflag = codec.encode(w).vflag.reshape(w.shape[0], -1)
    hot = np.argsort(-vflag.sum(axis=0))[:10] * 64 + np.arange(10) * 6
    cols = np.concatenate([hot, np.arange(60) * 17 + 1])
    x = np.zeros((len(cols), w.shape[1]), dtype=np.uint16)
    x[np.arange(len(cols)), cols] = 0x3F80
    X = to_dev_bf16(x)
    expect = numerics.bf16_to_f64(w[:, cols].T).astype(np.float32).view(np.uint32)
    import torch
    scr = torch.empty(4 * 4 * len(cols) * w.shape[0] + 256, dtype=torch.uint8, device="cuda")
    for split in (1, 4):
        print_case(f"lds gemm one-hot cfg={cfg} split={split}")
        _force(monkeypatch, cfg, 2, 1)
        got = uw.gemm_recon_pal(dm, None, X, kernel=uw.UW_KERNEL_MFMA, split_k=split, scratch=scr)
        assert np.array_equal(got.cpu().numpy().view(np.uint32), expect), f"split={split}"


def test_lds_gemm_mostly_verbatim(torch_cuda, monkeypatch):
    """85 % of the groups verbatim (exponents spread over 25 binades): the
    per-step verbatim flag and slot come from the staged tables."""
    print_case("lds gemm mostly verbatim")
    rng = np.random.default_rng(96)
    R, C, B = 200, 2048, 96
    wide = np.repeat(rng.random((R, C // 64)) < 0.85, 64, axis=1)
    scale = np.where(wide, np.exp2(rng.integers(-12, 13, (R, C))), 1.0)
    w = workloads.f32_to_bf16_bits((rng.standard_normal((R, C)) * 0.02 * scale).astype(np.float32))
    assert codec.encode(w).vflag.mean() > 0.5
    x = workloads.gaussian_activations(np.random.default_rng(7), B, C)
    dm = uw.compress(w).to_device()
    X = to_dev_bf16(x)
    _force(monkeypatch, 1, 2, 1)
    Y = uw.gemm_recon_pal(dm, None, X, kernel=uw.UW_KERNEL_MFMA, split_k=1)
    assert_matmul_close(Y.cpu().numpy(), w, x, what="lds gemm mostly verbatim")
    W = to_dev_bf16(w)
    Yb = uw.gemm_bf16(W, X, kernel=uw.UW_KERNEL_MFMA, split_k=1)
    assert np.array_equal(Y.cpu().numpy().view(np.uint32), Yb.cpu().numpy().view(np.uint32))


def test_lds_gemm_empty_slices(torch_cuda, monkeypatch):
    """split 8 over 4 steps: four K-slices are empty and write zero partial
    sums; the total is still the full product."""
    print_case("lds gemm empty slices")
    import torch
    R, C, B, split = 140, 256, 64, 8
    w = workloads.gaussian_weights(np.random.default_rng(3), R, C, 0.02, 0.004, 1.0)
    x = workloads.gaussian_activations(np.random.default_rng(4), B, C)
    dm = uw.compress(w).to_device()
    scr = torch.empty(split * 4 * B * R + 256, dtype=torch.uint8, device="cuda")
    _force(monkeypatch, 0, 2, 1)
    Y = uw.gemm_recon_pal(dm, None, to_dev_bf16(x), kernel=uw.UW_KERNEL_MFMA, split_k=split, scratch=scr)
    assert_matmul_close(Y.cpu().numpy(), w, x, what="lds gemm empty slices")


def test_lds_gemm_default_choice(torch_cuda):
    """Without overrides the library takes this kernel above batch 64 (the
    split it resolves to fits the scratch that uw_scratch_bytes reports) and
    matches the oracle; batch 64 stays on the register-rebuilding kernel."""
    print_case("lds gemm default choice")
    R, C = 384, 4096
    w = workloads.gaussian_weights(np.random.default_rng(11), R, C, 0.02, 0.004, 1.0)
    dm = uw.compress(w).to_device()
    for B in (64, 65, 100, 200):
        x = workloads.gaussian_activations(np.random.default_rng(B), B, C)
        scr = uw.alloc_scratch(uw.UW_PIPE_DIRECT, R, C, B, 0)
        Y = uw.matmul(dm, to_dev_bf16(x), pipeline=uw.UW_PIPE_DIRECT, kernel=uw.UW_KERNEL_MFMA, split_k=0,
                      scratch=scr)
        assert_matmul_close(Y.cpu().numpy(), w, x, what=f"lds gemm default B={B}")


def _bf16_key(b):
    b = np.asarray(b).astype(np.int64)
    return np.where(b & 0x8000, -(b & 0x7FFF), b & 0x7FFF)


@pytest.mark.parametrize("R,C,B", [(300, 4096 + 1024, 33), (129, 2048, 64), (300, 4096 + 1024, 70), (129, 2048, 128),
                                   (257, 1024, 129), (200, 1088, 300), (2088, 4096, 200)])
def test_lds_gate_up_pair(torch_cuda, monkeypatch, R, C, B):
    """The fused gate/up pair (uw_mlp_gate_up above batch 32; 64-row bands x
    64, 128 or 256 batch columns, no split): g and u bit for bit equal to
    single launches of the same kernel at split 1 (every tiling sums each
    output over K in the same order), h bit for bit equal to
    uw_silu_mul_bf16 on them and to the h-only call; g, u within tolerance
    of the oracle, h within one bf16 ulp of bf16(SiLU(g)*u) in fp64.  Bands
    past R, batch tiles past B, row segments straddling tiles."""
    print_case(f"lds gate/up pair R={R} C={C} B={B}")
    import torch
    from tests.gpu_util import from_dev_bits
    rng = np.random.default_rng(R + 3 * C + B)
    wg = workloads.gaussian_weights(rng, R, C, 0.02, 0.004, 1.0)
    wu = workloads.gaussian_weights(rng, R, C, 0.03, 0.002, 2.0)
    x = workloads.gaussian_activations(np.random.default_rng(B * 7), B, C)
    dg, du = uw.compress(wg).to_device(), uw.compress(wu).to_device()
    X = to_dev_bf16(x)
    g = torch.empty((B, R), dtype=torch.float32, device="cuda")
    u = torch.empty_like(g)
    h = uw.mlp_gate_up(dg, du, X, g=g, u=u)
    h_only = uw.mlp_gate_up(dg, du, X)
    _force(monkeypatch, 0 if B <= 128 else 1, 2, 1)       # the LDS-tile kernel at every batch
    g2 = uw.gemm_recon_pal(dg, None, X, kernel=uw.UW_KERNEL_MFMA, split_k=1)
    u2 = uw.gemm_recon_pal(du, None, X, kernel=uw.UW_KERNEL_MFMA, split_k=1)
    h2 = uw.silu_mul_bf16(g2, u2)
    gn, un = g.cpu().numpy(), u.cpu().numpy()
    assert np.array_equal(gn.view(np.uint32), g2.cpu().numpy().view(np.uint32)), "g"
    assert np.array_equal(un.view(np.uint32), u2.cpu().numpy().view(np.uint32)), "u"
    hb = from_dev_bits(h)
    assert np.array_equal(hb, from_dev_bits(h2)), "h"
    assert np.array_equal(hb, from_dev_bits(h_only)), "h without g/u"
    rows = None if R * C * B <= 300 * 5120 * 70 else np.arange(0, R, 7)
    if rows is None:
        assert_matmul_close(gn, wg, x, what="pair gate")
        assert_matmul_close(un, wu, x, what="pair up")
    else:
        assert_matmul_close(gn[:, rows], wg, x, rows=rows, what="pair gate")
        assert_matmul_close(un[:, rows], wu, x, rows=rows, what="pair up")
    href = numerics.f64_to_bf16_bits(numerics.silu_mul(gn.astype(np.float64), un.astype(np.float64)))
    assert np.abs(_bf16_key(hb) - _bf16_key(href)).max() <= 1


def test_lds_gate_up_pair_rejects(torch_cuda):
    """On a matrix too short for the skinny pairs, batch 17-32 has no fused
    pair (uw_mlp_gate_up reports it unsupported); batch 33 takes the
    LDS-tile pair."""
    print_case("lds gate/up pair batch range")
    w = workloads.gaussian_weights(np.random.default_rng(5), 256, 1024, 0.02, 0.0, 1.0)
    d = uw.compress(w).to_device()
    for B in (17, 32):
        X = to_dev_bf16(workloads.gaussian_activations(np.random.default_rng(6), B, 1024))
        with pytest.raises(uw.UnweightError) as e:
            uw.mlp_gate_up(d, d, X)
        assert e.value.code == uw.UW_EUNSUPPORTED, B
    uw.mlp_gate_up(d, d, to_dev_bf16(workloads.gaussian_activations(np.random.default_rng(6), 33, 1024)))
