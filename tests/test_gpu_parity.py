"""GPU parity: libunweight's gfx950 kernels against the CPU oracle.

Decoders are bit-exact on every element; matmuls are within 2e-3 of
sum |w*x| per output (fp32 accumulation against the fp64 oracle); the
one-hot activations pin the in-kernel reconstruction bit-exactly.
Every input comes from the seeded generators in workloads.py.
"""
import os

import numpy as np
import pytest

import mlp_matmul_amd as uw
from oracle import codec, numerics
import workloads
from tests.gpu_util import (TOL, assert_matmul_close, from_dev_bits, from_dev_u8, print_case,
                            to_dev_bf16)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    uw.lib()
    return torch


def _expected_nibbles(w):
    """4-bit palette indices from the oracle's palette and verbatim flags."""
    e, _ = codec.split_fields(w.ravel())
    pal = codec.top16_palette(codec.exponent_histogram(e))
    vflag = codec.verbatim_flags(e, pal)
    return codec.pack_nibbles(codec.element_symbols(e, pal, vflag))


def _check_decoders(dm, w, exp_nib=None):
    import torch
    full = uw.decode_full(dm)
    exps = uw.decode_exponents(dm)
    nib = uw.transcode_palette(dm)
    torch.cuda.synchronize()
    assert np.array_equal(from_dev_bits(full), w), "full decode"
    assert np.array_equal(from_dev_u8(exps), ((w >> 7) & 0xFF).astype(np.uint8)), "exponent decode"
    if exp_nib is None:
        exp_nib = _expected_nibbles(w)
    assert np.array_equal(from_dev_u8(nib), exp_nib), "palette transcode"
    return full, exps, nib


# ------------------------------------------------------------------ decoders
def test_decoders_small_workload(torch_cuda):
    print_case("decoders: 512x1024 small workload")
    w, _ = workloads.small_matrix()
    ref = codec.encode(w)
    dm = uw.compress(w).to_device()
    _check_decoders(dm, w, ref.nib)
    # the decoders match the oracle's own decode of the same stream too
    assert np.array_equal(codec.decode_parallel(ref, "full"), w)


@pytest.mark.parametrize("case", ["single", "spread", "allverbatim", "special", "partial", "one_group", "empty"])
def test_decoders_edge_cases(torch_cuda, case):
    print_case(f"decoders edge case {case}")
    rng = np.random.default_rng(7)
    if case == "single":
        w = ((rng.integers(0, 2, (9, 192)).astype(np.uint16) << 15) | (119 << 7)
             | rng.integers(0, 128, (9, 192)).astype(np.uint16)).astype(np.uint16)
    elif case == "spread":
        w = ((rng.integers(0, 2, (33, 256)).astype(np.uint16) << 15)
             | (rng.integers(90, 122, (33, 256)).astype(np.uint16) << 7)
             | rng.integers(0, 128, (33, 256)).astype(np.uint16)).astype(np.uint16)
    elif case == "allverbatim":
        w = workloads.random_bf16_bits(11, 64 * 700).reshape(350, 128)
    elif case == "special":
        w = workloads.gaussian_weights(rng, 70, 320, 0.02, 0.01, 1.0)
        flat = w.ravel()
        sp = np.array([0, 0x8000, 1, 0x807F, 0x7F80, 0xFF80, 0x7FC0, 0x7F81, 0xFFFF], np.uint16)
        flat[rng.choice(flat.size, sp.size * 5, replace=False)] = np.tile(sp, 5)
    elif case == "partial":
        w = workloads.gaussian_weights(rng, 129, 64 * 3, 0.02, 0.003, 1.0)
    elif case == "one_group":
        w = workloads.gaussian_weights(rng, 1, 64, 0.02)
    else:
        w = np.zeros((0, 128), np.uint16)
    dm = uw.compress(w).to_device()
    if w.size == 0:
        uw.decode_full(dm)
        return
    _check_decoders(dm, w)


def test_decoders_long_tile(torch_cuda):
    """A tile whose stream is longer than the 4 KiB the decoders stage in one
    pass, coded with 13-15-bit codewords (past the 12-bit multi-symbol
    table): all three decoders stay bit-exact, and so does the reconstructive
    GEMV that consumes the transcoded nibbles."""
    print_case("decoders long tile (geometric exponent frequencies)")
    w = workloads.geometric_exponent_matrix()
    b = uw.compress(w)
    assert b.info().max_tile_bytes > 4096 and b.info().lmax == 15
    dm = b.to_device()
    _, _, nib = _check_decoders(dm, w)
    x = workloads.gaussian_activations(np.random.default_rng(3), 1, w.shape[1])
    Y = uw.gemm_recon_pal(dm, nib, to_dev_bf16(x), kernel=uw.UW_KERNEL_GEMV)
    assert_matmul_close(Y.cpu().numpy(), w, x, what="long tile: palette transcode + GEMV")


@pytest.mark.parametrize("name", ["q", "k", "v", "o"])
def test_attention_projections_full_size(torch_cuda, name):
    """The second workload on the same codec: Llama-3.1-8B attention
    projections at full size.  Decoders bit-exact (K only, the other shapes
    add nothing new to the decoders), direct-palette matmul through the
    library's kernel choice within tolerance at batch 1, 4 and 16."""
    print_case(f"attention projection {name} full size")
    w = workloads.attention_weight(0, name)
    dm = uw.compress(w).to_device()
    if name == "k":
        _check_decoders(dm, w)
    for B in (1, 4, 16):
        x = workloads.attention_activation(0, name, B)
        Y = uw.matmul(dm, to_dev_bf16(x), pipeline=uw.UW_PIPE_DIRECT, kernel=uw.UW_KERNEL_AUTO, split_k=0,
                      scratch=uw.alloc_scratch(uw.UW_PIPE_DIRECT, w.shape[0], w.shape[1], B, 0))
        rows = np.random.default_rng(B).choice(w.shape[0], 256, replace=False)
        assert_matmul_close(Y.cpu().numpy()[:, rows], w, x, rows=rows, what=f"{name} B={B}")


def test_lm_head_full_size(torch_cuda):
    """The largest matrix of the model, the output projection (128256 x 4096,
    525M weights, the benchmark's lm_head workload): full and exponent decodes
    bit-exact on every element, direct-palette matmul through the library's
    kernel choice at batch 1, 4 and 16 on sampled rows against the fp64
    oracle."""
    import torch
    print_case("lm head 128256x4096 full size")
    w = workloads.lm_head_weight()
    dm = uw.compress(w, emit_palette=True).to_device()
    full = uw.decode_full(dm)
    torch.cuda.synchronize()
    assert np.array_equal(from_dev_bits(full), w), "full decode"
    del full
    exps = uw.decode_exponents(dm)
    torch.cuda.synchronize()
    assert np.array_equal(from_dev_u8(exps), ((w >> 7) & 0xFF).astype(np.uint8)), "exponent decode"
    del exps
    rows = np.sort(np.random.default_rng(11).choice(w.shape[0], 256, replace=False))
    for B in (1, 4, 16):
        x = workloads.lm_head_activation(B)
        Y = uw.matmul(dm, to_dev_bf16(x), pipeline=uw.UW_PIPE_DIRECT, kernel=uw.UW_KERNEL_AUTO, split_k=0,
                      scratch=uw.alloc_scratch(uw.UW_PIPE_DIRECT, w.shape[0], w.shape[1], B, 0))
        assert_matmul_close(Y.cpu().numpy()[:, rows], w, x, rows=rows, what=f"lm head B={B}")


@pytest.mark.parametrize("wl,m", [(2, 0), (2, 2), (4, 1), (5, 2)])
def test_decoders_full_size(torch_cuda, wl, m):
    print_case(f"decoders full size workload {wl} matrix {m}")
    w = workloads.layer_weight(wl, 0 if wl != 5 else 17, m)
    dm = uw.compress(w).to_device()
    _check_decoders(dm, w)


# --------------------------------------------------------------- one-hot pin
def _one_hot(cols, C):
    x = np.zeros((len(cols), C), np.uint16)
    x[np.arange(len(cols)), cols] = 0x3F80     # bf16 1.0
    return x


@pytest.mark.parametrize("kernel", [uw.UW_KERNEL_GEMV, uw.UW_KERNEL_MFMA, uw.UW_KERNEL_SKINNY])
def test_one_hot_reveals_rebuilt_weights(torch_cuda, kernel):
    """With X = rows of the identity, Y[b, r] = W[r, c_b] exactly: the fused
    kernels reveal the weights they rebuilt without writing them out."""
    print_case(f"one-hot pin kernel {kernel}")
    w, _ = workloads.small_matrix()
    dm = uw.compress(w).to_device()
    exps = uw.decode_exponents(dm)
    vflag = codec.encode(w).vflag.reshape(w.shape[0], -1)
    # columns inside groups that are verbatim in many rows, plus ordinary ones
    hot = np.argsort(-vflag.sum(axis=0))[:8] * 64 + np.array([0, 5, 17, 63, 31, 40, 2, 62])
    cols = np.concatenate([hot, np.arange(8) * 111 + 3])
    x = _one_hot(cols, w.shape[1])
    X = to_dev_bf16(x)
    expect = numerics.bf16_to_f64(w[:, cols].T).astype(np.float32)
    outs = {
        "bf16": uw.gemm_bf16(to_dev_bf16(w), X, kernel=kernel),
        "direct": uw.gemm_recon_pal(dm, None, X, kernel=kernel),
        "exp": uw.gemm_recon_exp(dm, exps, X, kernel=kernel),
    }
    torch_cuda.cuda.synchronize()
    for name, Y in outs.items():
        got = Y.cpu().numpy()
        assert np.array_equal(got.view(np.uint32), expect.view(np.uint32)), name


# ------------------------------------------------------------------ matmuls
def _x(seed, B, C):
    return workloads.gaussian_activations(np.random.default_rng(seed), B, C)


@pytest.mark.parametrize("B", [1, 2, 3, 4, 7, 8, 12, 16])
def test_gemv_small_workload(torch_cuda, B):
    print_case(f"gemv small workload B={B}")
    w, _ = workloads.small_matrix()
    x = _x(B, B, w.shape[1])
    dm = uw.compress(w).to_device()
    X = to_dev_bf16(x)
    exps = uw.decode_exponents(dm)
    for name, Y in [("bf16", uw.gemm_bf16(to_dev_bf16(w), X, kernel=uw.UW_KERNEL_GEMV)),
                    ("direct", uw.gemm_recon_pal(dm, None, X, kernel=uw.UW_KERNEL_GEMV)),
                    ("exp", uw.gemm_recon_exp(dm, exps, X, kernel=uw.UW_KERNEL_GEMV))]:
        assert_matmul_close(Y.cpu().numpy(), w, x, what=f"gemv {name} B={B}")


@pytest.mark.parametrize("B", [1, 5, 16, 17, 33, 64, 100, 128, 200, 256, 300])
def test_mfma_small_workload(torch_cuda, B):
    print_case(f"mfma small workload B={B}")
    w, _ = workloads.small_matrix()
    x = _x(100 + B, B, w.shape[1])
    dm = uw.compress(w).to_device()
    X = to_dev_bf16(x)
    exps = uw.decode_exponents(dm)
    for name, Y in [("bf16", uw.gemm_bf16(to_dev_bf16(w), X, kernel=uw.UW_KERNEL_MFMA)),
                    ("direct", uw.gemm_recon_pal(dm, None, X, kernel=uw.UW_KERNEL_MFMA)),
                    ("exp", uw.gemm_recon_exp(dm, exps, X, kernel=uw.UW_KERNEL_MFMA))]:
        assert_matmul_close(Y.cpu().numpy(), w, x, what=f"mfma {name} B={B}")


@pytest.mark.parametrize("R,C,B,split", [(300, 8192, 70, 1), (300, 8192, 70, 2), (129, 4096 + 1024, 40, 1),
                                         (257, 12288, 130, 4), (64, 2048, 17, 1), (96, 2048, 33, 2)])
def test_mfma_verbatim_tables_in_registers_and_lds(torch_cuda, monkeypatch, R, C, B, split):
    """The tiled kernel's two ways to find verbatim groups: bitmap words kept
    in registers (K-slices of at most 4096 columns) and the band's tables
    staged in LDS (forced with UW_MFMA_REGTAB=0, and the only way for longer
    slices): bit-identical to each other and within tolerance of the oracle,
    on row segments that straddle tiles and a matrix whose groups are mostly
    verbatim."""
    print_case(f"mfma verbatim tables R={R} C={C} B={B} split={split}")
    rng = np.random.default_rng(R + C + B + split)
    if R == 96:
        wide = np.repeat(rng.random((R, C // 64)) < 0.85, 64, axis=1)
        scale = np.where(wide, np.exp2(rng.integers(-12, 13, (R, C))), 1.0)
        w = workloads.f32_to_bf16_bits((rng.standard_normal((R, C)) * 0.02 * scale).astype(np.float32))
    else:
        w = workloads.gaussian_weights(rng, R, C, 0.02, 0.004, 1.0)
    x = _x(C + B, B, C)
    dm = uw.compress(w).to_device()
    X = to_dev_bf16(x)
    import torch
    scr = torch.empty(split * 4 * B * R + 256, dtype=torch.uint8, device="cuda")
    outs = []
    monkeypatch.setenv("UW_MFMA_LDS", "0")       # the register-rebuilding tiled kernel
    for regtab in ("1", "0"):
        monkeypatch.setenv("UW_MFMA_REGTAB", regtab)
        outs.append(uw.gemm_recon_pal(dm, None, X, kernel=uw.UW_KERNEL_MFMA, split_k=split,
                                      scratch=scr).cpu().numpy())
    assert np.array_equal(outs[0].view(np.uint32), outs[1].view(np.uint32))
    assert_matmul_close(outs[0], w, x, what=f"mfma R={R} C={C} B={B} split={split}")


# every (row blocks per wave, waves per workgroup, batch blocks, prefetch
# depth) the tiled kernel is instantiated with (tuning overrides UW_MFMA_RBW /
# _WPG / _NB / _PD)
_MFMA_TILINGS = [(1, 4, 4, 1), (1, 4, 4, 2), (1, 4, 8, 1), (1, 4, 8, 2), (1, 8, 4, 1), (1, 8, 4, 2),
                 (1, 8, 8, 1), (1, 8, 8, 2), (2, 4, 4, 1), (2, 4, 4, 3), (2, 4, 8, 2), (2, 8, 4, 2),
                 (2, 8, 8, 1), (4, 4, 4, 3), (4, 4, 8, 1)]


@pytest.mark.parametrize("rbw,wpg,nb,pd", _MFMA_TILINGS)
def test_mfma_tilings(torch_cuda, monkeypatch, rbw, wpg, nb, pd):
    """Each tiling of the tiled kernel gives the same bits as the default one
    for the same split (the tiling moves rows and batch columns between
    waves and workgroups, never the order of a sum), on bands past R, batch
    tiles past B and K-slices whose row segments straddle tiles; the palette
    source is also checked against the oracle."""
    print_case(f"mfma tiling rbw={rbw} wpg={wpg} nb={nb} pd={pd}")
    import torch
    R, C, B, split = 300, 4096 + 1024, 70, 2
    w = workloads.gaussian_weights(np.random.default_rng(R + C + B), R, C, 0.02, 0.004, 1.0)
    x = _x(C + B + 1, B, C)
    dm = uw.compress(w).to_device()
    X = to_dev_bf16(x)
    W = to_dev_bf16(w)
    exps = uw.decode_exponents(dm)
    scr = torch.empty(split * 4 * B * R + 256, dtype=torch.uint8, device="cuda")

    def run():
        return [f(X).cpu().numpy().view(np.uint32) for f in (
            lambda X: uw.gemm_recon_pal(dm, None, X, kernel=uw.UW_KERNEL_MFMA, split_k=split, scratch=scr),
            lambda X: uw.gemm_bf16(W, X, kernel=uw.UW_KERNEL_MFMA, split_k=split, scratch=scr),
            lambda X: uw.gemm_recon_exp(dm, exps, X, kernel=uw.UW_KERNEL_MFMA, split_k=split, scratch=scr))]

    monkeypatch.setenv("UW_MFMA_LDS", "0")       # the register-rebuilding tiled kernel
    ref = run()
    for k, v in (("UW_MFMA_RBW", rbw), ("UW_MFMA_WPG", wpg), ("UW_MFMA_NB", nb), ("UW_MFMA_PD", pd)):
        monkeypatch.setenv(k, str(v))
    got = run()
    for name, a, b in zip(("direct", "bf16", "exp"), got, ref):
        assert np.array_equal(a, b), name
    assert_matmul_close(got[0].view(np.float32), w, x, what=f"mfma tiling {rbw}/{wpg}/{nb}/{pd}")


@pytest.mark.parametrize("B", [1, 2, 3, 4, 5, 7, 8, 9, 16, 17, 31, 33, 48, 64, 65, 100])
def test_skinny_small_workload(torch_cuda, B):
    print_case(f"skinny small workload B={B}")
    w, _ = workloads.small_matrix()
    x = _x(300 + B, B, w.shape[1])
    dm = uw.compress(w).to_device()
    X = to_dev_bf16(x)
    exps = uw.decode_exponents(dm)
    for name, Y in [("bf16", uw.gemm_bf16(to_dev_bf16(w), X, kernel=uw.UW_KERNEL_SKINNY)),
                    ("direct", uw.gemm_recon_pal(dm, None, X, kernel=uw.UW_KERNEL_SKINNY)),
                    ("exp", uw.gemm_recon_exp(dm, exps, X, kernel=uw.UW_KERNEL_SKINNY))]:
        assert_matmul_close(Y.cpu().numpy(), w, x, what=f"skinny {name} B={B}")


@pytest.mark.parametrize("R,C", [(1, 128), (3, 256), (37, 384), (130, 1152), (67, 2048 + 128), (19, 16384),
                                 (5, 32768)])
@pytest.mark.parametrize("B", [2, 9, 40])
def test_skinny_ragged_shapes(torch_cuda, R, C, B):
    """Row blocks past R, batch tiles past B, K-slices of unequal length, wave
    slices that are empty (C = 128) and row segments that straddle tiles."""
    print_case(f"skinny ragged R={R} C={C} B={B}")
    w = workloads.gaussian_weights(np.random.default_rng(R * C + B + 7), R, C, 0.02, 0.004, 1.0)
    x = _x(R + B + 1, B, C)
    dm = uw.compress(w).to_device()
    X = to_dev_bf16(x)
    exps = uw.decode_exponents(dm)
    for name, Y in [("bf16", uw.gemm_bf16(to_dev_bf16(w), X, kernel=uw.UW_KERNEL_SKINNY)),
                    ("direct", uw.gemm_recon_pal(dm, None, X, kernel=uw.UW_KERNEL_SKINNY)),
                    ("exp", uw.gemm_recon_exp(dm, exps, X, kernel=uw.UW_KERNEL_SKINNY))]:
        assert_matmul_close(Y.cpu().numpy(), w, x, what=f"skinny {name}")


@pytest.mark.parametrize("kw", [2, 4, 8])
@pytest.mark.parametrize("pd", [1, 2])
@pytest.mark.parametrize("rb", [1, 2])
def test_skinny_launch_shapes(torch_cuda, monkeypatch, kw, pd, rb):
    """Every K-split width, prefetch depth and row-block count the launcher
    can pick (the tuning overrides UW_SKINNY_KW / _PD / _RB), on slices of
    1..9 steps with row segments that straddle tiles, rows past R, each
    batch-tile count and each count of loaded activation row quads."""
    monkeypatch.setenv("UW_SKINNY_KW", str(kw))
    monkeypatch.setenv("UW_SKINNY_PD", str(pd))
    monkeypatch.setenv("UW_SKINNY_RB", str(rb))
    for R, C, B in [(29, 2048 + 256, 3), (45, 1152, 5), (33, 4096 + 512, 20), (17, 9216, 64)]:
        print_case(f"skinny kw={kw} pd={pd} rb={rb} R={R} C={C} B={B}")
        w = workloads.gaussian_weights(np.random.default_rng(R + C + kw + pd), R, C, 0.02, 0.004, 1.0)
        x = _x(C + B, B, C)
        dm = uw.compress(w).to_device()
        X = to_dev_bf16(x)
        exps = uw.decode_exponents(dm)
        for name, Y in [("bf16", uw.gemm_bf16(to_dev_bf16(w), X, kernel=uw.UW_KERNEL_SKINNY)),
                        ("direct", uw.gemm_recon_pal(dm, None, X, kernel=uw.UW_KERNEL_SKINNY)),
                        ("exp", uw.gemm_recon_exp(dm, exps, X, kernel=uw.UW_KERNEL_SKINNY))]:
            assert_matmul_close(Y.cpu().numpy(), w, x, what=f"skinny {name} kw={kw} pd={pd} rb={rb} C={C}")


@pytest.mark.parametrize("kw", [1, 2, 4, 8])
@pytest.mark.parametrize("d", [2, 3, 4])
@pytest.mark.parametrize("nrb", [1, 2])
def test_skinny_dma_launch_shapes(torch_cuda, monkeypatch, kw, d, nrb):
    """The skinny kernel that streams its operands through LDS by DMA
    (palette source), forced on small matrices in every K-split, ring depth
    and row-block count the launcher can pick (UW_SKINNY_DMA / UW_DMA_KW /
    _D / _NRB): slices shorter than the ring and not a multiple of it, empty
    slices (one step split eight ways), rows past R, each count of loaded
    activation row quads, row segments that straddle tiles, verbatim groups."""
    monkeypatch.setenv("UW_SKINNY_DMA", "1")
    monkeypatch.setenv("UW_DMA_KW", str(kw))
    monkeypatch.setenv("UW_DMA_D", str(d))
    monkeypatch.setenv("UW_DMA_NRB", str(nrb))
    for R, C, B in [(29, 2048 + 256, 3), (45, 1152, 5), (33, 4096 + 512, 16), (17, 9216, 9), (70, 128, 12),
                    (1, 640, 1), (40, 1152, 27), (19, 2048 + 128, 32)]:
        print_case(f"skinny dma kw={kw} d={d} nrb={nrb} R={R} C={C} B={B}")
        w = workloads.gaussian_weights(np.random.default_rng(R + C + kw + d), R, C, 0.02, 0.004, 1.0)
        x = _x(C + B + nrb, B, C)
        Y = uw.gemm_recon_pal(uw.compress(w).to_device(), None, to_dev_bf16(x), kernel=uw.UW_KERNEL_SKINNY)
        assert_matmul_close(Y.cpu().numpy(), w, x, what=f"skinny dma kw={kw} d={d} nrb={nrb} R={R} C={C} B={B}")


def test_skinny_dma_one_hot_and_verbatim(torch_cuda, monkeypatch):
    """The DMA skinny kernel rebuilds every weight exactly (one-hot columns,
    including groups verbatim in many rows) and handles matrices whose groups
    are mostly verbatim."""
    monkeypatch.setenv("UW_SKINNY_DMA", "1")
    print_case("skinny dma one-hot")
    w, _ = workloads.small_matrix()
    dm = uw.compress(w).to_device()
    vflag = codec.encode(w).vflag.reshape(w.shape[0], -1)
    hot = np.argsort(-vflag.sum(axis=0))[:8] * 64 + np.array([0, 5, 17, 63, 31, 40, 2, 62])
    cols = np.concatenate([hot, np.arange(8) * 111 + 3])
    Y = uw.gemm_recon_pal(dm, None, to_dev_bf16(_one_hot(cols, w.shape[1])), kernel=uw.UW_KERNEL_SKINNY)
    expect = numerics.bf16_to_f64(w[:, cols].T).astype(np.float32)
    assert np.array_equal(Y.cpu().numpy().view(np.uint32), expect.view(np.uint32))
    print_case("skinny dma mostly verbatim")
    rng = np.random.default_rng(12)
    R, C = 96, 2048
    wide = np.repeat(rng.random((R, C // 64)) < 0.85, 64, axis=1)
    scale = np.where(wide, np.exp2(rng.integers(-12, 13, (R, C))), 1.0)
    w = workloads.f32_to_bf16_bits((rng.standard_normal((R, C)) * 0.02 * scale).astype(np.float32))
    x = _x(13, 11, C)
    dm = uw.compress(w).to_device()
    assert 0.8 * dm.info.groups < dm.info.verbatim_groups < dm.info.groups
    Y = uw.gemm_recon_pal(dm, None, to_dev_bf16(x), kernel=uw.UW_KERNEL_SKINNY)
    assert_matmul_close(Y.cpu().numpy(), w, x, what="skinny dma verbatim")


def test_skinny_mostly_verbatim(torch_cuda):
    """About 85% of the groups hold exponents far outside the palette (stored
    verbatim), mixed with ordinary groups: the verbatim override on most lanes
    of most steps, next to palette lanes."""
    print_case("skinny mostly verbatim")
    rng = np.random.default_rng(11)
    R, C = 96, 2048
    wide = np.repeat(rng.random((R, C // 64)) < 0.85, 64, axis=1)
    scale = np.where(wide, np.exp2(rng.integers(-12, 13, (R, C))), 1.0)
    w = workloads.f32_to_bf16_bits((rng.standard_normal((R, C)) * 0.02 * scale).astype(np.float32))
    x = _x(12, 24, C)
    dm = uw.compress(w).to_device()
    assert 0.8 * dm.info.groups < dm.info.verbatim_groups < dm.info.groups
    exps = uw.decode_exponents(dm)
    for name, Y in [("direct", uw.gemm_recon_pal(dm, None, to_dev_bf16(x), kernel=uw.UW_KERNEL_SKINNY)),
                    ("exp", uw.gemm_recon_exp(dm, exps, to_dev_bf16(x), kernel=uw.UW_KERNEL_SKINNY))]:
        assert_matmul_close(Y.cpu().numpy(), w, x, what=f"skinny verbatim {name}")


def test_skinny_rejects_unsupported_width(torch_cuda):
    w = workloads.gaussian_weights(np.random.default_rng(3), 16, 192, 0.02, 0.0, 1.0)
    dm = uw.compress(w).to_device()
    X = to_dev_bf16(_x(3, 4, 192))
    with pytest.raises(uw.UnweightError) as ei:
        uw.gemm_recon_pal(dm, None, X, kernel=uw.UW_KERNEL_SKINNY)
    assert ei.value.code == uw.UW_EUNSUPPORTED
    # AUTO falls back to the tiled MFMA kernel for such widths
    Y = uw.gemm_recon_pal(dm, None, X)
    assert_matmul_close(Y.cpu().numpy(), w, _x(3, 4, 192), what="auto width 192")


@pytest.mark.parametrize("split", [2, 3, 4, 16])
def test_mfma_split_k(torch_cuda, split):
    print_case(f"mfma split_k={split}")
    w = workloads.layer_weight(2, 3, 2, shape=(200, 14336))
    x = _x(split, 40, w.shape[1])
    dm = uw.compress(w).to_device()
    X = to_dev_bf16(x)
    scratch = uw.alloc_scratch(uw.UW_PIPE_DIRECT, 200, 14336, 40, split)
    Y = uw.gemm_recon_pal(dm, None, X, kernel=uw.UW_KERNEL_MFMA, split_k=split, scratch=scratch)
    assert_matmul_close(Y.cpu().numpy(), w, x, what=f"split {split}")


def test_split_k_library_choice(torch_cuda):
    """split_k 0: the library picks the K-slices (8 for this short, wide
    matrix at batch 256) and lowers them to what the scratch holds; the
    result is within tolerance with the full scratch, a scratch for two
    slices, and none."""
    print_case("split_k 0 (library choice), R=512 C=4096 B=256")
    R, C, B = 512, 4096, 256
    w = workloads.layer_weight(2, 4, 2, shape=(R, C))
    x = _x(5, B, C)
    dm = uw.compress(w).to_device()
    X = to_dev_bf16(x)
    full = uw.scratch_bytes(uw.UW_PIPE_DIRECT, R, C, B, 0)
    assert full == uw.scratch_bytes(uw.UW_PIPE_DIRECT, R, C, B, 8) > 0
    for n in (full, uw.scratch_bytes(uw.UW_PIPE_DIRECT, R, C, B, 2), 0):
        scratch = uw._torch().empty(max(n, 16), dtype=uw._torch().uint8, device="cuda")
        Y = uw.matmul(dm, X, pipeline=uw.UW_PIPE_DIRECT, kernel=uw.UW_KERNEL_AUTO, split_k=0,
                      scratch=scratch if n else None)
        assert_matmul_close(Y.cpu().numpy(), w, x, what=f"split 0 with {n} bytes of scratch")
    # the no-plan fallback of UW_PIPE_AUTO takes the same route
    assert uw.plan_lookup(R, C, B) is None
    Y = uw.matmul(dm, X, scratch=uw._torch().empty(full, dtype=uw._torch().uint8, device="cuda"))
    assert_matmul_close(Y.cpu().numpy(), w, x, what="auto, no plan")


@pytest.mark.parametrize("R,C,B,split", [(300, 128, 20, 4), (257, 64, 70, 3), (513, 1024, 129, 16)])
def test_mfma_split_k_short_slices(torch_cuda, R, C, B, split):
    """Split-K with empty and one-step K slices, a band past R, a batch tile
    past B: every partial tile is written and summed."""
    print_case(f"mfma split short R={R} C={C} B={B} split={split}")
    w = workloads.gaussian_weights(np.random.default_rng(R + C + split), R, C, 0.02, 0.004, 1.0)
    x = _x(R * split, B, C)
    dm = uw.compress(w).to_device()
    X = to_dev_bf16(x)
    exps = uw.decode_exponents(dm)
    for p in (uw.UW_PIPE_DIRECT, uw.UW_PIPE_EXP, uw.UW_PIPE_FULL):
        scratch = uw.alloc_scratch(p, R, C, B, split)
        Y = uw.matmul(dm, X, pipeline=p, kernel=uw.UW_KERNEL_MFMA, split_k=split, scratch=scratch)
        assert_matmul_close(Y.cpu().numpy(), w, x, what=f"pipeline {p} split {split}")
    Yb = uw.gemm_bf16(to_dev_bf16(w), X, kernel=uw.UW_KERNEL_MFMA)
    assert_matmul_close(Yb.cpu().numpy(), w, x, what="bf16")
    Ye = uw.gemm_recon_exp(dm, exps, X, kernel=uw.UW_KERNEL_MFMA)
    assert_matmul_close(Ye.cpu().numpy(), w, x, what="exp")


@pytest.mark.parametrize("R,C", [(1, 64), (3, 128), (37, 192), (130, 1088), (67, 2048 + 64)])
@pytest.mark.parametrize("B", [1, 6, 16, 40])
def test_ragged_shapes(torch_cuda, R, C, B):
    print_case(f"ragged R={R} C={C} B={B}")
    w = workloads.gaussian_weights(np.random.default_rng(R * C + B), R, C, 0.02, 0.004, 1.0)
    x = _x(R + B, B, C)
    dm = uw.compress(w).to_device()
    X = to_dev_bf16(x)
    kernels = [uw.UW_KERNEL_MFMA] + ([uw.UW_KERNEL_GEMV] if B <= 16 else [])
    for k in kernels:
        for name, Y in [("bf16", uw.gemm_bf16(to_dev_bf16(w), X, kernel=k)),
                        ("direct", uw.gemm_recon_pal(dm, None, X, kernel=k))]:
            assert_matmul_close(Y.cpu().numpy(), w, x, what=f"{name} k={k}")


def test_empty_and_zero_batch(torch_cuda):
    import torch
    w = np.zeros((0, 128), np.uint16)
    dm = uw.compress(w).to_device()
    X = to_dev_bf16(_x(0, 3, 128))
    Y = uw.gemm_recon_pal(dm, None, X)
    assert Y.shape == (3, 0)
    w2, _ = workloads.small_matrix()
    dm2 = uw.compress(w2).to_device()
    X0 = torch.empty((0, 1024), dtype=torch.bfloat16, device="cuda")
    Y0 = uw.gemm_recon_pal(dm2, None, X0)
    assert Y0.shape == (0, 512)


# ---------------------------------------------------------------- pipelines
@pytest.mark.parametrize("B", [1, 4, 16, 64])
def test_four_pipelines_small_workload(torch_cuda, B):
    print_case(f"pipelines small workload B={B}")
    w, _ = workloads.small_matrix()
    x = _x(200 + B, B, w.shape[1])
    X = to_dev_bf16(x)
    dm = uw.compress(w).to_device()
    base = uw.gemm_bf16(to_dev_bf16(w), X)
    outs = {}
    for name, p in uw.PIPELINES.items():
        scratch = uw.alloc_scratch(p, w.shape[0], w.shape[1], B)
        outs[name] = uw.matmul(dm, X, pipeline=p, scratch=scratch).cpu().numpy()
        assert_matmul_close(outs[name], w, x, what=f"pipeline {name} B={B}")
    # full decode feeds the same bf16 kernel as the baseline: identical bits
    assert np.array_equal(outs["full"].view(np.uint32), base.cpu().numpy().view(np.uint32))
    # the palette pipelines run the same kernel on identical nibbles
    assert np.array_equal(outs["pal"].view(np.uint32), outs["direct"].view(np.uint32))


def test_deterministic(torch_cuda):
    w, _ = workloads.small_matrix()
    dm = uw.compress(w).to_device()
    for B, k in [(1, uw.UW_KERNEL_GEMV), (64, uw.UW_KERNEL_MFMA), (32, uw.UW_KERNEL_SKINNY)]:
        X = to_dev_bf16(_x(B, B, 1024))
        a = uw.gemm_recon_pal(dm, None, X, kernel=k).cpu().numpy()
        b = uw.gemm_recon_pal(dm, None, X, kernel=k).cpu().numpy()
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_auto_plan_dispatch(torch_cuda):
    w, _ = workloads.small_matrix()
    x = _x(5, 4, 1024)
    dm = uw.compress(w).to_device()
    X = to_dev_bf16(x)
    uw.plan_clear()
    uw.plan_set(512, 1024, 4, uw.UW_PIPE_EXP, uw.UW_KERNEL_MFMA, 2)
    scratch = uw.alloc_scratch(uw.UW_PIPE_EXP, 512, 1024, 4, 2)
    Y = uw.matmul(dm, X, pipeline=uw.UW_PIPE_AUTO, scratch=scratch)
    assert_matmul_close(Y.cpu().numpy(), w, x, what="auto")
    uw.plan_clear()
    Y2 = uw.matmul(dm, X)       # no plan entry: direct palette, no scratch
    assert_matmul_close(Y2.cpu().numpy(), w, x, what="auto default")


def test_scratch_too_small_is_rejected(torch_cuda):
    w, _ = workloads.small_matrix()
    dm = uw.compress(w).to_device()
    X = to_dev_bf16(_x(1, 1, 1024))
    small = uw.alloc_scratch(uw.UW_PIPE_PAL, 512, 1024, 1)[:100]
    with pytest.raises(uw.UnweightError):
        uw.matmul(dm, X, pipeline=uw.UW_PIPE_FULL, scratch=small)


# ---------------------------------------------------------------- SiLU chain
def test_silu_mul_within_one_ulp(torch_cuda):
    import torch
    rng = np.random.default_rng(3)
    g = (rng.standard_normal(10007) * 4).astype(np.float32)
    u = (rng.standard_normal(10007) * 4).astype(np.float32)
    g[:6] = [0.0, -0.0, 80.0, -80.0, 1e-30, -1e-30]
    h = uw.silu_mul_bf16(torch.from_numpy(g).cuda(), torch.from_numpy(u).cuda())
    got = from_dev_bits(h).astype(np.int64)
    ref = numerics.f64_to_bf16_bits(numerics.silu_mul(g, u)).astype(np.int64)
    # compare as ordered integers: at most one bf16 ulp apart
    def key(b):
        return np.where(b & 0x8000, -(b & 0x7FFF), b & 0x7FFF)
    assert np.abs(key(got) - key(ref)).max() <= 1


@pytest.mark.parametrize("B", [1, 4, 16])
def test_mlp_layer_chain(torch_cuda, B):
    """gate/up -> bf16(SiLU(g)*u) -> down on reduced-width layer shapes."""
    print_case(f"mlp chain B={B}")
    F, H = 1536, 512
    wg = workloads.layer_weight(3, 0, 0, shape=(F, H))
    wu = workloads.layer_weight(3, 0, 1, shape=(F, H))
    wd = workloads.layer_weight(3, 0, 2, shape=(H, F))
    x = workloads.layer_activation(3, 0, 0, B, cols=H)
    dms = [uw.compress(m).to_device() for m in (wg, wu, wd)]
    X = to_dev_bf16(x)
    g = uw.matmul(dms[0], X, pipeline=uw.UW_PIPE_DIRECT)
    u = uw.matmul(dms[1], X, pipeline=uw.UW_PIPE_DIRECT)
    h = uw.silu_mul_bf16(g, u)
    y = uw.matmul(dms[2], h, pipeline=uw.UW_PIPE_DIRECT)
    gn, un = g.cpu().numpy(), u.cpu().numpy()
    assert_matmul_close(gn, wg, x, what="gate")
    assert_matmul_close(un, wu, x, what="up")
    hb = from_dev_bits(h)
    href = numerics.f64_to_bf16_bits(numerics.silu_mul(gn, un))
    key = lambda b: np.where(b & 0x8000, -(b.astype(np.int64) & 0x7FFF), b.astype(np.int64) & 0x7FFF)
    assert np.abs(key(hb) - key(href)).max() <= 1
    assert_matmul_close(y.cpu().numpy(), wd, hb, what="down")


@pytest.mark.parametrize("pipeline", ["full", "exp", "pal", "direct"])
@pytest.mark.parametrize("B", [1, 5, 24])
def test_mlp_layer_one_and_two_streams(torch_cuda, pipeline, B):
    """uw_mlp_layer on one stream and with the decodes on a second stream
    gives, bit for bit, what the single-matrix calls give for the same block
    (decode + matmul per matrix with the library's kernel and split-K
    choice, SiLU product between); that chain is checked against the fp64
    oracle on the GPU's h (reduced-width layer shapes)."""
    import torch
    print_case(f"mlp layer {pipeline} B={B}")
    F, H = 1536, 512
    wg = workloads.layer_weight(3, 1, 0, shape=(F, H))
    wu = workloads.layer_weight(3, 1, 1, shape=(F, H))
    wd = workloads.layer_weight(3, 1, 2, shape=(H, F))
    x = workloads.layer_activation(3, 1, 0, B, cols=H)
    dms = [uw.compress(m).to_device() for m in (wg, wu, wd)]
    p = uw.PIPELINES[pipeline]
    X = to_dev_bf16(x)
    scr = lambda R, C: uw.alloc_scratch(p, R, C, B, 0)
    g = uw.matmul(dms[0], X, pipeline=p, kernel=uw.UW_KERNEL_AUTO, split_k=0, scratch=scr(F, H))
    u = uw.matmul(dms[1], X, pipeline=p, kernel=uw.UW_KERNEL_AUTO, split_k=0, scratch=scr(F, H))
    h = uw.silu_mul_bf16(g, u)
    y_ref = uw.matmul(dms[2], h, pipeline=p, kernel=uw.UW_KERNEL_AUTO, split_k=0, scratch=scr(H, F))
    y1 = uw.mlp_layer(*dms, X, pipeline=p)
    aux = torch.cuda.Stream()
    y2 = uw.mlp_layer(*dms, X, pipeline=p, aux_stream=aux.cuda_stream)
    y3 = uw.mlp_layer(*dms, X, pipeline=p, aux_stream=aux.cuda_stream)     # events reused
    torch.cuda.synchronize()
    yr = y_ref.cpu().numpy()
    for name, yy in (("one stream", y1), ("two streams", y2), ("two streams, again", y3)):
        assert np.array_equal(yy.cpu().numpy().view(np.uint32), yr.view(np.uint32)), name
    assert_matmul_close(yr, wd, from_dev_bits(h), what=f"{pipeline} down on the GPU's h")


@pytest.mark.parametrize("B", [1, 3, 8, 16, 24])
def test_mlp_layer_direct_fused_pair(torch_cuda, B):
    """uw_mlp_layer on the direct-palette form (4096-row gate/up: one fused
    launch at batch 1 (GEMV pair) and 3-16 (skinny MFMA pair), separate
    skinny launches at 24): bit for bit what the single-matrix calls with the
    library's kernel choice give."""
    print_case(f"mlp layer direct fused pair B={B}")
    F, H = 4096, 512
    wg = workloads.layer_weight(3, 2, 0, shape=(F, H))
    wu = workloads.layer_weight(3, 2, 1, shape=(F, H))
    wd = workloads.layer_weight(3, 2, 2, shape=(H, F))
    x = workloads.layer_activation(3, 2, 0, B, cols=H)
    dms = [uw.compress(m).to_device() for m in (wg, wu, wd)]
    X = to_dev_bf16(x)
    p = uw.UW_PIPE_DIRECT
    g = uw.matmul(dms[0], X, pipeline=p, kernel=uw.UW_KERNEL_AUTO, split_k=0)
    u = uw.matmul(dms[1], X, pipeline=p, kernel=uw.UW_KERNEL_AUTO, split_k=0)
    h = uw.silu_mul_bf16(g, u)
    y_ref = uw.matmul(dms[2], h, pipeline=p, kernel=uw.UW_KERNEL_AUTO, split_k=0,
                      scratch=uw.alloc_scratch(p, H, F, B, 0))
    y = uw.mlp_layer(*dms, X, pipeline=p)
    assert np.array_equal(y.cpu().numpy().view(np.uint32), y_ref.cpu().numpy().view(np.uint32))
    assert_matmul_close(y.cpu().numpy(), wd, from_dev_bits(h), what=f"down on the GPU's h B={B}")


def test_mlp_layer_rejects(torch_cuda):
    print_case("mlp layer argument checks")
    rng = np.random.default_rng(2)
    dg = uw.compress(workloads.gaussian_weights(rng, 128, 64, 0.02)).to_device()
    dd = uw.compress(workloads.gaussian_weights(rng, 64, 128, 0.02)).to_device()
    X = to_dev_bf16(_x(1, 2, 64))
    with pytest.raises(uw.UnweightError, match="down"):
        uw.mlp_layer(dg, dg, dg, X)                       # down must be [H, F]
    import torch
    big = torch.empty(1 << 20, dtype=torch.uint8, device="cuda")
    with pytest.raises(uw.UnweightError, match="pipeline"):
        uw.mlp_layer(dg, dg, dd, X, pipeline=uw.UW_PIPE_AUTO, scratch=big)
    small = torch.empty(256, dtype=torch.uint8, device="cuda")
    with pytest.raises(uw.UnweightError, match="scratch"):
        uw.mlp_layer(dg, dg, dd, X, scratch=small)


# ----------------------------------------------------- fused gate/up + SiLU
def _bf16_key(b):
    b = b.astype(np.int64)
    return np.where(b & 0x8000, -(b & 0x7FFF), b & 0x7FFF)


def _dma_pair(R, B):
    """Whether the library runs the gate/up pair on the LDS-DMA skinny kernel
    (batch 3-32, at least three 16-row blocks per compute unit; or forced)."""
    import torch
    forced = os.environ.get("UW_SKINNY_DMA")
    if forced in ("0", "1"):
        return forced == "1" and B >= 3
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    return B >= 3 and (R + 15) // 16 >= 3 * cus


def _gate_up_case(wg, wu, x, rows=None, what=""):
    """The fused launch against the unfused three calls with the same kernel
    (the GEMV at batch 1-2, the register-staged or the DMA skinny kernel at
    3-32, whichever the pair takes; bit for bit) and against the fp64 oracle
    (g, u within tolerance; h within one bf16 ulp of bf16(SiLU(g)*u) on the
    GPU's g, u)."""
    import torch
    dg, du = uw.compress(wg).to_device(), uw.compress(wu).to_device()
    X = to_dev_bf16(x)
    B, R = x.shape[0], wg.shape[0]
    g = torch.empty((B, R), dtype=torch.float32, device="cuda")
    u = torch.empty_like(g)
    h = uw.mlp_gate_up(dg, du, X, g=g, u=u)
    h_only = uw.mlp_gate_up(dg, du, X)                       # no g/u outputs
    kernel = uw.UW_KERNEL_GEMV if B <= 2 else uw.UW_KERNEL_SKINNY
    saved = os.environ.get("UW_SKINNY_DMA")
    if _dma_pair(R, B):
        os.environ["UW_SKINNY_DMA"] = "1"                    # single launches on the pair's kernel
    try:
        g2 = uw.gemm_recon_pal(dg, None, X, kernel=kernel)
        u2 = uw.gemm_recon_pal(du, None, X, kernel=kernel)
    finally:
        if saved is None:
            os.environ.pop("UW_SKINNY_DMA", None)
        else:
            os.environ["UW_SKINNY_DMA"] = saved
    h2 = uw.silu_mul_bf16(g2, u2)
    gn, un = g.cpu().numpy(), u.cpu().numpy()
    assert np.array_equal(gn.view(np.uint32), g2.cpu().numpy().view(np.uint32)), what + " g"
    assert np.array_equal(un.view(np.uint32), u2.cpu().numpy().view(np.uint32)), what + " u"
    hb = from_dev_bits(h)
    assert np.array_equal(hb, from_dev_bits(h2)), what + " h"
    assert np.array_equal(hb, from_dev_bits(h_only)), what + " h without g/u"
    if rows is None:
        assert_matmul_close(gn, wg, x, what=what + " gate")
        assert_matmul_close(un, wu, x, what=what + " up")
    else:
        assert_matmul_close(gn[:, rows], wg, x, rows=rows, what=what + " gate")
        assert_matmul_close(un[:, rows], wu, x, rows=rows, what=what + " up")
    href = numerics.f64_to_bf16_bits(numerics.silu_mul(gn, un))
    assert np.abs(_bf16_key(hb) - _bf16_key(href)).max() <= 1


@pytest.mark.parametrize("B", [1, 2, 3, 4, 5, 8, 9, 16])
@pytest.mark.parametrize("dma", [False, True])
def test_gate_up_fused_small(torch_cuda, monkeypatch, B, dma):
    """Reduced-width gate/up pair (4096 x 512) at every batch the fused
    launch takes: the GEMV pair at 1-2, the skinny MFMA pair (each quad count
    of activation rows) at 3-16."""
    if dma and B <= 2:
        pytest.skip("the GEMV pair")
    if dma:
        monkeypatch.setenv("UW_SKINNY_DMA", "1")           # the pair and the unfused calls alike
    print_case(f"fused gate/up small B={B} dma={dma}")
    wg = workloads.layer_weight(3, 1, 0, shape=(4096, 512))
    wu = workloads.layer_weight(3, 1, 1, shape=(4096, 512))
    _gate_up_case(wg, wu, workloads.layer_activation(3, 1, 0, B, cols=512), what=f"B={B}")


@pytest.mark.parametrize("R,C,B", [(1, 64, 1), (37, 1088, 2), (5, 8192, 2), (4100, 1152, 3), (4111, 2176, 16),
                                   (12300, 1152, 13), (12290, 4096 + 128, 5), (12289, 640, 3), (12301, 1152, 29),
                                   (12320, 2176, 17)])
def test_gate_up_fused_ragged(torch_cuda, R, C, B):
    """Rows not a multiple of a workgroup, columns not a multiple of a slab
    (GEMV pair) or of the four K-slices (skinny pair: 9 and 17 steps), one-row
    and one-group matrices, outliers forcing verbatim groups; matrices tall
    enough for the DMA skinny pair, whose 9 and 33 steps leave a step after
    the two-step ring and whose last row block is partial, at batch 3-32
    (one and two batch tiles)."""
    print_case(f"fused gate/up ragged R={R} C={C} B={B}")
    rng = np.random.default_rng(R * C + B)
    wg = workloads.gaussian_weights(rng, R, C, 0.02, 0.004, 1.0)
    wu = workloads.gaussian_weights(rng, R, C, 0.03, 0.002, 2.0)
    _gate_up_case(wg, wu, _x(R + C, B, C), what=f"R={R} C={C} B={B}")


@pytest.mark.parametrize("B", [1, 4, 8, 12, 16, 24, 32])
def test_gate_up_fused_full_size(torch_cuda, B):
    """Llama-3.1-8B gate and up in the benchmark's launches (the GEMV pair at
    batch 1, the DMA skinny pair at 4 to 32: one, two, four and eight
    activation row quads, one and two batch tiles): bitwise equal to the
    unfused calls on the same kernel, sampled rows against the oracle."""
    print_case(f"fused gate/up full size B={B}")
    wg, wu = workloads.layer_weight(2, 0, 0), workloads.layer_weight(2, 0, 1)
    rows = np.sort(np.random.default_rng(5).choice(wg.shape[0], 384, replace=False))
    _gate_up_case(wg, wu, workloads.layer_activation(2, 0, 0, B), rows=rows, what=f"llama B={B}")


def test_gate_up_fused_rejects(torch_cuda):
    wg = workloads.layer_weight(3, 1, 0, shape=(64, 512))
    wu = workloads.layer_weight(3, 1, 1, shape=(64, 512))
    wo = workloads.layer_weight(3, 1, 1, shape=(64, 576))
    dg, du, do = (uw.compress(w).to_device() for w in (wg, wu, wo))
    with pytest.raises(uw.UnweightError) as ei:
        uw.mlp_gate_up(dg, du, to_dev_bf16(_x(1, 5, 512)))       # 64 rows split K 8 ways
    assert ei.value.code == uw.UW_EUNSUPPORTED
    big_g = uw.compress(workloads.layer_weight(3, 1, 0, shape=(4096, 512))).to_device()
    with pytest.raises(uw.UnweightError) as ei:
        uw.mlp_gate_up(big_g, big_g, to_dev_bf16(_x(1, 17, 512)))  # batch above 16, not tall enough for 17-32
    assert ei.value.code == uw.UW_EUNSUPPORTED
    tall = uw.compress(workloads.layer_weight(3, 1, 0, shape=(12288, 256))).to_device()
    uw.mlp_gate_up(tall, tall, to_dev_bf16(_x(1, 32, 256)))
    uw.mlp_gate_up(tall, tall, to_dev_bf16(_x(1, 33, 256)))       # the LDS-tile pair from batch 33
    with pytest.raises(uw.UnweightError) as ei:
        uw.mlp_gate_up(dg, do, to_dev_bf16(_x(1, 1, 512)))
    assert ei.value.code == uw.UW_EINVAL
    dn = uw.compress(wg).to_device(uw.DECODE_SECTIONS)      # no NIB section
    with pytest.raises(uw.UnweightError) as ei:
        uw.mlp_gate_up(dn, du, to_dev_bf16(_x(1, 1, 512)))
    assert ei.value.code == uw.UW_EINVAL
    # every exponent pattern: most groups verbatim, uploaded without VEXP
    spread = workloads.random_bf16_bits(9, 64 * 512).reshape(64, 512)
    blob = uw.compress(spread)
    assert blob.info().verbatim_groups > 0
    dv = blob.to_device(("sm", "nib", "bitmap", "tile_vbase"))
    with pytest.raises(uw.UnweightError) as ei:
        uw.mlp_gate_up(dv, dv, to_dev_bf16(_x(1, 1, 512)))
    assert ei.value.code == uw.UW_EINVAL and "verbatim" in str(ei.value)


# --------------------------------------------------------------- full sizes
@pytest.mark.parametrize("m", [0, 2])
def test_full_size_gemv_batch1_all_pipelines(torch_cuda, m):
    """Llama-3.1-8B gate and down at batch 1, in the launch configuration the
    benchmark times: every output against the fp64 oracle."""
    print_case(f"full-size batch-1 pipelines matrix {m}")
    w = workloads.layer_weight(2, 0, m)
    x = workloads.layer_activation(2, 0, m, 1)
    dm = uw.compress(w).to_device()
    X = to_dev_bf16(x)
    Yb = uw.gemm_bf16(to_dev_bf16(w), X).cpu().numpy()
    assert_matmul_close(Yb, w, x, what="bf16")
    for name, p in uw.PIPELINES.items():
        scratch = uw.alloc_scratch(p, w.shape[0], w.shape[1], 1)
        Y = uw.matmul(dm, X, pipeline=p, scratch=scratch).cpu().numpy()
        rel = assert_matmul_close(Y, w, x, what=f"{name}")
        assert rel < TOL


@pytest.mark.parametrize("m", [0, 2])
@pytest.mark.parametrize("B", [8, 64])
def test_full_size_skinny_all_pipelines(torch_cuda, m, B):
    """Llama-3.1-8B gate and down at batch 8 and 64 on the skinny MFMA kernel,
    every pipeline: sampled rows against the fp64 oracle."""
    print_case(f"full-size skinny matrix {m} B={B}")
    w = workloads.layer_weight(2, 1, m)
    x = workloads.layer_activation(2, 1, m, B)
    dm = uw.compress(w).to_device()
    X = to_dev_bf16(x)
    rows = np.sort(np.random.default_rng(B + m).choice(w.shape[0], 384, replace=False))
    for name, p in uw.PIPELINES.items():
        scratch = uw.alloc_scratch(p, w.shape[0], w.shape[1], B)
        Y = uw.matmul(dm, X, pipeline=p, kernel=uw.UW_KERNEL_SKINNY, scratch=scratch).cpu().numpy()
        assert_matmul_close(Y[:, rows], w, x, rows=rows, what=f"{name} B={B}")


@pytest.mark.parametrize("layer", [0, 17, 31])
def test_full_size_stack_layers(torch_cuda, layer):
    """Layers of the 32-layer stack (per-layer outlier rate): gate and down
    through the default (direct-palette) and palette-transcode pipelines at
    batch 1 and 16, sampled rows against the fp64 oracle."""
    for m in (0, 2):
        w = workloads.layer_weight(5, layer, m)
        dm = uw.compress(w).to_device()
        for B in (1, 16):
            print_case(f"stack layer {layer} matrix {m} B={B}")
            x = workloads.layer_activation(5, layer, m, B)
            X = to_dev_bf16(x)
            rows = np.sort(np.random.default_rng(layer * 7 + m + B).choice(w.shape[0], 256, replace=False))
            uw.plan_clear()
            for name, p in (("auto", uw.UW_PIPE_AUTO), ("pal", uw.UW_PIPE_PAL)):
                scratch = uw.alloc_scratch(p if p != uw.UW_PIPE_AUTO else uw.UW_PIPE_DIRECT, *w.shape, B)
                Y = uw.matmul(dm, X, pipeline=p, scratch=scratch).cpu().numpy()
                assert_matmul_close(Y[:, rows], w, x, rows=rows, what=f"{name} layer {layer} m {m} B={B}")


@pytest.mark.parametrize("B", [64, 128, 256])
def test_full_size_mfma_row_spread_workload(torch_cuda, B):
    """Per-row-scaled weights at large batch: sampled rows against the oracle."""
    print_case(f"full-size per-row sigma B={B}")
    w = workloads.layer_weight(4, 0, 0)
    x = workloads.layer_activation(4, 0, 0, B)
    dm = uw.compress(w).to_device()
    X = to_dev_bf16(x)
    rows = np.sort(np.random.default_rng(B).choice(w.shape[0], 512, replace=False))
    for name, Y in [("bf16", uw.gemm_bf16(to_dev_bf16(w), X)),
                    ("direct", uw.gemm_recon_pal(dm, None, X))]:
        assert_matmul_close(Y.cpu().numpy()[:, rows], w, x, rows=rows, what=f"{name} B={B}")
