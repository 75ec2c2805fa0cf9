"""GPU parity of the Huffman decode inside a batch-1 matmul (UW_PIPE_HUFF):
the Huffman form read once, weights rebuilt in registers from the decoded
palette indices, never written out; per-tile partial sums added per row in
tile order.  Against the fp64 oracle on every output, a one-hot pin that
reveals the rebuilt weights bit-exactly, run-to-run bit identity, and the
argument checks.  Inputs come from the seeded generators in workloads.py."""
import numpy as np
import pytest

import mlp_matmul_amd as uw
from oracle import numerics
import workloads
from tests.gpu_util import assert_matmul_close, print_case, to_dev_bf16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    uw.lib()
    return torch


def _huff(dm, x):
    X = to_dev_bf16(x)
    scr = uw.alloc_scratch(uw.UW_PIPE_HUFF, dm.rows, dm.cols, 1)
    return uw.matmul(dm, X, pipeline=uw.UW_PIPE_HUFF, scratch=scr).cpu().numpy()


@pytest.mark.parametrize("R,C", [(512, 4096), (300, 8192), (64, 14336), (7, 4160), (3, 4160), (1, 4096), (33, 12352)])
def test_huffman_gemv_shapes(torch_cuda, R, C):
    """Rows that span tile boundaries at every offset (4160 and 12352 are
    not multiples of 4096), a partial last tile (3 x 4160: 195 groups), one
    row, and the Llama down width (3.5 tiles per row)."""
    print_case(f"huffman gemv R={R} C={C}")
    rng = np.random.default_rng(R * 7 + C)
    w = workloads.gaussian_weights(rng, R, C, 0.02, 0.002, 0.5)
    x = workloads.gaussian_activations(rng, 1, C)
    dm = uw.compress(w).to_device()
    assert_matmul_close(_huff(dm, x), w, x, what=f"huff R={R} C={C}")


def test_huffman_gemv_mostly_verbatim(torch_cuda):
    """Exponents spread over 41 values: most groups are verbatim (raw
    exponents), the rest coded."""
    print_case("huffman gemv mostly verbatim")
    rng = np.random.default_rng(11)
    R, C = 96, 8192
    e = rng.integers(100, 141, size=(R, C)).astype(np.uint16)
    w = ((rng.integers(0, 2, size=(R, C)).astype(np.uint16) << 15) | (e << 7)
         | rng.integers(0, 128, size=(R, C)).astype(np.uint16)).astype(np.uint16)
    x = workloads.gaussian_activations(rng, 1, C)
    blob = uw.compress(w)
    assert blob.info().verbatim_groups > blob.info().groups // 2
    assert_matmul_close(_huff(blob.to_device(), x), w, x, what="huff verbatim")


def test_huffman_gemv_one_hot_reveals_weights(torch_cuda):
    """x = e_c gives y[r] = W[r, c] exactly: one nonzero product per row and
    exact zeros elsewhere (bf16 x bf16 is exact in fp32)."""
    rng = np.random.default_rng(5)
    R, C = 200, 8192
    w = workloads.gaussian_weights(rng, R, C, 0.02, 0.01, 1.0)
    dm = uw.compress(w).to_device()
    for c in (0, 63, 64, 4095, 4096, 5000, C - 1):
        print_case(f"huffman gemv one-hot column {c}")
        x = np.zeros((1, C), np.uint16)
        x[0, c] = 0x3F80                    # 1.0
        y = _huff(dm, x)[0]
        expect = numerics.bf16_to_f64(w[:, c]).astype(np.float32)
        assert np.array_equal(y.view(np.uint32), expect.view(np.uint32)), f"column {c}"


@pytest.mark.parametrize("wl,m", [(2, 0), (2, 2), (5, 2)])
def test_huffman_gemv_full_size(torch_cuda, wl, m):
    """Llama-3.1-8B gate and down (one-layer workload) and a stack layer's
    down: every output against the oracle; two runs bit-identical."""
    print_case(f"huffman gemv full size workload {wl} matrix {m}")
    w = workloads.layer_weight(wl, 3, m)
    x = workloads.layer_activation(wl, 3, m, 1)
    dm = uw.compress(w).to_device()
    y1, y2 = _huff(dm, x), _huff(dm, x)
    assert np.array_equal(y1.view(np.uint32), y2.view(np.uint32)), "not deterministic"
    assert_matmul_close(y1, w, x, what=f"huff full size {wl}/{m}")


def test_huffman_gemv_rejects(torch_cuda):
    import torch
    print_case("huffman gemv argument checks")
    rng = np.random.default_rng(2)
    w = workloads.gaussian_weights(rng, 64, 4096, 0.02)
    dm = uw.compress(w).to_device()
    scr = uw.alloc_scratch(uw.UW_PIPE_HUFF, 64, 4096, 1)
    with pytest.raises(uw.UnweightError) as ei:                     # batch 2
        uw.matmul(dm, to_dev_bf16(workloads.gaussian_activations(rng, 2, 4096)), pipeline=uw.UW_PIPE_HUFF,
                  scratch=scr)
    assert ei.value.code == uw.UW_EUNSUPPORTED
    narrow = uw.compress(workloads.gaussian_weights(rng, 64, 1024, 0.02)).to_device()
    with pytest.raises(uw.UnweightError) as ei:                     # cols below 4096
        uw.matmul(narrow, to_dev_bf16(workloads.gaussian_activations(rng, 1, 1024)), pipeline=uw.UW_PIPE_HUFF,
                  scratch=scr)
    assert ei.value.code == uw.UW_EUNSUPPORTED
    with pytest.raises(uw.UnweightError) as ei:                     # scratch too small
        uw.matmul(dm, to_dev_bf16(workloads.gaussian_activations(rng, 1, 4096)), pipeline=uw.UW_PIPE_HUFF,
                  scratch=torch.empty(16, dtype=torch.uint8, device="cuda"))
    assert ei.value.code == uw.UW_EINVAL
    assert uw.scratch_bytes(uw.UW_PIPE_HUFF, 64, 4096, 1) == 512    # 64 tiles x 8 bytes, rounded to 256
