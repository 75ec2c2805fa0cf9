"""The allocation-free palette matmul, uw_gemm_recon_pal_static, against
uw_gemm_recon_pal with caller scratch: bit-identical outputs for the same
kernel and split on two calls in a row (the second on a smaller input, so a
stale partial sum left in the shared array would show), both within the
tolerance of the fp64 oracle; explicit splits whose partial sums exceed the
static array are rejected before any launch."""
import numpy as np
import pytest

import mlp_matmul_amd as uw
import workloads
from tests.gpu_util import assert_matmul_close, print_case, to_dev_bf16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    uw.lib()
    return torch


def _case(R, C, B, seed):
    rng = np.random.default_rng(seed)
    w = workloads.gaussian_weights(rng, R, C, 0.02, 0.002, 0.5)
    x = workloads.gaussian_activations(rng, B, C)
    return w, x, uw.compress(w).to_device(uw.DIRECT_SECTIONS)


@pytest.mark.parametrize("kernel,split", [(uw.UW_KERNEL_MFMA, 4), (uw.UW_KERNEL_MFMA, 0), (uw.UW_KERNEL_AUTO, 0),
                                          (uw.UW_KERNEL_GEMV, 1)])
def test_static_scratch_matches_caller_scratch(torch_cuda, kernel, split):
    torch = torch_cuda
    for R, C, B, seed in ((4096, 2048, 128, 1), (1000, 1024, 40, 2)):     # second call smaller
        if kernel == uw.UW_KERNEL_GEMV:
            B = min(B, 16)
        print_case(f"static scratch R={R} C={C} B={B} kernel {kernel} split {split}")
        w, x, dm = _case(R, C, B, seed)
        X = to_dev_bf16(x)
        # caller scratch big enough for the split the static array allows
        scratch = torch.empty(uw.UW_STATIC_SCRATCH_BYTES, dtype=torch.uint8, device="cuda")
        y_ref = uw.gemm_recon_pal(dm, None, X, kernel=kernel, split_k=split, scratch=scratch)
        y_st = uw.gemm_recon_pal_static(dm, None, X, kernel=kernel, split_k=split)
        torch.cuda.synchronize()
        a, b = y_ref.cpu().numpy(), y_st.cpu().numpy()
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), "static scratch output differs"
        assert_matmul_close(b, w, x, what=f"static R={R} B={B}")


def test_static_scratch_full_size_gate(torch_cuda):
    """Llama gate at batch 256 on the tiled kernel with the library's split."""
    torch = torch_cuda
    print_case("static scratch full-size gate B=256")
    w = workloads.layer_weight(2, 0, 0)
    x = workloads.layer_activation(2, 0, 0, 256)
    dm = uw.compress(w).to_device(uw.DIRECT_SECTIONS)
    X = to_dev_bf16(x)
    scratch = torch.empty(uw.UW_STATIC_SCRATCH_BYTES, dtype=torch.uint8, device="cuda")
    for split in (0, 2):
        y_ref = uw.gemm_recon_pal(dm, None, X, kernel=uw.UW_KERNEL_MFMA, split_k=split, scratch=scratch)
        y_st = uw.gemm_recon_pal_static(dm, None, X, kernel=uw.UW_KERNEL_MFMA, split_k=split)
        torch.cuda.synchronize()
        assert np.array_equal(y_ref.cpu().numpy().view(np.uint32), y_st.cpu().numpy().view(np.uint32))
    rows = np.sort(np.random.default_rng(4).choice(w.shape[0], 256, replace=False))
    assert_matmul_close(y_st.cpu().numpy()[:, rows], w, x, rows=rows, what="static full-size gate")


def test_static_scratch_rejects_oversized_split(torch_cuda):
    print_case("static scratch: oversized split rejected")
    w, x, dm = _case(4096, 1024, 300, 3)
    X = to_dev_bf16(x)
    with pytest.raises(uw.UnweightError, match="static scratch") as ei:
        uw.gemm_recon_pal_static(dm, None, X, kernel=uw.UW_KERNEL_MFMA, split_k=16)   # 78.6 MB of partials
    assert ei.value.code == uw.UW_EINVAL
    y = uw.gemm_recon_pal_static(dm, None, X, kernel=uw.UW_KERNEL_MFMA, split_k=0)   # lowered to fit
    assert_matmul_close(y.cpu().numpy(), w, x, what="split 0 lowered")
