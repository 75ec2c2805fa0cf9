"""Autotuner: candidate space (CPU) and a small end-to-end tuning run (GPU)
whose every timed candidate is valid and whose choice lands in the plan
table that uw_matmul(UW_PIPE_AUTO) consults.  The choice itself depends on
timing and is not pinned; each candidate it may pick is covered by the
parity tests."""
import numpy as np
import pytest

import mlp_matmul_amd as uw
from mlp_matmul_amd import autotune
import workloads


def test_candidate_space():
    c = autotune.candidates(14336, 4096, 1)
    pipes = {p for p, _, _ in c}
    assert pipes == {uw.UW_PIPE_FULL, uw.UW_PIPE_EXP, uw.UW_PIPE_PAL, uw.UW_PIPE_DIRECT, uw.UW_PIPE_HUFF}
    assert any(k == uw.UW_KERNEL_GEMV for _, k, _ in c)
    # the Huffman decode inside the matmul: batch 1 and at least 4096 columns
    assert uw.UW_PIPE_HUFF not in {p for p, _, _ in autotune.candidates(14336, 4096, 2)}
    assert uw.UW_PIPE_HUFF not in {p for p, _, _ in autotune.candidates(512, 1024, 1)}
    # no GEMV beyond batch 16, split-K only offered to short matrices
    assert {k for _, k, _ in autotune.candidates(14336, 4096, 64)} == {uw.UW_KERNEL_MFMA, uw.UW_KERNEL_SKINNY}
    # the skinny kernel needs whole 128-column steps and at most 32768 columns
    assert uw.UW_KERNEL_SKINNY not in {k for _, k, _ in autotune.candidates(64, 192, 8)}
    assert uw.UW_KERNEL_SKINNY not in {k for _, k, _ in autotune.candidates(64, 32768 + 128, 8)}
    assert uw.UW_KERNEL_SKINNY in {k for _, k, _ in autotune.candidates(64, 32768, 8)}
    assert {s for _, _, s in autotune.candidates(4096, 14336, 256)} == {1, 2, 4, 8}
    assert {s for _, _, s in autotune.candidates(14336, 4096, 256)} == {1, 2, 4}
    assert {s for _, _, s in autotune.candidates(14336, 4096, 8)} == {1}
    assert uw.UW_PIPE_DIRECT not in {p for p, _, _ in autotune.candidates(64, 64, 1, has_palette=False)}


@pytest.mark.gpu
def test_tuner_fills_plan_and_auto_dispatch_is_correct():
    import torch
    from tests.gpu_util import assert_matmul_close, to_dev_bf16
    shape = (1024, 4096)
    ws = [workloads.layer_weight(2, l, 0, shape=shape) for l in range(2)]
    copies = [uw.compress(w).to_device() for w in ws]
    xs = {}

    def x_of(b, c):
        if b not in xs:
            xs[b] = to_dev_bf16(workloads.gaussian_activations(np.random.default_rng(b), b, c))
        return xs[b]

    uw.plan_clear()
    report = autotune.tune({shape: copies}, [1, 20], x_of, reps=3, warmup=1)
    assert uw.plan_count() == 2
    for r in report:
        assert r["best"] is not None
        assert all(c["valid"] for c in r["candidates"])
        X = x_of(r["batch"], shape[1])
        need = max(uw.scratch_bytes(p, *shape, r["batch"], s)
                   for p, _, s in autotune.candidates(*shape, r["batch"]))
        scratch = torch.empty(need, dtype=torch.uint8, device="cuda")
        Y = uw.matmul(copies[0], X, pipeline=uw.UW_PIPE_AUTO, scratch=scratch)
        assert_matmul_close(Y.cpu().numpy(), ws[0], xs[r["batch"]].view(torch.int16).cpu().numpy().view(np.uint16),
                            what=f"auto B={r['batch']}")
    uw.plan_clear()
