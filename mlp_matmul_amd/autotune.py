"""Measuring autotuner for the four pipelines.

The Unweight page ("Why no single pipeline wins") observes that the best way
to consume compressed weights changes with batch size and with the matrix
shape (gate/up against down), so the runtime picks a pipeline per weight
matrix and batch from end-to-end measurements on the target hardware.  This
module does that on one GPU: for each (rows, cols, batch) it times every
candidate (pipeline x kernel family x split-K) through ``uw_matmul``, keeps
the fastest, and records it in the library's plan table (``uw_plan_set``) that
``uw_matmul(UW_PIPE_AUTO)`` consults.

Timing rotates over several distinct copies of the matrix (different layers)
so that the 256 MiB Infinity Cache cannot serve the weights.  Each candidate's
output is checked once, element by element, against the full-decode pipeline
(whose rebuilt weights are bit-exact) with a per-output bound from
sum_c |W[r,c] X[b,c]|, so that a broken candidate can never win.
"""
from __future__ import annotations

import ctypes as ct
import json


from . import (UW_KERNEL_AUTO, UW_KERNEL_GEMV, UW_KERNEL_MFMA, UW_KERNEL_SKINNY, UW_PIPE_DIRECT, UW_PIPE_EXP, UW_PIPE_FULL,
               UW_PIPE_HUFF, UW_PIPE_PAL, check, decode_full, lib, plan_set, scratch_bytes)

PIPE_NAMES = {UW_PIPE_FULL: "full", UW_PIPE_EXP: "exp", UW_PIPE_PAL: "pal", UW_PIPE_DIRECT: "direct",
              UW_PIPE_HUFF: "huff"}
KERNEL_NAMES = {UW_KERNEL_AUTO: "decoder", UW_KERNEL_GEMV: "gemv", UW_KERNEL_MFMA: "mfma", UW_KERNEL_SKINNY: "skinny"}
# a candidate's outputs must stay within this many times sum_c |W[r,c] X[b,c]|
# of the exact product (fp32 accumulation over up to 14336 terms stays well
# inside it)
TOL = 2e-3


def skinny_ok(cols):
    steps = cols // 128
    return cols > 0 and cols % 128 == 0 and (steps + 7) // 8 * 128 <= 4096


def candidates(rows, cols, batch, has_palette=True):
    """(pipeline, kernel, split_k) triples worth timing for one shape/batch."""
    pipes = [UW_PIPE_FULL, UW_PIPE_EXP, UW_PIPE_PAL] + ([UW_PIPE_DIRECT] if has_palette else [])
    out = []
    if batch == 1 and cols >= 4096:
        out.append((UW_PIPE_HUFF, UW_KERNEL_AUTO, 1))      # decode inside the matmul (one kernel family)
    for p in pipes:
        if batch <= 16:
            out.append((p, UW_KERNEL_GEMV, 1))
        if batch >= 2 and skinny_ok(cols):
            out.append((p, UW_KERNEL_SKINNY, 1))
        splits = [1]
        # the tiled kernel covers 256 rows x 64-128 batch columns per
        # workgroup: split the K loop so every CU gets work
        if cols >= 2048 and batch >= 16:
            splits += [2, 4] + ([8] if rows <= 8192 else [])
        for s in splits:
            out.append((p, UW_KERNEL_MFMA, s))
    return out


class _Bound:
    """A pre-bound uw_matmul call (arguments marshalled once)."""

    def __init__(self, dm, pipeline, kernel, split_k, X, Y, scratch, stream):
        L = lib()
        self.fn = L.uw_matmul
        self.args = (ct.byref(dm.dmat), pipeline, kernel, split_k, ct.c_void_p(X.data_ptr()), X.shape[0],
                     ct.c_void_p(Y.data_ptr()), ct.c_void_p(scratch.data_ptr()),
                     ct.c_uint64(scratch.numel()), ct.c_void_p(stream.cuda_stream))

    def __call__(self):
        check(self.fn(*self.args), "uw_matmul")


def time_candidate(copies, X, Y, scratch, cand, stream, reps=20, warmup=3):
    """Seconds per call, averaged over `reps` calls rotating over `copies`."""
    import torch
    p, k, s = cand
    calls = [_Bound(dm, p, k, s, X, Y, scratch, stream) for dm in copies]
    with torch.cuda.stream(stream):
        for i in range(warmup):
            calls[i % len(calls)]()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(reps):
            calls[i % len(calls)]()
        e1.record(stream)
    e1.synchronize()
    return e0.elapsed_time(e1) / 1e3 / reps


def tune_shape(copies, batch, X, reps=20, warmup=3, stream=None):
    """Time every candidate for one (rows, cols, batch); returns (best, table)."""
    import torch
    stream = stream or torch.cuda.current_stream()
    rows, cols = copies[0].rows, copies[0].cols
    has_pal = all("nib" in dm.buffers for dm in copies)
    cands = candidates(rows, cols, batch, has_pal)
    need = max(scratch_bytes(p, rows, cols, batch, s) for p, _, s in cands)
    scratch = torch.empty(max(need, 16), dtype=torch.uint8, device="cuda")
    Y = torch.empty((batch, rows), dtype=torch.float32, device="cuda")
    # reference: full decode feeds the bf16 kernel with bit-exact weights
    with torch.cuda.stream(stream):
        _Bound(copies[0], UW_PIPE_FULL, UW_KERNEL_MFMA if batch > 16 else UW_KERNEL_GEMV, 1, X, Y, scratch,
               stream)()
    stream.synchronize()
    ref = Y.clone()
    # per-output scale S[b, r] = sum_c |W[r, c] X[b, c]| from the decoded
    # weights; a candidate and the reference each sit within 2e-3 * S of the
    # exact product, so they may differ by at most twice that
    with torch.cuda.stream(stream):
        Wd = decode_full(copies[0], stream=stream.cuda_stream)
        S = torch.matmul(X.float().abs(), Wd.float().abs().t().contiguous())
    stream.synchronize()
    del Wd
    table = []
    for cand in cands:
        with torch.cuda.stream(stream):
            Y.fill_(float("nan"))
            _Bound(copies[0], *cand, X, Y, scratch, stream)()
        stream.synchronize()
        diff = (Y - ref).abs()
        ok = bool(torch.isfinite(Y).all() and (diff <= 2 * TOL * S).all())
        t = time_candidate(copies, X, Y, scratch, cand, stream, reps, warmup) if ok else None
        table.append({"pipeline": PIPE_NAMES[cand[0]], "kernel": KERNEL_NAMES[cand[1]], "split_k": cand[2],
                      "us": None if t is None else round(t * 1e6, 3), "valid": ok})
    valid = [(r["us"], c) for r, c in zip(table, cands) if r["valid"]]
    best = min(valid)[1] if valid else None
    return best, table


def tune(copies_by_shape, batches, x_of, reps=20, warmup=3, apply=True):
    """Tune every shape x batch.  `copies_by_shape`: {(rows, cols): [DeviceMatrix, ...]};
    `x_of(batch, cols)` returns a bf16 activation tensor.  Returns a report."""
    report = []
    for (rows, cols), copies in copies_by_shape.items():
        for b in batches:
            X = x_of(b, cols)
            best, table = tune_shape(copies, b, X, reps, warmup)
            if best is not None and apply:
                plan_set(rows, cols, b, *best)
            report.append({"rows": rows, "cols": cols, "batch": b,
                           "best": None if best is None else {"pipeline": PIPE_NAMES[best[0]],
                                                              "kernel": KERNEL_NAMES[best[1]],
                                                              "split_k": best[2]},
                           "candidates": table})
    return report


def summarize(report):
    """Compact per-(shape, batch) view: best choice and the best time of each pipeline."""
    out = []
    for r in report:
        per_pipe = {}
        for c in r["candidates"]:
            if c["valid"] and (c["pipeline"] not in per_pipe or c["us"] < per_pipe[c["pipeline"]]):
                per_pipe[c["pipeline"]] = c["us"]
        out.append({"shape": [r["rows"], r["cols"]], "batch": r["batch"], "best": r["best"], "us": per_pipe})
    return out


def dumps(report):
    return json.dumps(report, indent=1)
