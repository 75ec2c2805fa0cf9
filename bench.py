#!/usr/bin/env python3
"""Benchmark: compressed-MLP matmul on one MI355X.

One step = one forward of a Llama-3.1-8B-shaped MLP layer at batch B (default
1): gate and up projections of the same activation, h = bf16(SiLU(g) * u),
then the down projection -- all through one pipeline of the Unweight method
(default: direct palette, the fused reconstructive matmul over 4-bit indices
made at load time).  Weights are synthetic with Llama's shapes (seeded,
N(0,0.02) + 0.05% N(0,0.5) outliers); steps rotate over --layers independent
layer copies (default 4, ~1.1 GB compressed) so the 256 MiB Infinity Cache
cannot serve them.

Prints one JSON line: bf16-equivalent weight GB/s of the whole step, the
dominant kernel's roofline (HIP events on its stream over the timed region),
the uncompressed-bf16 baseline and the other pipelines on the same workload,
and the CPU oracle timed on a bounded sample on the host's cores.
"""
from __future__ import annotations

import argparse
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "compressed-MLP matmul: bf16-equiv weight GB/s, % HBM peak, batch 1\u2013256"
MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
HBM_PEAK_GBPS = 8000.0
PROFILES = os.path.join(ROOT, "profiles")


def parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    # about 10 ms each at batch 1: the first launches after an idle host-side
    # phase run at ramping clocks (measured 49 against 47 us per step)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=200)
    p.add_argument("--batch", type=int, default=1)
    p.add_argument("--pipeline", default="direct", choices=["direct", "pal", "exp", "full", "auto"])
    p.add_argument("--layers", type=int, default=4, help="layer copies rotated through (MALL defeat)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-compare", action="store_true", help="skip the other pipelines and the bf16 baseline")
    p.add_argument("--no-graph", action="store_true", help="time eager launches only")
    p.add_argument("--no-kernel-timer", action="store_true",
                   help="skip the per-launch timer pass and report no roofline (for a run under a tracing "
                        "profiler, where the timer's dispatch events slow the kernels they time)")
    p.add_argument("--no-sweep", action="store_true",
                   help="skip the autotuned batch sweep (1..256) over the gate and down shapes")
    p.add_argument("--sweep-batches", default="1,2,4,8,16,32,64,128,256")
    p.add_argument("--no-config34", action="store_true",
                   help="skip the batch-4/16 layer steps and the per-row-sigma batch-64..256 comparison")
    p.add_argument("--no-stack", action="store_true",
                   help="skip the 32-layer stack (generation ~1 min, ~22 GB of device memory)")
    p.add_argument("--stack-layers", type=int, default=32)
    p.add_argument("--stack-batches", default="1,2,4,8,16,32,64,128,256")
    p.add_argument("--stack-workers", type=int, default=12)
    p.add_argument("--copy-calibration", action="store_true",
                   help="also launch a plain device copy of known size (for counter calibration)")
    return p.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# ------------------------------------------------------------------ workload
class Layer:
    """One MLP layer: compressed matrices on the device plus raw bf16 copies."""

    def __init__(self, layer, keep_bf16, workload=2, mats=(0, 1, 2)):
        import torch
        import mlp_matmul_amd as uw
        import workloads
        self.mats, self.bf16, self.info = [], [], []
        for m in range(3):
            if m not in mats:
                self.mats.append(None), self.bf16.append(None), self.info.append(None)
                continue
            w = workloads.layer_weight(workload, layer, m)
            blob = uw.compress(w, emit_palette=True)
            dm = blob.to_device(uw.DECODE_SECTIONS + ("nib",))
            self.mats.append(dm)
            self.info.append(dm.info)
            if keep_bf16:
                self.bf16.append(torch.from_numpy(w.view(np.int16)).view(torch.bfloat16).cuda())
            del w, blob


def gate_up_bytes(info_g, info_u, batch):
    """Algorithmic bytes of the fused gate/up launch: both matrices' 4-bit
    forms, the activations once, the bf16 SiLU product out."""
    return (palette_bytes(info_g, batch) + palette_bytes(info_u, batch) - 2 * batch * info_g.cols
            - 8 * batch * info_g.rows + 2 * batch * info_g.rows)


def palette_bytes(info, batch):
    """Algorithmic bytes one direct-palette matmul launch must move: the 4-bit
    form (sign/mantissa plane, nibbles, verbatim exponents, bitmap, verbatim
    bases) + activations in + fp32 outputs."""
    sb = info.section_bytes
    import mlp_matmul_amd as uw
    w = (sb[uw.UW_SEC_SM] + info.rows * info.cols // 2 + sb[uw.UW_SEC_VEXP] + sb[uw.UW_SEC_BITMAP]
         + sb[uw.UW_SEC_TILE_VBASE])
    return int(w + 2 * batch * info.cols + 4 * batch * info.rows)


class Step:
    """Preallocated buffers and pre-bound C-ABI calls of one layer forward, so
    that the host issues a step in a few microseconds and the GPU queue stays
    ahead of it (the timed region measures the GPU, not Python)."""

    def __init__(self, layers, batch, pipeline, stream=None, workload=2, bf16_choice=None, fuse=True):
        import ctypes as ct
        import functools
        import torch
        import mlp_matmul_amd as uw
        import workloads
        self.torch = torch
        self.layers, self.B = layers, batch
        pipe = {"direct": uw.UW_PIPE_DIRECT, "pal": uw.UW_PIPE_PAL, "exp": uw.UW_PIPE_EXP,
                "full": uw.UW_PIPE_FULL, "auto": uw.UW_PIPE_AUTO, "bf16": uw.UW_PIPE_BF16}[pipeline]
        F, H = workloads.LLAMA_FFN, workloads.LLAMA_HIDDEN
        self.X = [torch.from_numpy(workloads.layer_activation(workload, i, 0, batch).view(np.int16))
                  .view(torch.bfloat16).cuda() for i in range(len(layers))]
        self.g = torch.empty((batch, F), dtype=torch.float32, device="cuda")
        self.u = torch.empty_like(self.g)
        self.h = torch.empty((batch, F), dtype=torch.bfloat16, device="cuda")
        self.y = torch.empty((batch, H), dtype=torch.float32, device="cuda")
        sp = pipe if pipe not in (uw.UW_PIPE_AUTO, uw.UW_PIPE_BF16) else uw.UW_PIPE_FULL
        nscr = max(uw.scratch_bytes(sp, F, H, batch, 0), uw.scratch_bytes(sp, H, F, batch, 0),
                   uw.scratch_bytes(sp, F, H, batch, 4), uw.scratch_bytes(sp, H, F, batch, 4))
        self.scratch = torch.empty(nscr, dtype=torch.uint8, device="cuda")
        self.stream = stream if stream is not None else torch.cuda.current_stream()
        L = uw.lib()
        self.uw_lib = L
        st = ct.c_void_p(self.stream.cuda_stream)
        P = lambda t: ct.c_void_p(t.data_ptr())
        scr, nsc = P(self.scratch), ct.c_uint64(self.scratch.numel())
        self.calls = []          # per layer: [gate, up, silu, down] bound calls
        self.bytes = []          # per layer: algorithmic bytes of gate, up, down
        for li, lay in enumerate(layers):
            X = P(self.X[li])
            outs = [(X, P(self.g)), (X, P(self.u)), (P(self.h), P(self.y))]
            row = []
            for m in range(3):
                xin, yout = outs[m]
                if pipe == uw.UW_PIPE_BF16:
                    R, C = lay.bf16[m].shape
                    k, sk = (bf16_choice or {}).get((R, C), (0, 0))
                    row.append(functools.partial(L.uw_gemm_bf16, P(lay.bf16[m]), R, C, xin, batch, yout, k, sk,
                                                 scr, nsc, st))
                else:
                    # kernel and split-K: the plan's (AUTO) or the library's choice
                    row.append(functools.partial(L.uw_matmul, ct.byref(lay.mats[m].dmat), pipe, 0, 0, xin,
                                                 batch, yout, scr, nsc, st))
            silu = functools.partial(L.uw_silu_mul_bf16, P(self.g), P(self.u), batch * F, P(self.h), st)
            self.fused = fuse and batch <= 16 and self._plans_direct(uw, pipe, F, H, batch)
            if self.fused:
                # gate, up and the SiLU product in one launch (h only)
                gu = functools.partial(L.uw_mlp_gate_up, ct.byref(lay.mats[0].dmat), ct.byref(lay.mats[1].dmat),
                                       X, batch, P(self.h), None, None, st)
                self.calls.append([gu, row[2]])
                self.bytes.append([gate_up_bytes(lay.info[0], lay.info[1], batch),
                                   palette_bytes(lay.info[2], batch)])
            else:
                self.calls.append([row[0], row[1], silu, row[2]])
                self.bytes.append([palette_bytes(lay.info[m], batch) for m in range(3)])

    @staticmethod
    def _plans_direct(uw, pipe, F, H, batch):
        """Gate/up may be fused (uw_mlp_gate_up: the GEMV pair at batch 1-2,
        the skinny MFMA pair at 3-16) when they would run on the direct-palette
        form with those kernels: asked for directly, or what the plan table
        holds for the gate shape at this batch (no entry: direct palette with
        the library's kernel choice)."""
        if pipe == uw.UW_PIPE_DIRECT:
            return True
        if pipe != uw.UW_PIPE_AUTO:
            return False
        plan = uw.plan_lookup(F, H, batch)
        if plan is None:
            return True
        p, k, _ = plan
        want = uw.UW_KERNEL_GEMV if batch <= 2 else uw.UW_KERNEL_SKINNY
        return p in (uw.UW_PIPE_DIRECT, uw.UW_PIPE_AUTO) and k in (want, uw.UW_KERNEL_AUTO)

    def run(self, i):
        for f in self.calls[i % len(self.layers)]:
            if f():
                raise RuntimeError("launch failed: " + self.uw_lib.uw_last_error().decode())


def time_steps(step, steps, warmup):
    """Average seconds per step over `steps` eager steps on the step's stream,
    after `warmup` untimed ones."""
    import torch
    with torch.cuda.stream(step.stream):
        for i in range(warmup):
            step.run(i)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            step.run(warmup + i)
        torch.cuda.synchronize()
    return (time.perf_counter() - t0) / steps


class GraphStep:
    """One captured HIP graph per layer copy; a step replays one of them."""

    def __init__(self, step):
        import torch
        self.step = step
        self.graphs = []
        with torch.cuda.stream(step.stream):
            for li in range(len(step.layers)):      # warm the kernels outside capture
                step.run(li)
            torch.cuda.synchronize()
            for li in range(len(step.layers)):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=step.stream):
                    step.run(li)
                self.graphs.append(g)
        torch.cuda.synchronize()

    def check_against_eager(self):
        """Every graph replay reproduces the eager outputs bit for bit."""
        import torch
        st = self.step
        for li, g in enumerate(self.graphs):
            with torch.cuda.stream(st.stream):
                st.run(li)
            torch.cuda.synchronize()
            outs = (st.h, st.y) if st.fused else (st.g, st.u, st.h, st.y)   # what the step writes
            ref = tuple(t.clone() for t in outs)
            for _ in range(3):
                for t in outs:
                    if t.dtype == torch.bfloat16:
                        t.zero_()
                    else:
                        t.fill_(float("nan"))
                torch.cuda.synchronize()
                g.replay()
                torch.cuda.synchronize()
                for a_, b_ in zip(ref, outs):
                    if not torch.equal(a_.view(torch.int16) if a_.dtype == torch.bfloat16 else a_.view(torch.int32),
                                       b_.view(torch.int16) if b_.dtype == torch.bfloat16 else b_.view(torch.int32)):
                        return False
        return True

    def time(self, steps, warmup):
        import torch
        n = len(self.graphs)
        for i in range(warmup):
            self.graphs[i % n].replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            self.graphs[i % n].replay()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / steps


# --------------------------------------------------------------- batch sweep
def time_bf16(mats_bf16, X, reps=20, warmup=3, stream=None):
    """Best seconds per call of the hand-written uncompressed bf16 matmul (the
    same kernel families on bf16 weights: GEMV for batch <= 16, skinny MFMA
    for batch 2..64, tiled MFMA with split-K 1/2/4), rotating over the copies.
    Returns (seconds, kernel name, kernel id, split_k)."""
    import ctypes as ct
    import torch
    import mlp_matmul_amd as uw
    from mlp_matmul_amd import autotune
    L = uw.lib()
    stream = stream or torch.cuda.current_stream()
    R, C = mats_bf16[0].shape
    B = X.shape[0]
    Y = torch.empty((B, R), dtype=torch.float32, device="cuda")
    scratch = torch.empty(8 * 4 * B * R + 256, dtype=torch.uint8, device="cuda")
    opts = ([(uw.UW_KERNEL_GEMV, 1)] if B <= 16 else []) \
        + ([(uw.UW_KERNEL_SKINNY, 1)] if 2 <= B <= 64 and autotune.skinny_ok(C) else []) \
        + [(uw.UW_KERNEL_MFMA, s_) for s_ in ((1, 2, 4, 8) if R <= 8192 else (1, 2, 4))]
    best = None
    for k, sk in opts:
        calls = [lambda W=W: uw.check(L.uw_gemm_bf16(ct.c_void_p(W.data_ptr()), R, C, ct.c_void_p(X.data_ptr()), B,
                                                     ct.c_void_p(Y.data_ptr()), k, sk,
                                                     ct.c_void_p(scratch.data_ptr()), scratch.numel(),
                                                     ct.c_void_p(stream.cuda_stream)), "uw_gemm_bf16")
                 for W in mats_bf16]
        with torch.cuda.stream(stream):
            for i in range(warmup):
                calls[i % len(calls)]()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for i in range(reps):
                calls[i % len(calls)]()
            e1.record(stream)
        e1.synchronize()
        t = e0.elapsed_time(e1) / 1e3 / reps
        name = autotune.KERNEL_NAMES[k] + (f"(split {sk})" if sk > 1 else "")
        best = (t, name, k, sk) if best is None or t < best[0] else best
    return best


def time_torch_bf16(mats_bf16, X, reps=20, warmup=3):
    """Seconds per call of torch.matmul(X, W^T) on the same bf16 copies (the
    vendor GEMM library): context next to the hand-written baseline."""
    import torch
    with torch.no_grad():
        for i in range(warmup):
            torch.matmul(X, mats_bf16[i % len(mats_bf16)].t())
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(reps):
            torch.matmul(X, mats_bf16[i % len(mats_bf16)].t())
        e1.record()
    e1.synchronize()
    return e0.elapsed_time(e1) / 1e3 / reps


def batch_sweep(layers, batches):
    """Autotune (pipeline x kernel x split-K) per shape and batch, and compare
    the winner with the uncompressed bf16 matmul on the same copies."""
    import torch
    import mlp_matmul_amd as uw
    from mlp_matmul_amd import autotune
    import workloads
    F, H = workloads.LLAMA_FFN, workloads.LLAMA_HIDDEN
    copies = {(F, H): [L.mats[0] for L in layers], (H, F): [L.mats[2] for L in layers]}
    bf16 = {(F, H): [L.bf16[0] for L in layers], (H, F): [L.bf16[2] for L in layers]}
    xs = {}

    def x_of(b, c):
        m = 0 if c == H else 2
        if (b, c) not in xs:
            xs[(b, c)] = torch.from_numpy(workloads.layer_activation(2, 0, m, b, cols=c).view(np.int16)) \
                .view(torch.bfloat16).cuda()
        return xs[(b, c)]

    uw.plan_clear()
    report = autotune.tune(copies, batches, x_of)
    out = []
    for r, s_ in zip(report, autotune.summarize(report)):
        shape = (r["rows"], r["cols"])
        b = r["batch"]
        t_b16, k_b16, _, _ = time_bf16(bf16[shape], x_of(b, shape[1]))
        t_torch = time_torch_bf16(bf16[shape], x_of(b, shape[1]))
        best_us = min(s_["us"].values()) if s_["us"] else None
        info = copies[shape][0].info
        direct_bytes = palette_bytes(info, b)
        flops = 2 * b * info.rows * info.cols
        row = {"shape": list(shape), "batch": b, "best": r["best"], "us": s_["us"],
               "bf16_us": round(t_b16 * 1e6, 3), "bf16_kernel": k_b16,
               "speedup_vs_bf16": round(t_b16 * 1e6 / best_us, 4) if best_us else None,
               "torch_bf16_us": round(t_torch * 1e6, 3),
               "speedup_vs_torch_bf16": round(t_torch * 1e6 / best_us, 4) if best_us else None,
               "best_bf16_equiv_GBps": round(2 * info.rows * info.cols / (best_us * 1e-6) / 1e9, 1) if best_us else None}
        if "direct" in s_["us"]:
            row["direct_compressed_GBps"] = round(direct_bytes / (s_["us"]["direct"] * 1e-6) / 1e9, 1)
            row["direct_hbm_frac"] = round(row["direct_compressed_GBps"] / HBM_PEAK_GBPS, 4)
        if best_us and r["best"] and r["best"]["kernel"] != "gemv":
            # bf16 MFMA utilisation of the best candidate against the dense peak
            row["best_mfma_TFLOPs"] = round(flops / (best_us * 1e-6) / 1e12, 2)
            row["best_mfma_util"] = round(row["best_mfma_TFLOPs"] / MFMA_BF16_PEAK_TFLOPS, 5)
        out.append(row)
        log(f"sweep {shape} B={b}: best {r['best']} {s_['us']} bf16 {row['bf16_us']} ({k_b16}) "
            f"torch {row['torch_bf16_us']} us")
    return out


# ------------------------------------------------------------ config 3 / 4
def layer_steps(layers, batches, stream, steps=30, warmup=5):
    """The MLP-layer step (gate/up -> SiLU product -> down) at small batches:
    direct palette (kernel by the library's default choice; gate/up fused
    where it applies) against the hand-written bf16 kernels."""
    rows = []
    for b in batches:
        sd = Step(layers, b, "direct", stream=stream)
        t_d = time_steps(sd, steps, warmup)
        sb = Step(layers, b, "bf16", stream=stream)
        t_b = time_steps(sb, steps, warmup)
        rows.append({"batch": b, "direct_ms": round(t_d * 1e3, 5), "bf16_ms": round(t_b * 1e3, 5),
                     "speedup_vs_bf16": round(t_b / t_d, 4), "gate_up_fused": sd.fused,
                     "bf16_equiv_GBps": round(3 * 2 * 14336 * 4096 / t_d / 1e9, 1)})
        if sd.fused:
            # the same step with gate and up as separate matmuls and the SiLU product
            su = Step(layers, b, "direct", stream=stream, fuse=False)
            rows[-1]["direct_unfused_ms"] = round(time_steps(su, steps, warmup) * 1e3, 5)
            del su
        log(f"layer step B={b}: direct {rows[-1]['direct_ms']} ms, bf16 {rows[-1]['bf16_ms']} ms, "
            f"unfused {rows[-1].get('direct_unfused_ms')}")
        del sd, sb
    return rows


def layer_overlap(layers, batches, stream, steps=20, warmup=3):
    """One MLP block per call (uw_mlp_layer) through the decoding pipelines,
    every step on one stream against the decodes on a second stream that
    overlap the matmuls; 4 rotated layers, microseconds per layer."""
    import ctypes as ct
    import functools
    import torch
    import mlp_matmul_amd as uw
    import workloads
    F, H = workloads.LLAMA_FFN, workloads.LLAMA_HIDDEN
    aux = torch.cuda.Stream()
    L = uw.lib()
    rows = []
    for b in batches:
        X = [torch.from_numpy(workloads.layer_activation(2, i, 0, b).view(np.int16)).view(torch.bfloat16).cuda()
             for i in range(len(layers))]
        y = torch.empty((b, H), dtype=torch.float32, device="cuda")
        row = {"batch": b}
        for name in ("full", "exp", "pal", "direct"):
            p = {"full": uw.UW_PIPE_FULL, "exp": uw.UW_PIPE_EXP, "pal": uw.UW_PIPE_PAL, "direct": uw.UW_PIPE_DIRECT}[name]
            scratch = torch.empty(uw.mlp_scratch_bytes(p, F, H, b), dtype=torch.uint8, device="cuda")
            res = {}
            for mode, a in (("one_stream", None), ("two_streams", ct.c_void_p(aux.cuda_stream))):
                if name == "direct" and a is not None:
                    continue                      # nothing to decode
                calls = [functools.partial(L.uw_mlp_layer, ct.byref(lay.mats[0].dmat), ct.byref(lay.mats[1].dmat),
                                           ct.byref(lay.mats[2].dmat), p, ct.c_void_p(X[i].data_ptr()), b,
                                           ct.c_void_p(y.data_ptr()), ct.c_void_p(scratch.data_ptr()),
                                           ct.c_uint64(scratch.numel()), ct.c_void_p(stream.cuda_stream), a)
                         for i, lay in enumerate(layers)]
                for i in range(warmup):
                    uw.check(calls[i % len(calls)](), "uw_mlp_layer")
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                for i in range(steps):
                    uw.check(calls[i % len(calls)](), "uw_mlp_layer")
                e1.record(stream)
                e1.synchronize()
                res[mode] = round(e0.elapsed_time(e1) / steps * 1e3, 2)
            if "two_streams" in res:
                res["speedup"] = round(res["one_stream"] / res["two_streams"], 3)
            row[name] = res
            del scratch
        rows.append(row)
        log(f"layer overlap B={b}: {row}")
    return rows


def attention_bench(batches, n_layers=6, steps=30, warmup=4):
    """The second workload on the codec: Llama-3.1-8B attention projections
    (q, o 4096x4096; k, v 1024x4096) of 6 seeded layers.  One step runs the
    four projections of one layer, steps rotate over the layers (495 MB of
    bf16, 378 MB compressed: more than the 256 MiB Infinity Cache, so a
    layer's weights come from HBM as in a decode pass).  Direct palette with
    the library's kernel and split choice against the hand-written bf16
    kernels (the fastest per shape) and torch.matmul."""
    import ctypes as ct
    import functools
    import torch
    import mlp_matmul_amd as uw
    import workloads
    L = uw.lib()
    names = list(workloads.ATTN_SHAPES)
    dev, bf, sizes = [], [], {}
    for i in range(n_layers):
        dl, bl = {}, {}
        for name in names:
            w = workloads.attention_weight(i, name)
            blob = uw.compress(w, emit_palette=True)
            dl[name] = blob.to_device(("sm", "nib", "vexp", "bitmap", "tile_vbase"))
            bl[name] = torch.from_numpy(w.view(np.int16)).view(torch.bfloat16).cuda()
            if i == 0:
                inf = blob.info()
                R, C = w.shape
                sizes[name] = {"shape": [R, C], "bf16_bytes": 2 * R * C,
                               "huffman_ratio": round(inf.huffman_form_bytes / (2 * R * C), 4),
                               "palette_ratio": round(inf.palette_form_bytes / (2 * R * C), 4)}
        dev.append(dl)
        bf.append(bl)
    bf16_bytes = sum(v["bf16_bytes"] for v in sizes.values())
    stream = torch.cuda.current_stream()
    st = ct.c_void_p(stream.cuda_stream)
    rows = []
    for b in batches:
        X = {n: torch.from_numpy(workloads.attention_activation(0, n, b).view(np.int16)).view(torch.bfloat16).cuda()
             for n in names}
        Y = {n: torch.empty((b, workloads.ATTN_SHAPES[n][0]), dtype=torch.float32, device="cuda") for n in names}
        scr = torch.empty(max(max(uw.scratch_bytes(uw.UW_PIPE_DIRECT, *workloads.ATTN_SHAPES[n], b, 0) for n in names),
                              8 * 4 * b * 4096 + 256), dtype=torch.uint8, device="cuda")
        P = lambda t: ct.c_void_p(t.data_ptr())
        # the bf16 kernel per shape: the fastest hand-written one
        choice = {}
        for n in names:
            _, kname, k, sk = time_bf16([bl[n] for bl in bf], X[n])
            choice[n] = (k, sk, kname)
        direct = [[functools.partial(L.uw_matmul, ct.byref(dl[n].dmat), uw.UW_PIPE_DIRECT, 0, 0, P(X[n]), b, P(Y[n]),
                                     P(scr), ct.c_uint64(scr.numel()), st) for n in names] for dl in dev]
        hand = [[functools.partial(L.uw_gemm_bf16, P(bl[n]), *workloads.ATTN_SHAPES[n], P(X[n]), b, P(Y[n]),
                                   choice[n][0], choice[n][1], P(scr), ct.c_uint64(scr.numel()), st) for n in names]
                for bl in bf]

        def run(calls):
            for i in range(warmup):
                for f in calls[i % n_layers]:
                    uw.check(f(), "attention")
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for i in range(steps):
                for f in calls[i % n_layers]:
                    uw.check(f(), "attention")
            e1.record(stream)
            e1.synchronize()
            return e0.elapsed_time(e1) / steps * 1e3

        t_d, t_b = run(direct), run(hand)
        with torch.no_grad():
            tc = [[functools.partial(torch.matmul, X[n], bl[n].t()) for n in names] for bl in bf]
            for i in range(warmup):
                for f in tc[i % n_layers]:
                    f()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for i in range(steps):
                for f in tc[i % n_layers]:
                    f()
            e1.record(stream)
            e1.synchronize()
            t_t = e0.elapsed_time(e1) / steps * 1e3
        rows.append({"batch": b, "direct_us": round(t_d, 2), "bf16_us": round(t_b, 2), "torch_bf16_us": round(t_t, 2),
                     "speedup_vs_bf16": round(t_b / t_d, 3), "speedup_vs_torch_bf16": round(t_t / t_d, 3),
                     "bf16_kernels": {n: choice[n][2] for n in names},
                     "bf16_equiv_GBps": round(bf16_bytes / t_d / 1e3, 1)})
        log(f"attention q/k/v/o step B={b}: {rows[-1]}")
    del dev, bf
    return {"sizes": sizes, "rows": rows}


def lm_head_bench(batches, copies=2, steps=20, warmup=3):
    """The embedding-sized matmul of the model: Llama-3.1-8B's output
    projection (128256 x 4096, 1.05 GB of bf16), one seeded matrix uploaded
    `copies` times at different addresses (rotating over them keeps the
    256 MiB Infinity Cache from serving it).  Direct palette with the
    library's kernel choice against the hand-written bf16 kernels (the
    fastest) and torch.matmul."""
    import ctypes as ct
    import functools
    import torch
    import mlp_matmul_amd as uw
    import workloads
    L = uw.lib()
    R, C = workloads.LM_HEAD_SHAPE
    t0 = time.perf_counter()
    w = workloads.lm_head_weight()
    blob = uw.compress(w, emit_palette=True)
    inf = blob.info()
    dev = [blob.to_device(("sm", "nib", "vexp", "bitmap", "tile_vbase")) for _ in range(copies)]
    wt = torch.from_numpy(w.view(np.int16)).view(torch.bfloat16)
    bf = [wt.cuda() for _ in range(copies)]
    del w, wt, blob
    log(f"lm head: generated, compressed and uploaded in {time.perf_counter() - t0:.1f} s")
    sizes = {"shape": [R, C], "bf16_bytes": 2 * R * C,
             "huffman_ratio": round(inf.huffman_form_bytes / (2 * R * C), 4),
             "palette_ratio": round(inf.palette_form_bytes / (2 * R * C), 4),
             "verbatim_group_frac": round(inf.verbatim_groups / inf.groups, 5)}
    stream = torch.cuda.current_stream()
    st = ct.c_void_p(stream.cuda_stream)
    P = lambda t: ct.c_void_p(t.data_ptr())
    rows = []
    for b in batches:
        X = torch.from_numpy(workloads.lm_head_activation(b).view(np.int16)).view(torch.bfloat16).cuda()
        Y = torch.empty((b, R), dtype=torch.float32, device="cuda")
        scr = torch.empty(max(uw.scratch_bytes(uw.UW_PIPE_DIRECT, R, C, b, 0), 16), dtype=torch.uint8, device="cuda")
        _, kname, k, sk = time_bf16(bf, X)
        direct = [functools.partial(L.uw_matmul, ct.byref(d.dmat), uw.UW_PIPE_DIRECT, 0, 0, P(X), b, P(Y), P(scr),
                                    ct.c_uint64(scr.numel()), st) for d in dev]
        bscr = torch.empty(8 * 4 * b * R + 256, dtype=torch.uint8, device="cuda")
        hand = [functools.partial(L.uw_gemm_bf16, P(W), R, C, P(X), b, P(Y), k, sk, P(bscr),
                                  ct.c_uint64(bscr.numel()), st) for W in bf]
        with torch.no_grad():
            tch = [functools.partial(torch.matmul, X, W.t()) for W in bf]

        def run(calls, checked=True):
            for i in range(warmup):
                r = calls[i % copies]()
                if checked:
                    uw.check(r, "lm head")
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for i in range(steps):
                r = calls[i % copies]()
                if checked:
                    uw.check(r, "lm head")
            e1.record(stream)
            e1.synchronize()
            return e0.elapsed_time(e1) / steps * 1e3

        t_d, t_b = run(direct), run(hand)
        with torch.no_grad():
            t_t = run(tch, checked=False)
        rows.append({"batch": b, "direct_us": round(t_d, 2), "bf16_us": round(t_b, 2), "bf16_kernel": kname,
                     "torch_bf16_us": round(t_t, 2), "speedup_vs_bf16": round(t_b / t_d, 3),
                     "speedup_vs_torch_bf16": round(t_t / t_d, 3),
                     "bf16_equiv_GBps": round(2 * R * C / t_d / 1e3, 1),
                     "compressed_GBps": round(inf.palette_form_bytes / t_d / 1e3, 1),
                     "compressed_hbm_frac": round(inf.palette_form_bytes / t_d / 1e3 / HBM_PEAK_GBPS, 4)})
        log(f"lm head B={b}: {rows[-1]}")
        del bscr, scr
    del dev, bf
    torch.cuda.empty_cache()
    return {"workload": "llama3.1-8b output projection 128256x4096, one seeded matrix, "
                        f"{copies} device copies rotated", "sizes": sizes, "rows": rows}


def time_pipeline(copies, pipeline, kernel, split_k, X, reps=20, warmup=3, stream=None):
    """Seconds per uw_matmul call (pipeline, kernel, split_k), rotating copies."""
    import torch
    import mlp_matmul_amd as uw
    from mlp_matmul_amd import autotune
    stream = stream or torch.cuda.current_stream()
    R, C, B = copies[0].rows, copies[0].cols, X.shape[0]
    Y = torch.empty((B, R), dtype=torch.float32, device="cuda")
    scratch = torch.empty(max(uw.scratch_bytes(pipeline, R, C, B, split_k), 16), dtype=torch.uint8, device="cuda")
    return autotune.time_candidate(copies, X, Y, scratch, (pipeline, kernel, split_k), stream, reps, warmup)


def config4(batches, n_copies=4):
    """Per-row-scaled weights (sigma_r log-uniform in [0.005, 0.05]) at batch
    64/128/256 on both Llama shapes: palette transcode (P3) vs direct palette
    (P4), each with its best kernel, vs the best hand-written bf16 kernel and
    torch.matmul; MFMA utilisation of each against the dense bf16 peak."""
    import torch
    import mlp_matmul_amd as uw
    from mlp_matmul_amd import autotune
    import workloads
    F, H = workloads.LLAMA_FFN, workloads.LLAMA_HIDDEN
    layers = [Layer(i, keep_bf16=True, workload=4, mats=(0, 2)) for i in range(n_copies)]
    out = []
    for m in (0, 2):
        R, C = workloads.MLP_SHAPES[m]
        copies = [L.mats[m] for L in layers]
        for b in batches:
            X = torch.from_numpy(workloads.layer_activation(4, 0, m, b).view(np.int16)).view(torch.bfloat16).cuda()
            row = {"shape": [R, C], "batch": b}
            flops = 2.0 * b * R * C
            for name, p in (("pal", uw.UW_PIPE_PAL), ("direct", uw.UW_PIPE_DIRECT)):
                best = None
                for (p_, k, sk) in autotune.candidates(R, C, b):
                    if p_ != p:
                        continue
                    t = time_pipeline(copies, p, k, sk, X)
                    if best is None or t < best[0]:
                        best = (t, autotune.KERNEL_NAMES[k] + (f"(split {sk})" if sk > 1 else ""))
                row[name] = {"us": round(best[0] * 1e6, 3), "kernel": best[1],
                             "mfma_util": round(flops / best[0] / 1e12 / MFMA_BF16_PEAK_TFLOPS, 5)}
            t_b, k_b, _, _ = time_bf16([L.bf16[m] for L in layers], X)
            t_t = time_torch_bf16([L.bf16[m] for L in layers], X)
            row["bf16"] = {"us": round(t_b * 1e6, 3), "kernel": k_b,
                           "mfma_util": round(flops / t_b / 1e12 / MFMA_BF16_PEAK_TFLOPS, 5)}
            row["torch_bf16"] = {"us": round(t_t * 1e6, 3),
                                 "mfma_util": round(flops / t_t / 1e12 / MFMA_BF16_PEAK_TFLOPS, 5)}
            out.append(row)
            log(f"config4 {R}x{C} B={b}: pal {row['pal']} direct {row['direct']} bf16 {row['bf16']} "
                f"torch {row['torch_bf16']}")
    del layers
    return out


# ------------------------------------------------------------ 32-layer stack
def _stack_blob(job):
    """Pool worker: generate and compress one matrix of the stack (host only,
    no GPU call).  Returns (layer, matrix, serialized blob)."""
    layer, m = job
    import mlp_matmul_amd as uw
    import workloads
    w = workloads.layer_weight(5, layer, m)
    return layer, m, uw.compress(w, emit_palette=True, threads=2).serialize()


def generate_stack_blobs(n_layers, workers):
    """Serialized blobs of every gate/up/down matrix of the stack, generated by
    a fork pool.  Must run before this process initialises the GPU (the
    children are forked copies of it)."""
    import multiprocessing as mp
    import torch
    assert not torch.cuda.is_initialized(), "generate the stack before touching the GPU"
    jobs = [(l, m) for l in range(n_layers) for m in range(3)]
    blobs = {}
    t0 = time.perf_counter()
    with mp.get_context("fork").Pool(workers) as pool:
        for i, (l, m, data) in enumerate(pool.imap_unordered(_stack_blob, jobs)):
            blobs[(l, m)] = data
            if (i + 1) % 12 == 0:
                log(f"stack: {i + 1}/{len(jobs)} matrices compressed ({time.perf_counter() - t0:.0f} s)")
    return blobs


class StackLayer:
    """One layer of the stack on the device: compressed gate/up/down, and bf16
    copies rebuilt by the full-decode kernel (bit-exact)."""

    def __init__(self, blobs, layer, keep_bf16):
        import mlp_matmul_amd as uw
        self.mats, self.bf16, self.info = [], [], []
        self.huffman_bytes = self.palette_bytes = self.bf16_bytes = self.device_bytes = 0
        for m in range(3):
            blob = uw.Blob.deserialize(blobs.pop((layer, m)))
            dm = blob.to_device(uw.DECODE_SECTIONS + ("nib",))
            inf = dm.info
            self.mats.append(dm)
            self.info.append(inf)
            self.huffman_bytes += inf.huffman_form_bytes
            self.palette_bytes += inf.palette_form_bytes
            self.bf16_bytes += 2 * inf.rows * inf.cols
            self.device_bytes += dm.device_bytes()
            if keep_bf16:
                self.bf16.append(uw.decode_full(dm))
            del blob


def time_stack(step, reps, warmup=1):
    """Seconds per pass of the whole stack (every layer once)."""
    import torch
    n = len(step.layers)
    with torch.cuda.stream(step.stream):
        for _ in range(warmup):
            for li in range(n):
                step.run(li)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(reps):
            for li in range(n):
                step.run(li)
        torch.cuda.synchronize()
    return (time.perf_counter() - t0) / reps


def time_torch_stack(layers, batch, reps, warmup=1):
    """The same stack through torch.matmul and torch's SiLU (vendor library
    context; bf16 outputs)."""
    import torch
    import workloads
    Xs = [torch.from_numpy(workloads.layer_activation(5, i, 0, batch).view(np.int16)).view(torch.bfloat16).cuda()
          for i in range(len(layers))]

    def one():
        for lay, X in zip(layers, Xs):
            g = torch.matmul(X, lay.bf16[0].t())
            u = torch.matmul(X, lay.bf16[1].t())
            h = torch.nn.functional.silu(g) * u
            torch.matmul(h, lay.bf16[2].t())
    with torch.no_grad():
        for _ in range(warmup):
            one()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(reps):
            one()
        torch.cuda.synchronize()
    return (time.perf_counter() - t0) / reps


def stack_bench(blobs, n_layers, batches, tune_copies=4, reps=5):
    """The 32-layer Llama-3.1-8B MLP stack with per-layer outlier rates:
    total sizes, the autotuner's plan per matrix shape and batch (tuned on
    the stack's own first layers), and whole-stack time per batch against the
    hand-written bf16 kernels and torch on the same (decoded) weights."""
    import torch
    import mlp_matmul_amd as uw
    from mlp_matmul_amd import autotune
    import workloads
    t0 = time.perf_counter()
    layers = [StackLayer(blobs, l, keep_bf16=True) for l in range(n_layers)]
    log(f"stack: {n_layers} layers on the device in {time.perf_counter() - t0:.1f} s")
    F, H = workloads.LLAMA_FFN, workloads.LLAMA_HIDDEN
    sizes = {k: int(sum(getattr(L, k) for L in layers))
             for k in ("bf16_bytes", "huffman_bytes", "palette_bytes", "device_bytes")}
    verb = sum(i.verbatim_groups for L in layers for i in L.info) / sum(i.groups for L in layers for i in L.info)
    nt = min(tune_copies, n_layers)
    copies = {(F, H): [L.mats[0] for L in layers[:nt]], (H, F): [L.mats[2] for L in layers[:nt]]}
    bf16_copies = {(F, H): [L.bf16[0] for L in layers[:nt]], (H, F): [L.bf16[2] for L in layers[:nt]]}
    stream = torch.cuda.Stream()
    rows = []
    for b in batches:
        def x_of(bb, c, _m={}):
            key = (bb, c)
            if key not in _m:
                _m[key] = torch.from_numpy(workloads.layer_activation(5, 0, 0 if c == H else 2, bb, cols=c)
                                           .view(np.int16)).view(torch.bfloat16).cuda()
            return _m[key]
        uw.plan_clear()
        report = autotune.tune(copies, [b], x_of)
        choice = {}
        for shape in copies:
            _, name, k, sk = time_bf16(bf16_copies[shape], x_of(b, shape[1]))
            choice[shape] = (k, sk)
        st = Step(layers, b, "auto", stream=stream, workload=5)
        t_c = time_stack(st, reps)
        fused = st.fused
        del st
        sb = Step(layers, b, "bf16", stream=stream, workload=5, bf16_choice=choice)
        t_b = time_stack(sb, reps)
        del sb
        t_t = time_torch_stack(layers, b, reps)
        row = {"batch": b, "ms": round(t_c * 1e3, 4), "bf16_ms": round(t_b * 1e3, 4), "torch_bf16_ms": round(t_t * 1e3, 4),
               "speedup_vs_bf16": round(t_b / t_c, 4), "speedup_vs_torch_bf16": round(t_t / t_c, 4),
               "bf16_equiv_GBps": round(sizes["bf16_bytes"] / t_c / 1e9, 1),
               "plan": [{"shape": [r["rows"], r["cols"]], **(r["best"] or {})} for r in report],
               "gate_up_fused": fused,
               "bf16_kernels": {f"{s_[0]}x{s_[1]}": autotune.KERNEL_NAMES[k] + (f"(split {sk})" if sk > 1 else "")
                                for s_, (k, sk) in choice.items()}}
        rows.append(row)
        log(f"stack B={b}: {row['ms']} ms (bf16 {row['bf16_ms']}, torch {row['torch_bf16_ms']}) plan {row['plan']}")
    uw.plan_clear()
    return {"workload": "llama3.1-8b-mlp-stack", "layers": n_layers,
            "weights": "N(0,0.02) + per-layer outlier rate U[0.01%, 0.2%] of N(0,0.5), seeded",
            "inputs": "one seeded N(0,1) bf16 activation per layer (unit-variance, as after a norm)",
            **sizes, "verbatim_group_frac": round(verb, 5),
            "huffman_saved_bytes": sizes["bf16_bytes"] - sizes["huffman_bytes"],
            "huffman_ratio": round(sizes["huffman_bytes"] / sizes["bf16_bytes"], 5),
            "palette_ratio": round(sizes["palette_bytes"] / sizes["bf16_bytes"], 5),
            "sweep": rows}


# ------------------------------------------------------------- CPU baseline
def cpu_baseline(frac_rows=8, min_seconds=10.0):
    """The oracle's per-step work (rebuild bf16 from the direct-palette form,
    fp64 matmul, SiLU chain) on the first 1/8 of each matrix's rows, repeated
    until ~10 s of CPU work; scaled to bf16-equivalent GB/s."""
    from oracle import codec, numerics
    import workloads
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([d.get("num_threads", 1) for d in threadpool_info()] + [1])
    except Exception:
        blas_threads = 1
    mats = []
    for m in range(3):
        R, C = workloads.MLP_SHAPES[m]
        w = workloads.layer_weight(2, 0, m)[: R // frac_rows]
        x = workloads.layer_activation(2, 0, m, 1)
        mats.append((codec.encode(w), x))
    nbytes = sum(2 * c.R * c.C for c, _ in mats)
    reps, t0 = 0, time.perf_counter()
    while True:
        g = u = None
        for m, (c, x) in enumerate(mats):
            wr = codec.reconstruct_from_palette(c)
            y = numerics.matmul(wr, x)
            if m == 0:
                g = y
            elif m == 1:
                u = y
        numerics.f64_to_bf16_bits(numerics.silu_mul(g, u))
        reps += 1
        el = time.perf_counter() - t0
        if el >= min_seconds:
            break
    return {"value": round(nbytes * reps / el / 1e9, 4), "unit": "GB/s", "cores": int(blas_threads),
            "kind": "oracle",
            "sample": (f"first 1/{frac_rows} of the rows of gate, up (1792x4096) and down (512x14336), batch 1: "
                       f"oracle rebuild from the 4-bit form + fp64 matmul + SiLU chain, {reps} reps in "
                       f"{el:.1f} s; bf16-equivalent bytes of the sample / time")}


# --------------------------------------------------------------- profiles
def kernel_source(kernel_tag):
    """The source file of the kernel a profile tag names (gemv_*, skinny_*, mfma_*)."""
    return {"gemv": "gemv.hip", "skinny": "mfma_gemv.hip", "mfma": "gemm_mfma.hip"}[kernel_tag.split("_")[0]]


def traffic_from_profiles(kernel_tag):
    """HBM bytes per launch from the committed rocprofv3 counter summary (two
    --pmc runs, FETCH_SIZE and WRITE_SIZE, scaled by a 1 GiB copy), if the
    summary was taken on the current kernel source (else None)."""
    import hashlib
    path = os.path.join(PROFILES, f"{kernel_tag}.md")
    if not os.path.exists(path):
        return None
    txt = open(path).read()
    m = re.search(r"kernel_source_sha256:\s*([0-9a-f]+)", txt)
    t = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", txt)
    if not m or not t:
        return None
    src = open(os.path.join(ROOT, "mlp_matmul_amd", "csrc", kernel_source(kernel_tag)), "rb").read()
    src += open(os.path.join(ROOT, "mlp_matmul_amd", "csrc", "device_common.h"), "rb").read()
    if hashlib.sha256(src).hexdigest()[:16] != m.group(1)[:16]:
        return None
    return float(t.group(1))


def main():
    a = parse()
    if a.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {a.gpus}); the compressed matmul path is "
              "per-GPU work, measured here on a single MI355X", file=sys.stderr)
        sys.exit(2)
    import torch
    import mlp_matmul_amd as uw
    import workloads
    blobs = None
    if not a.no_stack:
        # host-only generation first: the pool forks this process, which must
        # not have touched the GPU yet
        blobs = generate_stack_blobs(a.stack_layers, a.stack_workers)
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    uw.lib()
    B = a.batch
    t0 = time.perf_counter()
    layers = [Layer(i, keep_bf16=not a.no_compare) for i in range(a.layers)]
    log(f"built {a.layers} layer copies in {time.perf_counter() - t0:.1f} s")
    if a.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    F, H = workloads.LLAMA_FFN, workloads.LLAMA_HIDDEN
    weights_bf16_bytes = 3 * 2 * F * H
    stream = torch.cuda.Stream()

    def measure(pipeline, fuse=True):
        st = Step(layers, B, pipeline, stream=stream, fuse=fuse)
        eager = time_steps(st, a.steps, a.warmup)
        graph, ok = None, None
        if not a.no_graph:
            gs = GraphStep(st)
            ok = gs.check_against_eager()
            graph = gs.time(a.steps, a.warmup)
        return st, eager, graph, ok

    step, eager, graph, graph_ok = measure(a.pipeline)
    # the library's kernel timer records HIP events at the start and end of
    # every matmul launch (on its stream) over a second pass of the same eager
    # steps; launches come in step order (fused gate/up + down, or gate, up,
    # down), so each position of the step is one kernel
    # (its own warmup steps are recorded too and dropped: the graph check
    # before it leaves the GPU idle, and the first launches after that run
    # at ramping clocks)
    nl = len(step.bytes[0])
    if a.no_kernel_timer:
        durs = np.full((a.steps, nl), np.nan)
    else:
        with uw.KernelTimer(capacity=nl * (a.warmup + a.steps) + 8) as kt:
            time_steps(step, a.steps, a.warmup)
        durs = np.array(kt.ms, dtype=np.float64)[nl * a.warmup: nl * (a.warmup + a.steps)].reshape(a.steps, nl) / 1e3
    bytes_ = np.array([step.bytes[i % len(layers)] for i in range(a.steps)], dtype=np.float64)
    per_kernel = [{"bytes": float(bytes_[:, m].mean()), "avg_s": float(durs[:, m].mean()),
                   "total_s": float(durs[:, m].sum())} for m in range(nl)]
    dom = max(range(nl), key=lambda m: per_kernel[m]["total_s"])
    achieved = per_kernel[dom]["bytes"] / per_kernel[dom]["avg_s"] / 1e9
    achieved_all = bytes_.sum() / durs.sum() / 1e9
    # the kernel family UW_KERNEL_AUTO takes for the rebuilding sources
    family = "gemv" if B == 1 else ("skinny" if B <= 32 else "mfma")
    pair = "GEMV" if B <= 2 else "skinny MFMA"
    kernel_names = ([f"fused gate/up {pair} + SiLU (palette source)", f"down {family} (palette source)"]
                    if step.fused else [f"{n} recon matmul ({family})" for n in ("gate", "up", "down")])
    # the step time is the faster of the two valid timings
    use_graph = graph is not None and graph_ok and graph < eager
    sec = graph if use_graph else eager
    compressed_step_bytes = sum(step.bytes[0])
    log(f"{a.pipeline}: eager {eager * 1e3:.4f} ms/step, graph {graph and graph * 1e3}, graph==eager {graph_ok}, "
        f"kernels " + ", ".join(f"{kernel_names[m]} {per_kernel[m]['avg_s'] * 1e6:.2f} us" for m in range(nl)))
    unfused = None
    if step.fused and not a.no_compare:
        _, ue, ug, uok = measure(a.pipeline, fuse=False)
        unfused = {"eager_ms": round(ue * 1e3, 5), "graph_ms": ug and round(ug * 1e3, 5), "graph_matches_eager": uok}
        log(f"unfused step: {unfused}")

    extra = {}
    if not a.no_compare:
        for name in ("bf16", "full", "exp", "pal", "direct"):
            if name == a.pipeline:
                extra[name] = {"eager_ms": round(eager * 1e3, 5), "graph_ms": graph and round(graph * 1e3, 5)}
                continue
            _, e_, g_, ok_ = measure(name)
            extra[name] = {"eager_ms": round(e_ * 1e3, 5), "graph_ms": g_ and round(g_ * 1e3, 5),
                           "graph_matches_eager": ok_}
        log(f"ms/step by pipeline: {extra}")

    tag = (f"{'gemv' if B <= 2 else 'skinny'}_gateup_pal_llama_mlp_b{B}" if step.fused
           else f"{family}_recon_pal_llama_mlp_b{B}")
    traffic = traffic_from_profiles(tag) if a.pipeline == "direct" else None
    out = {
        "metric": METRIC,
        "value": round(weights_bf16_bytes / sec / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(sec * 1e3, 5),
        "timing": "hip-graph replay per step" if use_graph else "eager launches",
        "ms_per_step_eager": round(eager * 1e3, 5),
        "ms_per_step_graph": graph and round(graph * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "llama3.1-8b-mlp-layer", "batch": B, "pipeline": a.pipeline,
                   "gate_up": [F, H], "down": [H, F], "layer_copies_rotated": a.layers,
                   "step": ("fused gate/up + SiLU launch, down launch" if step.fused else
                            "gate, up, SiLU product, down launches"),
                   "weights": "N(0,0.02)+0.05% N(0,0.5), seeded"},
        "compressed_GBps": round(compressed_step_bytes / sec / 1e9, 2),
        "compressed_hbm_frac": round(compressed_step_bytes / sec / 1e9 / HBM_PEAK_GBPS, 4),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic,
                     "kernel": kernel_names[dom],
                     "launches": int(a.steps), "avg_launch_us": round(per_kernel[dom]["avg_s"] * 1e6, 3),
                     "algorithmic_bytes_per_launch": round(per_kernel[dom]["bytes"]),
                     "all_matmul_launches": {"achieved": round(achieved_all, 2),
                                             "frac": round(achieved_all / HBM_PEAK_GBPS, 4),
                                             "per_kernel_avg_us": {kernel_names[m]: round(per_kernel[m]["avg_s"] * 1e6, 3)
                                                                   for m in range(nl)}}},
    }
    if a.no_kernel_timer:
        out["roofline"] = None
    if unfused:
        out["ms_per_step_unfused"] = unfused
    if extra:
        out["ms_per_step_by_pipeline"] = extra
        b16 = min(v for v in (extra["bf16"]["graph_ms"], extra["bf16"]["eager_ms"]) if v)
        out["speedup_vs_bf16"] = round(b16 / (sec * 1e3), 4)
    if not a.no_sweep:
        batches = [int(v) for v in a.sweep_batches.split(",") if v]
        out["batch_sweep"] = batch_sweep(layers, batches)
        out["plan"] = [{"shape": r["shape"], "batch": r["batch"], **(r["best"] or {})} for r in out["batch_sweep"]]
    if not a.no_config34 and not a.no_compare:
        out["layer_steps"] = {"workload": "llama3.1-8b-mlp-layer, direct palette vs bf16, batch 2, 4, 8 and 16",
                              "rows": layer_steps(layers, [2, 4, 8, 16], stream)}
        out["attention"] = {"workload": "llama3.1-8b attention projections q/k/v/o, one step per layer, 6 seeded "
                                        "layers rotated",
                            **attention_bench([1, 4, 16])}
        out["lm_head"] = lm_head_bench([1, 4, 16])
        out["layer_overlap"] = {"workload": "llama3.1-8b-mlp-layer through uw_mlp_layer, us per layer: decodes on the "
                                            "layer's stream vs on a second stream overlapping the matmuls",
                                "rows": layer_overlap(layers, [1, 16], stream)}
        out["per_row_sigma"] = {"workload": "llama3.1-8b gate/down shapes, per-row sigma log-U[0.005,0.05], "
                                            "4 copies rotated",
                                "rows": config4([64, 128, 256])}
    if blobs is not None:
        out["stack"] = stack_bench(blobs, a.stack_layers, [int(v) for v in a.stack_batches.split(",") if v])
    if not a.no_cpu_baseline:
        log("timing the CPU oracle sample")
        out["cpu_baseline"] = cpu_baseline()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
