#!/usr/bin/env python3
"""Benchmark: the compressed-MLP matmul on one MI355X, over a 32-layer
Llama-3.1-8B MLP stack.

One step = one forward of the whole stack at batch B (default 1): for each of
32 layers, the gate and up projections of the layer's activation,
h = bf16(SiLU(g) * u), then the down projection.  Each matrix runs through the
pipeline the autotuner picked for its shape at this batch ("Why no single
pipeline wins" on the Unweight page): at batch 1-16 that is the direct-palette
form with gate and up fused into one launch.  Weights are synthetic with
Llama's shapes (gate/up 14336x4096, down 4096x14336), seeded N(0, 0.02) with a
per-layer outlier rate uniform in [0.01 %, 0.2 %] of N(0, 0.5): 11.27 GB of
bf16, 8.65 GB in the direct-palette form, far beyond the 256 MiB Infinity
Cache, so every step streams its weights from HBM.

stdout: ONE compact JSON line, printed last: the step's bf16-equivalent weight
GB/s, the dominant kernel's roofline (its launches timed with HIP events on
its own stream), the uncompressed bf16 stack on the same GPU, a compact batch
sweep 1..256 and the CPU oracle timed per stage on the host's cores.
stderr: progress.  --detail FILE: the full sweep with the autotuner's tables,
and with --extras the one-layer pipeline comparison, the per-row-sigma
matrices at batch 64-256, the tensor-parallel shard shapes, the attention
projections and the output projection.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "compressed-MLP matmul: bf16-equiv weight GB/s, % HBM peak, batch 1–256"
MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
HBM_PEAK_GBPS = 8000.0
PROFILES = os.path.join(ROOT, "profiles")
STACK_WORKLOAD = 5
TUNE_LAYERS = 4                  # layers the autotuner times on (rotated: ~360 MB compressed per shape)


def parse(argv=None):
    p = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=30, help="timed steps (one step = one 32-layer forward)")
    p.add_argument("--warmup", type=int, default=5, help="untimed steps before the timed ones")
    p.add_argument("--min-warmup-ms", type=float, default=200.0,
                   help="warm up for at least this long, whatever --warmup says (clocks ramp after host phases)")
    p.add_argument("--batch", type=int, default=1)
    p.add_argument("--pipeline", default="auto", choices=["auto", "direct", "pal", "exp", "full", "huff"],
                   help="auto: the autotuner's plan per shape at this batch; huff: Huffman decode inside the "
                        "matmul (batch 1)")
    p.add_argument("--layers", type=int, default=32)
    p.add_argument("--gen-threads", type=int, default=0, help="host threads generating the stack (0: up to 16)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-compare", action="store_true", help="skip the uncompressed bf16 stack")
    p.add_argument("--graph", action="store_true", help="also time the step as HIP-graph replays")
    p.add_argument("--no-kernel-timer", action="store_true",
                   help="skip the per-launch timer pass and report no roofline (for a run under a tracing "
                        "profiler, where the timer's dispatch events slow the kernels they time)")
    p.add_argument("--no-sweep", action="store_true", help="skip the stack's batch sweep")
    p.add_argument("--sweep-batches", default="1,2,4,8,16,32,64,128,256")
    p.add_argument("--extras", action="store_true",
                   help="also the one-layer pipelines, per-row-sigma matrices, shard shapes, attention and output "
                        "projection (into the detail file)")
    p.add_argument("--detail", default=os.path.join(ROOT, "bench_out", "bench_detail.json"),
                   help="JSON file for the sweep, per-launch rows and the other legs (the printed line stays compact)")
    p.add_argument("--copy-calibration", action="store_true",
                   help="also launch a plain device copy of known size (for counter calibration)")
    return p.parse_args(argv)


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# ------------------------------------------------------------ byte accounting
def palette_bytes(info, batch):
    """Algorithmic bytes one direct-palette matmul launch must move: the 4-bit
    form (sign/mantissa plane, nibbles, verbatim exponents, bitmap, verbatim
    bases) + activations in + fp32 outputs."""
    import mlp_matmul_amd as uw
    sb = info.section_bytes
    w = (sb[uw.UW_SEC_SM] + info.rows * info.cols // 2 + sb[uw.UW_SEC_VEXP] + sb[uw.UW_SEC_BITMAP]
         + sb[uw.UW_SEC_TILE_VBASE])
    return int(w + 2 * batch * info.cols + 4 * batch * info.rows)


def gate_up_bytes(info_g, info_u, batch):
    """Algorithmic bytes of the fused gate/up launch: both matrices' 4-bit
    forms, the activations once, the bf16 SiLU product out."""
    return (palette_bytes(info_g, batch) + palette_bytes(info_u, batch) - 2 * batch * info_g.cols
            - 8 * batch * info_g.rows + 2 * batch * info_g.rows)


def bf16_bytes(R, C, batch):
    return int(2 * R * C + 2 * batch * C + 4 * batch * R)


def huffman_bytes(info, batch):
    """Algorithmic bytes of the Huffman-decode matmul: the Huffman form's
    sections (sign/mantissa, stream, group lengths, tile tables, verbatim
    exponents, bitmap) + activations in + outputs."""
    import mlp_matmul_amd as uw
    sb = info.section_bytes
    w = sum(int(sb[k]) for k in (uw.UW_SEC_SM, uw.UW_SEC_STREAM, uw.UW_SEC_GLEN, uw.UW_SEC_TILE_OFF,
                                 uw.UW_SEC_TILE_VBASE, uw.UW_SEC_VEXP, uw.UW_SEC_BITMAP))
    return int(w + 2 * batch * info.cols + 4 * batch * info.rows)


# ------------------------------------------------------------------ the stack
class MlpLayer:
    """One MLP layer on the device: compressed gate/up/down (Huffman sections
    and the 4-bit form) and the uncompressed bf16 weights (the baseline)."""

    def __init__(self):
        self.mats, self.bf16, self.info = [None] * 3, [None] * 3, [None] * 3


def _gen_one(job):
    """Host thread: draw and compress one matrix.  numpy's fills and the
    library's compressor release the GIL, so threads overlap."""
    import mlp_matmul_amd as uw
    import workloads
    workload, layer, m, shape = job
    w = workloads.layer_weight(workload, layer, m, shape=shape)
    return layer, m, w, uw.compress(w, emit_palette=True, threads=2)


def build_layers(workload, n_layers, threads=0, keep_bf16=True, mats=(0, 1, 2), shapes=None, verify=True,
                 sections=None):
    """Generate, compress and upload `n_layers` MLP layers.  Every matrix's
    full Huffman decode on the device is compared bit for bit with the
    uploaded original (which serves as the bf16 baseline).  Returns
    (layers, stats)."""
    import torch
    import mlp_matmul_amd as uw
    sections = sections or (uw.DECODE_SECTIONS + ("nib",))
    threads = threads or min(16, len(os.sched_getaffinity(0)))
    layers = [MlpLayer() for _ in range(n_layers)]
    jobs = [(workload, l, m, None if shapes is None else shapes[m]) for l in range(n_layers) for m in mats]
    stats = {"bf16_bytes": 0, "huffman_bytes": 0, "palette_bytes": 0, "groups": 0, "verbatim_groups": 0,
             "decode_checked": 0, "decode_bitexact": 0}
    scratch = None
    t0 = time.perf_counter()
    done_n = 0
    with cf.ThreadPoolExecutor(max_workers=threads) as ex:
        pending, todo = set(), list(jobs)
        while todo or pending:
            # a bounded window of matrices in flight, so finished ones are
            # released once uploaded (each holds ~230 MB of host memory)
            while todo and len(pending) < 2 * threads:
                pending.add(ex.submit(_gen_one, todo.pop(0)))
            finished, pending = cf.wait(pending, return_when=cf.FIRST_COMPLETED)
            for fut in finished:
                l, m, w, blob = fut.result()
                dm = blob.to_device(sections)
                inf = dm.info
                lay = layers[l]
                lay.mats[m], lay.info[m] = dm, inf
                wdev = torch.from_numpy(w.view(np.int16)).view(torch.bfloat16).cuda()
                if verify:
                    if scratch is None or scratch.numel() < w.size:
                        scratch = torch.empty(w.size, dtype=torch.bfloat16, device="cuda")
                    dec = uw.decode_full(dm, out=scratch[:w.size].view(w.shape))
                    stats["decode_checked"] += 1
                    stats["decode_bitexact"] += int(torch.equal(dec.view(torch.int16), wdev.view(torch.int16)))
                if keep_bf16:
                    lay.bf16[m] = wdev
                stats["bf16_bytes"] += 2 * w.size
                stats["huffman_bytes"] += int(inf.huffman_form_bytes)
                stats["palette_bytes"] += int(inf.palette_form_bytes)
                stats["groups"] += int(inf.groups)
                stats["verbatim_groups"] += int(inf.verbatim_groups)
                del w, blob, wdev, fut
                done_n += 1
                if done_n % 24 == 0 or done_n == len(jobs):
                    log(f"workload {workload}: {done_n}/{len(jobs)} matrices generated, compressed and uploaded "
                        f"({time.perf_counter() - t0:.0f} s)")
            del finished
    del scratch
    torch.cuda.synchronize()
    return layers, stats


# --------------------------------------------------------------------- steps
class Step:
    """Preallocated buffers and pre-bound C-ABI calls of one forward through a
    list of MLP layers, so that the host issues a launch in a few
    microseconds and the GPU queue stays ahead (the timed region measures the
    GPU, not Python).  step.run(i) runs every layer once."""

    def __init__(self, layers, batch, pipeline, stream, workload, bf16_choice=None, fuse=True):
        import ctypes as ct
        import functools
        import torch
        import mlp_matmul_amd as uw
        self.layers, self.B = layers, batch
        pipe = {"direct": uw.UW_PIPE_DIRECT, "pal": uw.UW_PIPE_PAL, "exp": uw.UW_PIPE_EXP,
                "full": uw.UW_PIPE_FULL, "auto": uw.UW_PIPE_AUTO, "bf16": uw.UW_PIPE_BF16,
                "huff": uw.UW_PIPE_HUFF}[pipeline]
        lay0 = layers[0]
        F, H = (lay0.info[0].rows, lay0.info[0].cols) if lay0.info[0] is not None else lay0.bf16[0].shape
        self.X = [torch.from_numpy(_act(workload, i, batch, H)).view(torch.bfloat16).cuda()
                  for i in range(len(layers))]
        self.g = torch.empty((batch, F), dtype=torch.float32, device="cuda")
        self.u = torch.empty_like(self.g)
        self.h = torch.empty((batch, F), dtype=torch.bfloat16, device="cuda")
        self.y = torch.empty((batch, H), dtype=torch.float32, device="cuda")
        self.scratch = torch.empty(max(self._scratch_need(uw, pipe, F, H, batch), 16), dtype=torch.uint8,
                                   device="cuda")
        self.stream = stream
        L = uw.lib()
        self.uw_lib = L
        st = ct.c_void_p(stream.cuda_stream)
        P = lambda t: ct.c_void_p(t.data_ptr())
        scr, nsc = P(self.scratch), ct.c_uint64(self.scratch.numel())
        self.fused = fuse and self._plans_direct(uw, pipe, F, H, batch) and \
            self._pair_supported(uw, layers[0], self.X[0], batch)
        self.calls = []          # per layer: the bound calls in launch order
        self.kinds = []          # per layer: what each timed (matmul) launch is
        self.bytes = []          # per layer: algorithmic bytes of each timed launch
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
            if pipe == uw.UW_PIPE_BF16:
                self.calls.append([row[0], row[1], silu, row[2]])
                self.kinds.append(["gate", "up", "down"])
                self.bytes.append([bf16_bytes(*lay.bf16[m].shape, batch) for m in range(3)])
            elif self.fused:
                # gate, up and the SiLU product in one launch (h only)
                gu = functools.partial(L.uw_mlp_gate_up, ct.byref(lay.mats[0].dmat), ct.byref(lay.mats[1].dmat),
                                       X, batch, P(self.h), None, None, st)
                self.calls.append([gu, row[2]])
                self.kinds.append(["gate_up", "down"])
                self.bytes.append([gate_up_bytes(lay.info[0], lay.info[1], batch), palette_bytes(lay.info[2], batch)])
            else:
                self.calls.append([row[0], row[1], silu, row[2]])
                self.kinds.append(["gate", "up", "down"])
                nbytes = huffman_bytes if pipe == uw.UW_PIPE_HUFF else palette_bytes
                self.bytes.append([nbytes(lay.info[m], batch) for m in range(3)])

    @staticmethod
    def _scratch_need(uw, pipe, F, H, batch):
        """Scratch for every matmul of the step: the decoded plane and split-K
        partials of the plan's choice per shape (AUTO), or of the pipeline
        with the library's split choice; for bf16 weights the partials of the
        largest split the baseline tries."""
        if pipe == uw.UW_PIPE_BF16:
            return 8 * 4 * batch * max(F, H) + 256
        need = 0
        for R, C in ((F, H), (H, F)):
            if pipe == uw.UW_PIPE_AUTO:
                plan = uw.plan_lookup(R, C, batch)
                p, s = (plan[0], plan[2]) if plan else (uw.UW_PIPE_DIRECT, 0)
            else:
                p, s = pipe, 0
            need = max(need, uw.scratch_bytes(p, R, C, batch, s))
        return need

    @staticmethod
    def _pair_supported(uw, lay, X, batch):
        """Whether uw_mlp_gate_up takes this shape at this batch (batch 17-32
        only on tall matrices; the LDS-tile pair above 32)."""
        if lay.mats[0] is None:
            return False
        try:
            uw.mlp_gate_up(lay.mats[0], lay.mats[1], X)
            return True
        except uw.UnweightError as e:
            if e.code != uw.UW_EUNSUPPORTED:
                raise
            return False

    @staticmethod
    def _plans_direct(uw, pipe, F, H, batch):
        """Gate/up may be fused (uw_mlp_gate_up: the GEMV pair at batch 1-2,
        a skinny MFMA pair at 3-32, the LDS-tile MFMA pair above 32) when they
        would run on the direct-palette form with those kernels: asked for
        directly, or what the plan table holds for the gate shape at this
        batch (no entry: direct palette with the library's kernel choice)."""
        if pipe == uw.UW_PIPE_DIRECT:
            return True
        if pipe != uw.UW_PIPE_AUTO:
            return False
        plan = uw.plan_lookup(F, H, batch)
        if plan is None:
            return True
        p, k, _ = plan
        want = uw.UW_KERNEL_GEMV if batch <= 2 else uw.UW_KERNEL_SKINNY if batch <= 32 else uw.UW_KERNEL_MFMA
        return p in (uw.UW_PIPE_DIRECT, uw.UW_PIPE_AUTO) and k in (want, uw.UW_KERNEL_AUTO)

    def run_layer(self, li):
        for f in self.calls[li]:
            if f():
                raise RuntimeError("launch failed: " + self.uw_lib.uw_last_error().decode())

    def run(self, i=0):
        for li in range(len(self.layers)):
            self.run_layer(li)

    @property
    def launch_bytes(self):
        return [b for row in self.bytes for b in row]

    @property
    def launch_kinds(self):
        return [k for row in self.kinds for k in row]


def _act(workload, layer, batch, cols):
    import workloads
    return workloads.layer_activation(workload, layer, 0, batch, cols=cols).view(np.int16)


def time_steps(step, steps, warmup, min_warmup_s=0.0):
    """Seconds per step over exactly `steps` timed steps on the step's stream,
    after at least `warmup` untimed ones and at least `min_warmup_s` of them.
    Returns (seconds per step, warmup steps run)."""
    import torch
    with torch.cuda.stream(step.stream):
        w, t0 = 0, time.perf_counter()
        while w < warmup or time.perf_counter() - t0 < min_warmup_s:
            step.run(w)
            w += 1
            if w >= warmup:
                torch.cuda.synchronize()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            step.run(i)
        torch.cuda.synchronize()
    return (time.perf_counter() - t0) / steps, w


def kernel_durations(step, steps, warmup):
    """Per-launch durations (s) of the step's matmul kernels over `steps`
    steps (after `warmup` recorded and dropped), from the library's timer:
    HIP events that each launch records at its own start and end on its
    stream.  Returns an array [steps, launches per step]."""
    import mlp_matmul_amd as uw
    nl = len(step.launch_kinds)
    with uw.KernelTimer(capacity=nl * (warmup + steps) + 8) as kt:
        time_steps(step, steps, warmup)
    ms = np.array(kt.ms, dtype=np.float64)
    if ms.size < nl * (warmup + steps):
        raise RuntimeError(f"kernel timer recorded {ms.size} launches, expected {nl * (warmup + steps)}")
    return ms[nl * warmup: nl * (warmup + steps)].reshape(steps, nl) / 1e3


class GraphStep:
    """The whole step captured as one HIP graph."""

    def __init__(self, step):
        import torch
        self.step = step
        with torch.cuda.stream(step.stream):
            step.run()
            torch.cuda.synchronize()
            self.graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(self.graph, stream=step.stream):
                step.run()
        torch.cuda.synchronize()

    def check_against_eager(self):
        """Three replays, each bit-identical to an eager run."""
        import torch
        st = self.step
        with torch.cuda.stream(st.stream):
            st.run()
        torch.cuda.synchronize()
        ref = st.y.clone()
        for _ in range(3):
            st.y.fill_(float("nan"))
            torch.cuda.synchronize()
            self.graph.replay()
            torch.cuda.synchronize()
            if not torch.equal(ref.view(torch.int32), st.y.view(torch.int32)):
                return False
        return True

    def time(self, steps, warmup):
        import torch
        for _ in range(warmup):
            self.graph.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            self.graph.replay()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / steps


# ----------------------------------------------------- baselines and tuning
def time_bf16(mats_bf16, X, reps=20, warmup=3, stream=None):
    """Best seconds per call of the hand-written uncompressed bf16 matmul (the
    same kernel families on bf16 weights: GEMV for batch <= 16, skinny MFMA
    for batch 2..64, tiled MFMA with split-K 1/2/4/8), rotating over the
    copies.  Returns (seconds, kernel name, kernel id, split_k)."""
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


def time_torch_stack(layers, batch, workload, reps, warmup=1):
    """The same stack through torch.matmul and torch's SiLU (vendor library
    context; bf16 outputs)."""
    import torch
    H = layers[0].bf16[0].shape[1]
    Xs = [torch.from_numpy(_act(workload, i, batch, H)).view(torch.bfloat16).cuda() for i in range(len(layers))]

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


def tune_stack(layers, batch, workload):
    """Autotune (pipeline x kernel x split-K) per shape at this batch on the
    stack's first layers; the plan serves every layer.  Returns the report."""
    import torch
    import mlp_matmul_amd as uw
    from mlp_matmul_amd import autotune
    nt = min(TUNE_LAYERS, len(layers))
    F, H = layers[0].info[0].rows, layers[0].info[0].cols
    copies = {(F, H): [L.mats[0] for L in layers[:nt]], (H, F): [L.mats[2] for L in layers[:nt]]}
    xs = {}

    def x_of(b, c):
        if (b, c) not in xs:
            xs[(b, c)] = torch.from_numpy(_act(workload, 0, b, c)).view(torch.bfloat16).cuda()
        return xs[(b, c)]
    return autotune.tune(copies, [batch], x_of)


def bf16_choice(layers, batch, workload):
    """The fastest hand-written bf16 kernel per shape at this batch."""
    import torch
    nt = min(TUNE_LAYERS, len(layers))
    out = {}
    for m in (0, 2):
        R, C = layers[0].bf16[m].shape
        X = torch.from_numpy(_act(workload, 0, batch, C)).view(torch.bfloat16).cuda()
        t, name, k, sk = time_bf16([L.bf16[m] for L in layers[:nt]], X)
        out[(R, C)] = (k, sk, name)
    return out


def plan_name(report):
    """'direct/gemv' style names of the plan per shape."""
    out = {}
    for r in report:
        b = r["best"]
        out[f"{r['rows']}x{r['cols']}"] = (None if b is None else
                                           f"{b['pipeline']}/{b['kernel']}" + (f"/split{b['split_k']}"
                                                                               if b["split_k"] > 1 else ""))
    return out


def stack_sweep(layers, batches, workload, stream, reps=5):
    """Whole-stack time per batch: the autotuned plan against the hand-written
    bf16 kernels and torch on the same weights."""
    import torch
    import mlp_matmul_amd as uw
    from mlp_matmul_amd import autotune
    bf16_total = sum(2 * t.numel() for L in layers for t in L.bf16)
    rows = []
    for b in batches:
        report = tune_stack(layers, b, workload)
        choice = bf16_choice(layers, b, workload)
        st = Step(layers, b, "auto", stream, workload)
        t_c, _ = time_steps(st, reps, 1)
        fused = st.fused
        del st
        sb = Step(layers, b, "bf16", stream, workload, bf16_choice={k: v[:2] for k, v in choice.items()})
        t_b, _ = time_steps(sb, reps, 1)
        del sb
        t_t = time_torch_stack(layers, b, workload, reps)
        flops = 2.0 * b * bf16_total / 2
        row = {"batch": b, "ms": round(t_c * 1e3, 4), "bf16_ms": round(t_b * 1e3, 4),
               "torch_bf16_ms": round(t_t * 1e3, 4), "speedup_vs_bf16": round(t_b / t_c, 4),
               "speedup_vs_torch_bf16": round(t_t / t_c, 4),
               "bf16_equiv_GBps": round(bf16_total / t_c / 1e9, 1),
               "mfma_TFLOPs": round(flops / t_c / 1e12, 1),
               "plan": plan_name(report), "gate_up_fused": fused,
               "bf16_kernels": {f"{R}x{C}": v[2] for (R, C), v in choice.items()},
               "autotune": autotune.summarize(report)}
        rows.append(row)
        log(f"stack B={b}: {row['ms']} ms (bf16 {row['bf16_ms']}, torch {row['torch_bf16_ms']}) "
            f"plan {row['plan']} fused={fused}")
        torch.cuda.empty_cache()
    uw.plan_clear()
    return rows


# ------------------------------------------------------------- CPU baseline
CPU_STAGES = ("encode", "full", "exp", "pal", "rebuild", "matmul")


def _timed(fn, min_s=0.3):
    """Seconds per call of fn(), repeated until min_s has passed."""
    n, t0 = 0, time.perf_counter()
    while True:
        fn()
        n += 1
        el = time.perf_counter() - t0
        if el >= min_s:
            return el / n


def cpu_baseline(batch, frac_rows=16, step_seconds=6.0):
    try:
        from threadpoolctl import threadpool_limits
    except ImportError:
        return _cpu_baseline(batch, frac_rows, step_seconds)
    with threadpool_limits(limits=len(os.sched_getaffinity(0)), user_api="blas"):
        return _cpu_baseline(batch, frac_rows, step_seconds)


def _cpu_baseline(batch, frac_rows, step_seconds):
    """The oracle on the host: per configuration, each stage of the method on
    a sample of one matrix (the whole 512x1024 matrix; 1/16 of the rows of
    the Llama-shaped ones) -- encode, the three decodes, the rebuild from the
    4-bit form, the fp64 matmul at the configuration's batch -- as
    bf16-equivalent GB/s; and the oracle's version of the benchmark step
    (rebuild from the 4-bit form, fp64 matmul, SiLU chain over gate, up and
    down) on 1/16 of the rows of the stack's first layer, repeated for
    ~step_seconds."""
    from oracle import codec, numerics
    import workloads
    cores = len(os.sched_getaffinity(0))
    t_all = time.perf_counter()
    weights = {"c1": workloads.small_matrix()[0],
               "c2": workloads.layer_weight(2, 0, 0)[: workloads.LLAMA_FFN // frac_rows],
               "c4": workloads.layer_weight(4, 0, 0)[: workloads.LLAMA_FFN // frac_rows],
               "c5": workloads.layer_weight(5, 0, 0)[: workloads.LLAMA_FFN // frac_rows]}
    weights["c3"] = weights["c2"]          # the direct-palette workload reuses the one-layer weights
    batches = {"c1": 1, "c2": 1, "c3": 16, "c4": 256, "c5": batch}
    stages, comp = {}, {}
    for key in ("c1", "c2", "c3", "c4", "c5"):
        w, B = weights[key], batches[key]
        nb = 2.0 * w.size
        x = workloads.gaussian_activations(np.random.default_rng([int(key[1]), 0, 0, 1]), B, w.shape[1])
        if key == "c3":
            row = [None] * 4                # codec stages as c2
        else:
            t = time.perf_counter()
            comp[key] = codec.encode(w)
            row = [time.perf_counter() - t]
            row += [_timed(lambda m=m: codec.decode_parallel(comp[key], m)) for m in ("full", "exp", "pal")]
        c = comp["c2" if key == "c3" else key]
        row.append(_timed(lambda: codec.reconstruct_from_palette(c)))
        row.append(_timed(lambda: numerics.matmul(w, x)))
        stages[key] = [None if t is None else float(f"{nb / t / 1e9:.3g}") for t in row]
    # the step: rebuild every matrix from its 4-bit form, fp64 matmuls, SiLU chain
    mats = []
    for m in range(3):
        R, C = workloads.MLP_SHAPES[m]
        w = workloads.layer_weight(5, 0, m)[: R // frac_rows]
        mats.append((codec.encode(w), workloads.layer_activation(5, 0, m, batch, cols=C)))
    nbytes = sum(2 * c.R * c.C for c, _ in mats)
    reps, t0 = 0, time.perf_counter()
    while True:
        g = u = None
        for m, (c, x) in enumerate(mats):
            y = numerics.matmul(codec.reconstruct_from_palette(c), x)
            g, u = (y, u) if m == 0 else ((g, y) if m == 1 else (g, u))
        numerics.f64_to_bf16_bits(numerics.silu_mul(g, u))
        reps += 1
        el = time.perf_counter() - t0
        if el >= step_seconds:
            break
    return {"value": round(nbytes * reps / el / 1e9, 4), "unit": "GB/s", "cores": cores, "kind": "oracle",
            "sample": (f"stack layer 0, 1/{frac_rows} of gate/up/down rows, B={batch}: 4-bit rebuild + fp64 "
                       f"matmul + SiLU, {reps} reps/{el:.1f} s; codec 1 thread, BLAS {cores}"),
            "stages_GBps": stages, "stage_order": ",".join(CPU_STAGES),
            "seconds": round(time.perf_counter() - t_all, 1)}


# --------------------------------------------------------------- profiles
def kernel_sources(kernel_tag):
    """The source files of the kernels a profile tag names (gemv_*, skinny_*,
    mfma_*, huffman_*); the skinny family has two kernels, one dispatching to
    the other."""
    return {"gemv": ["gemv.hip"], "skinny": ["mfma_gemv.hip", "skinny_dma.hip"], "mfma": ["gemm_mfma.hip", "gemm_lds.hip"],
            "huffman": ["decode.hip"]}[kernel_tag.split("_")[0]]


def profile_source_hash(kernel_tag):
    import hashlib
    csrc = os.path.join(ROOT, "mlp_matmul_amd", "csrc")
    src = b"".join(open(os.path.join(csrc, f), "rb").read() for f in kernel_sources(kernel_tag))
    src += open(os.path.join(csrc, "device_common.h"), "rb").read()
    return hashlib.sha256(src).hexdigest()[:16]


def profile_figures(kernel_tag):
    """(traffic bytes per launch, average launch us) from the committed
    rocprofv3 summary of this kernel and workload, if it was taken on the
    current kernel source; else (None, None)."""
    path = os.path.join(PROFILES, f"{kernel_tag}.md")
    if not os.path.exists(path):
        return None, None
    txt = open(path).read()
    m = re.search(r"kernel_source_sha256:\s*([0-9a-f]+)", txt)
    if not m or profile_source_hash(kernel_tag) != m.group(1)[:16]:
        return None, None
    t = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", txt)
    a = re.search(r"avg_launch_us:\s*([0-9.eE+]+)", txt)
    return (float(t.group(1)) if t else None), (float(a.group(1)) if a else None)


def traffic_from_profiles(kernel_tag):
    return profile_figures(kernel_tag)[0]


def headline_tag(step, batch):
    """Profile tag of the step's dominant kernel."""
    if step.fused:
        fam = "gemv" if batch <= 2 else ("skinny" if batch <= 32 else "mfma")
        return f"{fam}_gateup_pal_llama_mlp_stack_b{batch}"
    fam = "gemv" if batch == 1 else ("skinny" if batch <= 32 else "mfma")
    return f"{fam}_recon_llama_mlp_stack_b{batch}"


KIND_NAMES = {"gate_up": "fused gate/up + SiLU", "gate": "gate matmul", "up": "up matmul", "down": "down matmul"}


# ------------------------------------------------------------------- extras
def one_layer_pipelines(batches, stream, n_copies=4):
    """One Llama MLP layer (the single-layer workloads: 0.05 % outliers) at
    small batches through each pipeline -- full Huffman decode + bf16
    matmul, exponent-only decode + reconstructive matmul, palette transcode +
    reconstructive matmul, direct palette -- and the bf16 kernels; ms per
    layer, n_copies layers rotated."""
    import mlp_matmul_amd as uw
    layers, _ = build_layers(2, n_copies, verify=False)
    out = []
    for b in batches:
        row = {"batch": b}
        for name in ("full", "exp", "pal", "direct"):
            st = Step(layers, b, name, stream, 2)
            t, _ = time_steps(st, 20, 3)
            row[name] = round(t * 1e3 / n_copies, 4)
        choice = bf16_choice(layers, b, 2)
        st = Step(layers, b, "bf16", stream, 2, bf16_choice={k: v[:2] for k, v in choice.items()})
        row["bf16"] = round(time_steps(st, 20, 3)[0] * 1e3 / n_copies, 4)
        out.append(row)
        log(f"one layer B={b}: {row}")
    uw.plan_clear()
    return {"workload": "llama3.1-8b-mlp-layer, 0.05% outliers, ms per layer", "rows": out}


def matrix_comparison(workload, shapes_by_m, batches, n_copies=4, pipes=("pal", "direct")):
    """Per matrix shape and batch: the best kernel of each pipeline against
    the best hand-written bf16 kernel and torch.matmul, n_copies seeded
    copies rotated; MFMA utilisation against the dense bf16 peak."""
    import torch
    import mlp_matmul_amd as uw
    from mlp_matmul_amd import autotune
    mats = tuple(shapes_by_m)
    layers, _ = build_layers(workload, n_copies, mats=mats,
                             shapes={m: shapes_by_m[m] for m in mats} if shapes_by_m else None, verify=False)
    out = []
    for m in mats:
        R, C = shapes_by_m[m]
        copies = [L.mats[m] for L in layers]
        for b in batches:
            X = torch.from_numpy(workloads_act(workload, m, b, C)).view(torch.bfloat16).cuda()
            Y = torch.empty((b, R), dtype=torch.float32, device="cuda")
            flops = 2.0 * b * R * C
            row = {"shape": [R, C], "batch": b}
            for name in pipes:
                p = uw.PIPELINES[name]
                best = None
                for (p_, k, sk) in autotune.candidates(R, C, b):
                    if p_ != p:
                        continue
                    scr = torch.empty(max(uw.scratch_bytes(p, R, C, b, sk), 16), dtype=torch.uint8, device="cuda")
                    t = autotune.time_candidate(copies, X, Y, scr, (p, k, sk), torch.cuda.current_stream())
                    if best is None or t < best[0]:
                        best = (t, autotune.KERNEL_NAMES[k] + (f"(split {sk})" if sk > 1 else ""))
                row[name] = {"us": round(best[0] * 1e6, 2), "kernel": best[1],
                             "mfma_util": round(flops / best[0] / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)}
            t_b, k_b, _, _ = time_bf16([L.bf16[m] for L in layers], X)
            t_t = time_torch_bf16([L.bf16[m] for L in layers], X)
            row["bf16"] = {"us": round(t_b * 1e6, 2), "kernel": k_b,
                           "mfma_util": round(flops / t_b / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)}
            row["torch_bf16"] = {"us": round(t_t * 1e6, 2),
                                 "mfma_util": round(flops / t_t / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)}
            out.append(row)
            log(f"workload {workload} {R}x{C} B={b}: {row}")
    del layers
    torch.cuda.empty_cache()
    return out


def workloads_act(workload, m, batch, cols):
    import workloads
    return workloads.layer_activation(workload, 0, m, batch, cols=cols).view(np.int16)


def timed_rotation(calls, steps, warmup, stream, min_warm_s=0.1):
    """us per step of calls[i % len(calls)]() (each a list of launches, or one
    launch): warmed up for at least `warmup` steps and min_warm_s seconds
    (after a host phase the clocks ramp for longer than a few steps), then
    `steps` steps between two events on `stream`."""
    import torch
    import mlp_matmul_amd as uw
    n = len(calls)

    def one(i):
        c = calls[i % n]
        for f in (c if isinstance(c, list) else [c]):
            uw.check(f(), "timed launch")
    t0, i = time.perf_counter(), 0
    while i < warmup or time.perf_counter() - t0 < min_warm_s:
        one(i)
        i += 1
        if i % 16 == 0:
            torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(steps):
        one(i)
    e1.record(stream)
    e1.synchronize()
    return e0.elapsed_time(e1) / steps * 1e3


def interleaved_pair(a_calls, b_calls, steps, warmup, stream):
    """(us of a, us of b): each timed twice, interleaved, the faster run of each."""
    ta = timed_rotation(a_calls, steps, warmup, stream)
    tb = timed_rotation(b_calls, steps, warmup, stream)
    return (min(ta, timed_rotation(a_calls, steps, warmup, stream)),
            min(tb, timed_rotation(b_calls, steps, warmup, stream)))


def attention_bench(batches, n_layers=6, steps=30, warmup=4):
    """A second workload on the codec: Llama-3.1-8B attention projections
    (q, o 4096x4096; k, v 1024x4096) of 6 seeded layers.  One step runs the
    four projections of one layer, steps rotate over the layers (495 MB of
    bf16, more than the 256 MiB Infinity Cache).  Direct palette with the
    library's kernel and split choice against the hand-written bf16 kernels
    (the fastest per shape); us per step, each side warmed up for at least
    0.1 s and timed twice, interleaved, keeping the faster run."""
    import ctypes as ct
    import functools
    import torch
    import mlp_matmul_amd as uw
    import workloads
    L = uw.lib()
    names = list(workloads.ATTN_SHAPES)
    dev, bf = [], []
    for i in range(n_layers):
        dl, bl = {}, {}
        for name in names:
            w = workloads.attention_weight(i, name)
            dl[name] = uw.compress(w, emit_palette=True).to_device(uw.DIRECT_SECTIONS)
            bl[name] = torch.from_numpy(w.view(np.int16)).view(torch.bfloat16).cuda()
        dev.append(dl)
        bf.append(bl)
    stream = torch.cuda.current_stream()
    st = ct.c_void_p(stream.cuda_stream)
    P = lambda t: ct.c_void_p(t.data_ptr())
    rows = []
    for b in batches:
        X = {n: torch.from_numpy(workloads.attention_activation(0, n, b).view(np.int16)).view(torch.bfloat16).cuda()
             for n in names}
        Y = {n: torch.empty((b, workloads.ATTN_SHAPES[n][0]), dtype=torch.float32, device="cuda") for n in names}
        scr = torch.empty(8 * 4 * b * 4096 + 256, dtype=torch.uint8, device="cuda")
        choice = {n: time_bf16([bl[n] for bl in bf], X[n])[1:] for n in names}
        direct = [[functools.partial(L.uw_matmul, ct.byref(dl[n].dmat), uw.UW_PIPE_DIRECT, 0, 0, P(X[n]), b, P(Y[n]),
                                     P(scr), ct.c_uint64(scr.numel()), st) for n in names] for dl in dev]
        hand = [[functools.partial(L.uw_gemm_bf16, P(bl[n]), *workloads.ATTN_SHAPES[n], P(X[n]), b, P(Y[n]),
                                   choice[n][1], choice[n][2], P(scr), ct.c_uint64(scr.numel()), st) for n in names]
                for bl in bf]

        t_d, t_b = interleaved_pair(direct, hand, steps, warmup, stream)
        rows.append({"batch": b, "direct_us": round(t_d, 2), "bf16_us": round(t_b, 2),
                     "speedup_vs_bf16": round(t_b / t_d, 3), "bf16_kernels": {n: choice[n][0] for n in names}})
        log(f"attention q/k/v/o step B={b}: {rows[-1]}")
    del dev, bf
    torch.cuda.empty_cache()
    return {"workload": "llama3.1-8b attention projections, 6 seeded layers rotated", "rows": rows}


def lm_head_bench(batches, copies=2, steps=20, warmup=3):
    """The embedding-sized matmul of the model: the output projection
    (128256 x 4096, 1.05 GB of bf16), one seeded matrix uploaded `copies`
    times and rotated.  Direct palette with the library's kernel choice
    against the fastest hand-written bf16 kernel, each timed twice,
    interleaved, after a minimum warm-up (timed_rotation)."""
    import ctypes as ct
    import functools
    import torch
    import mlp_matmul_amd as uw
    import workloads
    L = uw.lib()
    R, C = workloads.LM_HEAD_SHAPE
    w = workloads.lm_head_weight()
    blob = uw.compress(w, emit_palette=True)
    inf = blob.info()
    dev = [blob.to_device(uw.DIRECT_SECTIONS) for _ in range(copies)]
    wt = torch.from_numpy(w.view(np.int16)).view(torch.bfloat16)
    bf = [wt.cuda() for _ in range(copies)]
    del w, wt, blob
    stream = torch.cuda.current_stream()
    st = ct.c_void_p(stream.cuda_stream)
    P = lambda t: ct.c_void_p(t.data_ptr())
    rows = []
    for b in batches:
        X = torch.from_numpy(workloads.lm_head_activation(b).view(np.int16)).view(torch.bfloat16).cuda()
        Y = torch.empty((b, R), dtype=torch.float32, device="cuda")
        scr = torch.empty(8 * 4 * b * R + 256, dtype=torch.uint8, device="cuda")
        _, kname, k, sk = time_bf16(bf, X)
        direct = [functools.partial(L.uw_matmul, ct.byref(d.dmat), uw.UW_PIPE_DIRECT, 0, 0, P(X), b, P(Y), P(scr),
                                    ct.c_uint64(scr.numel()), st) for d in dev]
        hand = [functools.partial(L.uw_gemm_bf16, P(W), R, C, P(X), b, P(Y), k, sk, P(scr),
                                  ct.c_uint64(scr.numel()), st) for W in bf]

        t_d, t_b = interleaved_pair(direct, hand, steps, warmup, stream)
        rows.append({"batch": b, "direct_us": round(t_d, 2), "bf16_us": round(t_b, 2), "bf16_kernel": kname,
                     "speedup_vs_bf16": round(t_b / t_d, 3),
                     "compressed_hbm_frac": round(inf.palette_form_bytes / t_d / 1e3 / HBM_PEAK_GBPS, 4)})
        log(f"output projection B={b}: {rows[-1]}")
    del dev, bf
    torch.cuda.empty_cache()
    return {"workload": "llama3.1-8b output projection 128256x4096", "rows": rows}


# ----------------------------------------------------------------------- main
def main():
    a = parse()
    if a.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {a.gpus}); the compressed matmul path is "
              "per-GPU work, measured here on a single MI355X", file=sys.stderr)
        sys.exit(2)
    import torch
    import mlp_matmul_amd as uw
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    uw.lib()
    B, W5 = a.batch, STACK_WORKLOAD
    t0 = time.perf_counter()
    layers, stats = build_layers(W5, a.layers, threads=a.gen_threads, keep_bf16=not a.no_compare)
    log(f"stack: {a.layers} layers ready in {time.perf_counter() - t0:.1f} s; full decode bit-exact on "
        f"{stats['decode_bitexact']}/{stats['decode_checked']} matrices")
    if a.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    F, H = layers[0].info[0].rows, layers[0].info[0].cols
    stream = torch.cuda.Stream()
    detail = {"stack": {"layers": a.layers, **stats}}

    # ---- the headline step: the plan at this batch (or a forced pipeline)
    plan = None
    if a.pipeline == "auto":
        report = tune_stack(layers, B, W5)
        plan = plan_name(report)
        detail["headline_autotune"] = report
        log(f"plan at batch {B}: {plan}")
    step = Step(layers, B, a.pipeline, stream, W5)
    sec, warm_run = time_steps(step, a.steps, a.warmup, a.min_warmup_ms / 1e3)
    log(f"stack step B={B}: {sec * 1e3:.4f} ms ({a.steps} timed, {warm_run} warmup steps), fused gate/up: "
        f"{step.fused}")
    graph = None
    if a.graph:
        gs = GraphStep(step)
        ok = gs.check_against_eager()
        graph = {"ms": round(gs.time(a.steps, a.warmup) * 1e3, 4), "matches_eager": ok}
        del gs
        log(f"graph replay: {graph}")

    roof = None
    if not a.no_kernel_timer:
        durs = kernel_durations(step, a.steps, max(a.warmup, 3))
        kinds = step.launch_kinds
        by = np.array(step.launch_bytes, dtype=np.float64)
        per_kind = {}
        for k in dict.fromkeys(kinds):
            idx = [i for i, kk in enumerate(kinds) if kk == k]
            tot_s, tot_b = durs[:, idx].sum(), by[idx].sum() * a.steps
            per_kind[k] = {"avg_us": float(durs[:, idx].mean() * 1e6), "bytes": float(by[idx].mean()),
                           "total_s": float(tot_s), "GBps": float(tot_b / tot_s / 1e9), "launches": len(idx) * a.steps}
        dom = max(per_kind, key=lambda k: per_kind[k]["total_s"])
        d = per_kind[dom]
        all_gbps = float(by.sum() * a.steps / durs.sum() / 1e9)
        tag = headline_tag(step, B)
        traffic, prof_us = profile_figures(tag)
        roof = {"bound": "hbm", "achieved": round(d["GBps"], 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(d["GBps"] / HBM_PEAK_GBPS, 4), "traffic": traffic,
                "kernel": KIND_NAMES[dom] + (" (direct palette)" if dom == "gate_up" else
                                             {"auto": " (autotuned plan)", "direct": " (direct palette)",
                                              "huff": " (Huffman decode in the matmul)"}.get(a.pipeline, "")),
                "launches": d["launches"], "avg_launch_us": round(d["avg_us"], 3),
                "bytes_per_launch": int(round(d["bytes"])), "profile_avg_us": prof_us,
                "all_matmuls_frac": round(all_gbps / HBM_PEAK_GBPS, 4),
                "per_kind_avg_us": {k: round(v["avg_us"], 2) for k, v in per_kind.items()}}
        log(f"roofline: {roof}")

    bf16_ms = None
    if not a.no_compare:
        choice = bf16_choice(layers, B, W5)
        sb = Step(layers, B, "bf16", stream, W5, bf16_choice={k: v[:2] for k, v in choice.items()})
        t_b, _ = time_steps(sb, a.steps, a.warmup, a.min_warmup_ms / 1e3)
        bf16_ms = t_b * 1e3
        detail["bf16_kernels"] = {f"{R}x{C}": v[2] for (R, C), v in choice.items()}
        del sb
        log(f"bf16 stack step B={B}: {bf16_ms:.4f} ms ({detail['bf16_kernels']})")

    compressed = sum(step.launch_bytes)
    out = {
        "metric": METRIC,
        "value": round(stats["bf16_bytes"] / sec / 1e9, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "warmup_steps_run": warm_run,
        "ms_per_step": round(sec * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "llama3.1-8b-mlp-stack", "layers": a.layers, "batch": B,
                   "gate_up": [F, H], "down": [H, F], "pipeline": a.pipeline, "plan": plan,
                   "gate_up_fused": step.fused,
                   "weights": "N(0,0.02)+U[0.01%,0.2%] N(0,0.5) outliers per layer, seeded"},
        "compressed_GBps": round(compressed / sec / 1e9, 1),
        "compressed_hbm_frac": round(compressed / sec / 1e9 / HBM_PEAK_GBPS, 4),
        "bf16_ms_per_step": bf16_ms and round(bf16_ms, 4),
        "speedup_vs_bf16": bf16_ms and round(bf16_ms / (sec * 1e3), 4),
        "sizes_GB": {"bf16": round(stats["bf16_bytes"] / 1e9, 2), "huffman": round(stats["huffman_bytes"] / 1e9, 2),
                     "palette": round(stats["palette_bytes"] / 1e9, 2)},
        "verbatim_group_frac": round(stats["verbatim_groups"] / max(stats["groups"], 1), 5),
        "decode_bitexact": f"{stats['decode_bitexact']}/{stats['decode_checked']}",
        "roofline": roof,
    }
    if graph:
        out["graph"] = graph
    if not a.no_sweep and not a.no_compare:
        sweep = stack_sweep(layers, [int(v) for v in a.sweep_batches.split(",") if v], W5, stream)
        detail["sweep"] = sweep
        out["sweep"] = {"cols": "batch,ms,bf16_ms,x_bf16",
                        "rows": [[r["batch"], round(r["ms"], 3), round(r["bf16_ms"], 3), round(r["speedup_vs_bf16"], 3)]
                                 for r in sweep]}
    if a.extras:
        del layers, step
        torch.cuda.empty_cache()
        import workloads as wl
        detail["one_layer"] = one_layer_pipelines([1, 4, 16], stream)
        detail["per_row_sigma"] = matrix_comparison(4, {0: wl.MLP_SHAPES[0], 2: wl.MLP_SHAPES[2]}, [64, 128, 256])
        detail["shards_tp8"] = matrix_comparison(5, {0: (wl.LLAMA_FFN // 8, wl.LLAMA_HIDDEN),
                                                     2: (wl.LLAMA_HIDDEN, wl.LLAMA_FFN // 8)},
                                                 [1, 16, 256], n_copies=48, pipes=("direct",))
        detail["attention"] = attention_bench([1, 4, 16])
        detail["output_projection"] = lm_head_bench([1, 4, 16])
    if not a.no_cpu_baseline:
        log("timing the CPU oracle")
        out["cpu_baseline"] = cpu_baseline(B)
    if a.detail:
        os.makedirs(os.path.dirname(os.path.abspath(a.detail)), exist_ok=True)
        with open(a.detail, "w") as f:
            json.dump({"headline": out, **detail}, f, indent=1, default=str)
        out["detail"] = os.path.relpath(a.detail, ROOT)
    print(json.dumps(out, separators=(",", ":"), ensure_ascii=False), flush=True)


if __name__ == "__main__":
    main()
