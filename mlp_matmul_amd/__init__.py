"""MI355X (gfx950) compressed-MLP matmul: Python binding of libunweight.

Argument marshalling only: every step runs in libunweight's host code or
gfx950 kernels.  PyTorch provides device memory and the current HIP stream.
The names follow include/unweight.h without the ``uw_`` prefix.

Method: Cloudflare, "Unweight: how we compressed an LLM 22% without
sacrificing quality" -- lossless BF16 exponent compression of MLP weights with
four pipelines ("Four ways to use compressed weights") and a reconstructive
matmul ("How the reconstructive matmul works").
"""
from __future__ import annotations

import ctypes as ct

import numpy as np

from ._capi import (  # noqa: F401
    SECTION_NAMES, UW_KERNEL_AUTO, UW_KERNEL_GEMV, UW_KERNEL_MFMA, UW_KERNEL_SKINNY, UW_NUM_SECTIONS,
    UW_PIPE_AUTO, UW_PIPE_BF16, UW_PIPE_DIRECT, UW_PIPE_EXP, UW_PIPE_FULL, UW_PIPE_HUFF, UW_PIPE_PAL,
    UW_SEC_BITMAP, UW_SEC_DLUT, UW_SEC_GLEN, UW_SEC_MLUT, UW_SEC_NIB, UW_SEC_SM, UW_SEC_STREAM,
    UW_SEC_TILE_OFF, UW_SEC_TILE_VBASE, UW_SEC_VEXP, UW_EUNSUPPORTED, UW_EINVAL, UW_STATIC_SCRATCH_BYTES,
    UnweightError, check, lib,
    uw_dmat, uw_info,
    uw_opts,
)

PIPELINES = {"full": UW_PIPE_FULL, "exp": UW_PIPE_EXP, "pal": UW_PIPE_PAL, "direct": UW_PIPE_DIRECT}
KERNELS = {"auto": UW_KERNEL_AUTO, "gemv": UW_KERNEL_GEMV, "mfma": UW_KERNEL_MFMA, "skinny": UW_KERNEL_SKINNY}

# sections each use reads on the device
DECODE_SECTIONS = ("sm", "stream", "glen", "tile_off", "tile_vbase", "vexp", "bitmap", "dlut", "mlut")
DIRECT_SECTIONS = ("sm", "nib", "vexp", "bitmap", "tile_vbase")
SECTION_DTYPES = {"sm": np.uint8, "stream": np.uint8, "glen": np.uint8, "tile_off": np.uint32,
                  "tile_vbase": np.uint32, "vexp": np.uint8, "bitmap": np.uint64, "nib": np.uint8,
                  "dlut": np.uint8, "mlut": np.uint32}


def _torch():
    import torch
    return torch


def _stream(stream):
    if stream is not None:
        return ct.c_void_p(stream)
    return ct.c_void_p(_torch().cuda.current_stream().cuda_stream)


def _ptr(t):
    return ct.c_void_p(0 if t is None else t.data_ptr())


# ------------------------------------------------------------------ host blob
class Blob:
    """A compressed matrix on the host (owns a uw_blob*)."""

    def __init__(self, handle: ct.c_void_p):
        self._h = handle

    def __del__(self):
        h = getattr(self, "_h", None)
        if h and h.value:
            lib().uw_blob_free(h)
            self._h = None

    @property
    def handle(self):
        return self._h

    def info(self) -> uw_info:
        inf = uw_info()
        check(lib().uw_blob_info(self._h, ct.byref(inf)), "uw_blob_info")
        return inf

    def section(self, name) -> np.ndarray:
        """Copy of a section as a numpy array of its on-disk dtype."""
        idx = SECTION_NAMES.index(name)
        p, n = ct.c_void_p(), ct.c_uint64()
        check(lib().uw_blob_section(self._h, idx, ct.byref(p), ct.byref(n)), "uw_blob_section")
        if n.value == 0:
            return np.zeros(0, dtype=SECTION_DTYPES[name])
        raw = np.ctypeslib.as_array(ct.cast(p, ct.POINTER(ct.c_uint8)), shape=(n.value,)).copy()
        return raw.view(SECTION_DTYPES[name])

    def validate(self):
        check(lib().uw_validate(self._h), "uw_validate")

    def add_palette(self):
        check(lib().uw_blob_add_palette(self._h), "uw_blob_add_palette")

    def serialize(self) -> bytes:
        need = ct.c_uint64()
        check(lib().uw_blob_serialize(self._h, None, 0, ct.byref(need)), "uw_blob_serialize")
        buf = (ct.c_uint8 * need.value)()
        check(lib().uw_blob_serialize(self._h, buf, need.value, ct.byref(need)), "uw_blob_serialize")
        return bytes(buf)

    @staticmethod
    def deserialize(data: bytes) -> "Blob":
        h = ct.c_void_p()
        buf = (ct.c_uint8 * len(data)).from_buffer_copy(data)
        check(lib().uw_blob_deserialize(buf, len(data), ct.byref(h)), "uw_blob_deserialize")
        return Blob(h)

    def to_device(self, sections=DECODE_SECTIONS + ("nib",), device="cuda") -> "DeviceMatrix":
        return DeviceMatrix(self, sections, device)


def compress(w, emit_palette: bool = True, threads: int = 0) -> Blob:
    """uw_compress on a host [rows, cols] array of bf16 bit patterns."""
    a = np.ascontiguousarray(np.asarray(w).view(np.uint16))
    if a.ndim != 2:
        raise ValueError("w must be 2-D [rows, cols]")
    h = ct.c_void_p()
    opts = uw_opts(1 if emit_palette else 0, int(threads))
    check(lib().uw_compress(a.ctypes.data_as(ct.c_void_p), a.shape[0], a.shape[1], ct.byref(opts),
                            ct.byref(h)), "uw_compress")
    return Blob(h)


# ---------------------------------------------------------- device matrices
class DeviceMatrix:
    """A compressed matrix with the chosen sections copied to device memory
    (torch uint8 buffers, 16-byte padded) and its uw_dmat descriptor."""

    def __init__(self, blob: Blob, sections, device="cuda"):
        torch = _torch()
        self.info = blob.info()
        self.buffers = {}
        ptrs = (ct.c_void_p * UW_NUM_SECTIONS)()
        for name in sections:
            host = blob.section(name)
            if host.nbytes == 0:
                continue
            raw = host.view(np.uint8)
            pad = (-raw.size) % 16 + 16
            t = torch.zeros(raw.size + pad, dtype=torch.uint8, device=device)
            t[:raw.size].copy_(torch.from_numpy(raw))
            self.buffers[name] = t
            ptrs[SECTION_NAMES.index(name)] = t.data_ptr()
        self.dmat = uw_dmat()
        check(lib().uw_dmat_init(ct.byref(self.dmat), ct.byref(self.info), ptrs), "uw_dmat_init")

    @property
    def rows(self):
        return self.info.rows

    @property
    def cols(self):
        return self.info.cols

    def device_bytes(self):
        return sum(int(self.info.section_bytes[SECTION_NAMES.index(n)]) for n in self.buffers)


# ---------------------------------------------------------------- operations
def decode_full(dm: DeviceMatrix, out=None, stream=None):
    torch = _torch()
    if out is None:
        out = torch.empty((dm.rows, dm.cols), dtype=torch.bfloat16, device="cuda")
    check(lib().uw_decode_full(ct.byref(dm.dmat), _ptr(out), _stream(stream)), "uw_decode_full")
    return out


def decode_exponents(dm: DeviceMatrix, out=None, stream=None):
    torch = _torch()
    if out is None:
        out = torch.empty((dm.rows, dm.cols), dtype=torch.uint8, device="cuda")
    check(lib().uw_decode_exponents(ct.byref(dm.dmat), _ptr(out), _stream(stream)), "uw_decode_exponents")
    return out


def transcode_palette(dm: DeviceMatrix, out=None, stream=None):
    torch = _torch()
    if out is None:
        out = torch.empty((dm.rows * dm.cols // 2,), dtype=torch.uint8, device="cuda")
    check(lib().uw_transcode_palette(ct.byref(dm.dmat), _ptr(out), _stream(stream)), "uw_transcode_palette")
    return out


def _y(Y, batch, rows):
    if Y is None:
        Y = _torch().empty((batch, rows), dtype=_torch().float32, device="cuda")
    return Y


def _scratch_args(scratch):
    if scratch is None:
        return ct.c_void_p(0), 0
    return _ptr(scratch), scratch.numel() * scratch.element_size()


def gemm_bf16(W, X, Y=None, kernel=UW_KERNEL_AUTO, split_k=1, scratch=None, stream=None):
    rows, cols = W.shape
    batch = X.shape[0]
    Y = _y(Y, batch, rows)
    sp, sb = _scratch_args(scratch)
    check(lib().uw_gemm_bf16(_ptr(W), rows, cols, _ptr(X), batch, _ptr(Y), kernel, split_k, sp, sb,
                             _stream(stream)), "uw_gemm_bf16")
    return Y


def gemm_recon_exp(dm: DeviceMatrix, e, X, Y=None, kernel=UW_KERNEL_AUTO, split_k=1, scratch=None, stream=None):
    batch = X.shape[0]
    Y = _y(Y, batch, dm.rows)
    sp, sb = _scratch_args(scratch)
    check(lib().uw_gemm_recon_exp(ct.byref(dm.dmat), _ptr(e), _ptr(X), batch, _ptr(Y), kernel, split_k, sp, sb,
                                  _stream(stream)), "uw_gemm_recon_exp")
    return Y


def gemm_recon_pal(dm: DeviceMatrix, nib, X, Y=None, kernel=UW_KERNEL_AUTO, split_k=1, scratch=None,
                   stream=None):
    batch = X.shape[0]
    Y = _y(Y, batch, dm.rows)
    sp, sb = _scratch_args(scratch)
    nibp = _ptr(nib) if nib is not None else ct.c_void_p(dm.dmat.nib)
    check(lib().uw_gemm_recon_pal(ct.byref(dm.dmat), nibp, _ptr(X), batch, _ptr(Y), kernel, split_k, sp, sb,
                                  _stream(stream)), "uw_gemm_recon_pal")
    return Y


def gemm_recon_pal_static(dm: DeviceMatrix, nib, X, Y=None, kernel=UW_KERNEL_AUTO, split_k=0, stream=None):
    """uw_gemm_recon_pal_static: the palette-source matmul with its split-K
    partials in the library's static device array (no caller scratch)."""
    batch = X.shape[0]
    Y = _y(Y, batch, dm.rows)
    nibp = _ptr(nib) if nib is not None else ct.c_void_p(dm.dmat.nib)
    check(lib().uw_gemm_recon_pal_static(ct.byref(dm.dmat), nibp, _ptr(X), batch, _ptr(Y), kernel, split_k,
                                         _stream(stream)), "uw_gemm_recon_pal_static")
    return Y


def scratch_bytes(pipeline, rows, cols, batch, split_k=1) -> int:
    n = lib().uw_scratch_bytes(pipeline, rows, cols, batch, split_k)
    if n < 0:
        check(int(n), "uw_scratch_bytes")
    return int(n)


def alloc_scratch(pipeline, rows, cols, batch, split_k=1):
    n = scratch_bytes(pipeline, rows, cols, batch, split_k)
    return _torch().empty(max(n, 16), dtype=_torch().uint8, device="cuda")


def matmul(dm: DeviceMatrix, X, pipeline=UW_PIPE_AUTO, kernel=UW_KERNEL_AUTO, split_k=1, Y=None, scratch=None,
           stream=None):
    batch = X.shape[0]
    Y = _y(Y, batch, dm.rows)
    sp, sb = _scratch_args(scratch)
    check(lib().uw_matmul(ct.byref(dm.dmat), pipeline, kernel, split_k, _ptr(X), batch, _ptr(Y), sp, sb,
                          _stream(stream)), "uw_matmul")
    return Y


def mlp_gate_up(gate: DeviceMatrix, up: DeviceMatrix, X, h=None, g=None, u=None, stream=None):
    """h = bf16(SiLU(X.gate^T) * (X.up^T)) in one fused launch (direct-palette
    form, batch 1..16, and 17..32 on matrices of at least 48 rows per compute
    unit); g and u (fp32) are also written when given."""
    torch = _torch()
    batch = X.shape[0]
    if h is None:
        h = torch.empty((batch, gate.rows), dtype=torch.bfloat16, device="cuda")
    check(lib().uw_mlp_gate_up(ct.byref(gate.dmat), ct.byref(up.dmat), _ptr(X), batch, _ptr(h),
                               _ptr(g) if g is not None else None, _ptr(u) if u is not None else None,
                               _stream(stream)), "uw_mlp_gate_up")
    return h


def mlp_scratch_bytes(pipeline, rows, cols, batch) -> int:
    n = lib().uw_mlp_scratch_bytes(pipeline, rows, cols, batch)
    if n < 0:
        check(int(n), "uw_mlp_scratch_bytes")
    return int(n)


def mlp_layer(gate: DeviceMatrix, up: DeviceMatrix, down: DeviceMatrix, X, pipeline=UW_PIPE_DIRECT, y=None,
              scratch=None, stream=None, aux_stream=None):
    """y = down . bf16(SiLU(X.gate^T) * (X.up^T)) through one pipeline; with an
    aux_stream the decodes overlap the matmuls (uw_mlp_layer)."""
    torch = _torch()
    batch = X.shape[0]
    if y is None:
        y = torch.empty((batch, down.rows), dtype=torch.float32, device="cuda")
    if scratch is None:
        scratch = torch.empty(max(mlp_scratch_bytes(pipeline, gate.rows, gate.cols, batch), 16), dtype=torch.uint8,
                              device="cuda")
    aux = ct.c_void_p(aux_stream) if aux_stream is not None else None
    check(lib().uw_mlp_layer(ct.byref(gate.dmat), ct.byref(up.dmat), ct.byref(down.dmat), pipeline, _ptr(X), batch,
                             _ptr(y), _ptr(scratch), scratch.numel(), _stream(stream), aux), "uw_mlp_layer")
    return y


def silu_mul_bf16(g, u, h=None, stream=None):
    torch = _torch()
    if h is None:
        h = torch.empty(g.shape, dtype=torch.bfloat16, device="cuda")
    check(lib().uw_silu_mul_bf16(_ptr(g), _ptr(u), g.numel(), _ptr(h), _stream(stream)), "uw_silu_mul_bf16")
    return h


class KernelTimer:
    """Context manager: durations (ms) of the matmul kernels launched inside it,
    recorded by the launches themselves (uw_kernel_timer_*)."""

    def __init__(self, capacity=4096):
        self.capacity = capacity
        self.ms = []

    def __enter__(self):
        check(lib().uw_kernel_timer_enable(self.capacity), "uw_kernel_timer_enable")
        return self

    def __exit__(self, *exc):
        lib().uw_kernel_timer_disable()
        n = ct.c_int()
        buf = (ct.c_float * self.capacity)()
        check(lib().uw_kernel_timer_read(buf, self.capacity, ct.byref(n)), "uw_kernel_timer_read")
        self.ms = [buf[i] for i in range(min(n.value, self.capacity))]
        return False


def plan_set(rows, cols, batch, pipeline, kernel=UW_KERNEL_AUTO, split_k=1):
    check(lib().uw_plan_set(rows, cols, batch, pipeline, kernel, split_k), "uw_plan_set")


def plan_lookup(rows, cols, batch):
    p, k, s = ct.c_int(), ct.c_int(), ct.c_int()
    rc = lib().uw_plan_lookup(rows, cols, batch, ct.byref(p), ct.byref(k), ct.byref(s))
    return (p.value, k.value, s.value) if rc == 0 else None


def plan_clear():
    check(lib().uw_plan_clear(), "uw_plan_clear")


def plan_count() -> int:
    return int(lib().uw_plan_count())


def plan_save(path):
    check(lib().uw_plan_save(str(path).encode()), "uw_plan_save")


def plan_load(path):
    check(lib().uw_plan_load(str(path).encode()), "uw_plan_load")
