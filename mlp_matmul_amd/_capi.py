"""ctypes mirror of include/unweight.h.  Loading fails loudly if the library
has not been built: there is no fallback path."""
from __future__ import annotations

import ctypes as ct
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libunweight.so")

UW_OK = 0
UW_EINVAL = -1
UW_ENOMEM = -2
UW_EFORMAT = -3
UW_EHIP = -4
UW_EUNSUPPORTED = -5

(UW_SEC_SM, UW_SEC_STREAM, UW_SEC_GLEN, UW_SEC_TILE_OFF, UW_SEC_TILE_VBASE, UW_SEC_VEXP,
 UW_SEC_BITMAP, UW_SEC_NIB, UW_SEC_DLUT, UW_SEC_MLUT, UW_NUM_SECTIONS) = range(11)
SECTION_NAMES = ("sm", "stream", "glen", "tile_off", "tile_vbase", "vexp", "bitmap", "nib", "dlut", "mlut")

UW_KERNEL_AUTO, UW_KERNEL_GEMV, UW_KERNEL_MFMA, UW_KERNEL_SKINNY = 0, 1, 2, 3
UW_PIPE_AUTO, UW_PIPE_FULL, UW_PIPE_EXP, UW_PIPE_PAL, UW_PIPE_DIRECT, UW_PIPE_BF16, UW_PIPE_HUFF = range(7)
UW_STATIC_SCRATCH_BYTES = 64 << 20


class uw_opts(ct.Structure):
    _fields_ = [("emit_palette", ct.c_int), ("threads", ct.c_int)]


class uw_info(ct.Structure):
    _fields_ = [
        ("rows", ct.c_int64), ("cols", ct.c_int64),
        ("groups", ct.c_int64), ("tiles", ct.c_int64), ("verbatim_groups", ct.c_int64),
        ("palette_size", ct.c_int32), ("lmax", ct.c_int32),
        ("palette", ct.c_uint8 * 16), ("lengths", ct.c_uint8 * 16), ("codes", ct.c_uint16 * 16),
        ("hist", ct.c_uint64 * 256),
        ("section_bytes", ct.c_uint64 * UW_NUM_SECTIONS),
        ("huffman_form_bytes", ct.c_uint64), ("palette_form_bytes", ct.c_uint64),
        ("has_palette", ct.c_int32), ("max_tile_bytes", ct.c_uint32),
    ]


class uw_dmat(ct.Structure):
    _fields_ = [
        ("rows", ct.c_int64), ("cols", ct.c_int64), ("groups", ct.c_int64), ("tiles", ct.c_int64),
        ("verbatim_groups", ct.c_int64), ("stream_bytes", ct.c_uint64),
        ("max_tile_bytes", ct.c_uint64), ("palette_size", ct.c_int32), ("lmax", ct.c_int32), ("palette", ct.c_uint8 * 16),
        ("sm", ct.c_void_p), ("stream", ct.c_void_p), ("glen", ct.c_void_p), ("tile_off", ct.c_void_p),
        ("tile_vbase", ct.c_void_p), ("vexp", ct.c_void_p), ("bitmap", ct.c_void_p), ("nib", ct.c_void_p),
        ("dlut", ct.c_void_p), ("mlut", ct.c_void_p),
    ]


_P = ct.c_void_p
_I64 = ct.c_int64
_U64 = ct.c_uint64
_INT = ct.c_int

# name -> (restype, argtypes); every function declared in include/unweight.h
SIGNATURES = {
    "uw_last_error": (ct.c_char_p, []),
    "uw_version": (_INT, []),
    "uw_abi_struct_sizes": (_INT, [ct.POINTER(_U64), ct.POINTER(_U64), ct.POINTER(_U64)]),
    "uw_compress": (_INT, [_P, _I64, _I64, ct.POINTER(uw_opts), ct.POINTER(_P)]),
    "uw_blob_info": (_INT, [_P, ct.POINTER(uw_info)]),
    "uw_blob_section": (_INT, [_P, _INT, ct.POINTER(_P), ct.POINTER(_U64)]),
    "uw_blob_serialize": (_INT, [_P, _P, _U64, ct.POINTER(_U64)]),
    "uw_blob_deserialize": (_INT, [_P, _U64, ct.POINTER(_P)]),
    "uw_blob_add_palette": (_INT, [_P]),
    "uw_blob_free": (None, [_P]),
    "uw_validate": (_INT, [_P]),
    "uw_dmat_init": (_INT, [ct.POINTER(uw_dmat), ct.POINTER(uw_info), ct.POINTER(_P)]),
    "uw_decode_full": (_INT, [ct.POINTER(uw_dmat), _P, _P]),
    "uw_decode_exponents": (_INT, [ct.POINTER(uw_dmat), _P, _P]),
    "uw_transcode_palette": (_INT, [ct.POINTER(uw_dmat), _P, _P]),
    "uw_gemm_bf16": (_INT, [_P, _I64, _I64, _P, _I64, _P, _INT, _INT, _P, _U64, _P]),
    "uw_gemm_recon_exp": (_INT, [ct.POINTER(uw_dmat), _P, _P, _I64, _P, _INT, _INT, _P, _U64, _P]),
    "uw_gemm_recon_pal": (_INT, [ct.POINTER(uw_dmat), _P, _P, _I64, _P, _INT, _INT, _P, _U64, _P]),
    "uw_gemm_recon_pal_static": (_INT, [ct.POINTER(uw_dmat), _P, _P, _I64, _P, _INT, _INT, _P]),
    "uw_scratch_bytes": (_I64, [_INT, _I64, _I64, _I64, _INT]),
    "uw_matmul": (_INT, [ct.POINTER(uw_dmat), _INT, _INT, _INT, _P, _I64, _P, _P, _U64, _P]),
    "uw_silu_mul_bf16": (_INT, [_P, _P, _I64, _P, _P]),
    "uw_mlp_gate_up": (_INT, [ct.POINTER(uw_dmat), ct.POINTER(uw_dmat), _P, _I64, _P, _P, _P, _P]),
    "uw_mlp_scratch_bytes": (_I64, [_INT, _I64, _I64, _I64]),
    "uw_mlp_layer": (_INT, [ct.POINTER(uw_dmat), ct.POINTER(uw_dmat), ct.POINTER(uw_dmat), _INT, _P, _I64, _P, _P,
                             _U64, _P, _P]),
    "uw_kernel_timer_enable": (_INT, [_INT]),
    "uw_kernel_timer_disable": (_INT, []),
    "uw_kernel_timer_reset": (_INT, []),
    "uw_kernel_timer_read": (_INT, [ct.POINTER(ct.c_float), _INT, ct.POINTER(_INT)]),
    "uw_plan_set": (_INT, [_I64, _I64, _I64, _INT, _INT, _INT]),
    "uw_plan_lookup": (_INT, [_I64, _I64, _I64, ct.POINTER(_INT), ct.POINTER(_INT), ct.POINTER(_INT)]),
    "uw_plan_clear": (_INT, []),
    "uw_plan_count": (_INT, []),
    "uw_plan_save": (_INT, [ct.c_char_p]),
    "uw_plan_load": (_INT, [ct.c_char_p]),
}

_lib = None


class UnweightError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"{msg} (code {code})")
        self.code = code


def lib():
    """The loaded libunweight.so with every signature declared."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with mlp_matmul_amd/build.py "
                               "(or __graft_entry__.build()); there is no fallback path")
        L = ct.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        sizes = [_U64(), _U64(), _U64()]
        L.uw_abi_struct_sizes(*[ct.byref(s) for s in sizes])
        mine = (ct.sizeof(uw_info), ct.sizeof(uw_dmat), ct.sizeof(uw_opts))
        if tuple(s.value for s in sizes) != mine:
            raise RuntimeError(f"ABI struct size mismatch: library {[s.value for s in sizes]}, binding {mine}")
        _lib = L
    return _lib


def check(rc, what=""):
    if rc != UW_OK:
        msg = lib().uw_last_error().decode(errors="replace")
        raise UnweightError(rc, f"{what}: {msg}" if what else msg)
    return rc
