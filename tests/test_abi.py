"""The C-ABI library loads and exports every function include/unweight.h
declares, and the binding's struct mirrors match the compiled sizes.  No
device calls."""
import os
import re
import subprocess

import pytest

import mlp_matmul_amd as uw
from mlp_matmul_amd import _capi

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "unweight.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(uw_[a-z0-9_]+)\s*\(", src)))


def test_header_declares_the_binding_signatures():
    assert _declared() == sorted(_capi.SIGNATURES)


def test_library_exports_every_declared_symbol():
    out = subprocess.run(["nm", "-D", "--defined-only", _capi.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = set(re.findall(r"\bT (uw_[a-z0-9_]+)\b", out))
    missing = [n for n in _declared() if n not in exported]
    assert not missing, missing


def test_library_loads_and_struct_sizes_match():
    L = uw.lib()   # raises on a size mismatch
    assert L.uw_version() >> 16 == 1


def test_errors_are_reported_not_raised():
    L = uw.lib()
    import ctypes as ct
    h = ct.c_void_p()
    rc = L.uw_compress(None, 1, 100, None, ct.byref(h))
    assert rc == _capi.UW_EINVAL
    assert b"multiple of 64" in L.uw_last_error()
    assert L.uw_scratch_bytes(99, 1, 64, 1, 1) == _capi.UW_EINVAL


def test_no_fallback_when_library_missing(monkeypatch, tmp_path):
    monkeypatch.setattr(_capi, "LIB_PATH", str(tmp_path / "absent.so"))
    monkeypatch.setattr(_capi, "_lib", None)
    with pytest.raises(RuntimeError, match="no fallback"):
        _capi.lib()


def _fake_dmat(blob, drop=(), **override):
    """A descriptor whose device pointers are aligned placeholders: the calls
    below must reject it during argument checks, before any launch."""
    import ctypes as ct
    info = blob.info()
    ptrs = (ct.c_void_p * _capi.UW_NUM_SECTIONS)()
    for i, name in enumerate(_capi.SECTION_NAMES):
        if name not in drop:
            ptrs[i] = 0x10000 * (i + 1)
    d = _capi.uw_dmat()
    assert uw.lib().uw_dmat_init(ct.byref(d), ct.byref(info), ptrs) == 0
    for k, v in override.items():
        setattr(d, k, v)
    return d


def test_decoders_check_descriptors_before_launch():
    import ctypes as ct
    import workloads
    L = uw.lib()
    b = uw.compress(workloads.small_matrix()[0])
    inf = b.info()
    assert 0 < inf.max_tile_bytes <= 512 * inf.lmax
    # the multi-symbol table is required by every decoder
    d = _fake_dmat(b, drop=("mlut",))
    assert L.uw_transcode_palette(ct.byref(d), ct.c_void_p(0x100000), None) == _capi.UW_EINVAL
    assert b"NULL" in L.uw_last_error()
    # a longest-tile size no tile of lmax-bit codes can reach sizes no LDS buffer
    d = _fake_dmat(b, max_tile_bytes=512 * inf.lmax + 2)
    assert L.uw_decode_full(ct.byref(d), ct.c_void_p(0x100000), None) == _capi.UW_EINVAL
    assert b"max_tile_bytes" in L.uw_last_error()
    d = _fake_dmat(b, max_tile_bytes=0)
    assert L.uw_decode_exponents(ct.byref(d), ct.c_void_p(0x100000), None) == _capi.UW_EINVAL


def test_scratch_for_library_split_choice():
    """split_k 0 sizes scratch for the largest split the library would pick
    over the weight sources: none for the GEMV batches; at batch 256 a
    4096x14336 matrix has 32 tiles of 128 rows x 256 columns (eight
    K-slices) and a 14336x4096 one 224 of 128 x 128 (none), the CU count
    falling back to 256 without a device."""
    L = uw.lib()
    P = _capi.UW_PIPE_DIRECT
    assert L.uw_scratch_bytes(P, 4096, 14336, 1, 0) == 0
    assert L.uw_scratch_bytes(P, 4096, 14336, 256, 0) == 8 * 256 * 4096 * 4
    assert L.uw_scratch_bytes(P, 14336, 4096, 256, 0) == 0
    assert L.uw_scratch_bytes(P, 4096, 14336, 256, -1) == _capi.UW_EINVAL


def test_mlp_scratch_bytes():
    """Scratch of one MLP block: a decoded plane per matrix, g, u, h and the
    split-K partials; rejects shapes that are not whole 64-element groups."""
    L = uw.lib()
    F, H, B = 14336, 4096, 1
    planes = {_capi.UW_PIPE_FULL: 2 * F * H, _capi.UW_PIPE_EXP: F * H, _capi.UW_PIPE_PAL: F * H // 2,
              _capi.UW_PIPE_DIRECT: 0}
    for p, n in planes.items():
        assert L.uw_mlp_scratch_bytes(p, F, H, B) == 3 * n + 2 * B * F * 4 + 256 * ((B * F * 2 + 255) // 256)
    assert L.uw_mlp_scratch_bytes(_capi.UW_PIPE_AUTO, F, H, B) == _capi.UW_EINVAL
    assert L.uw_mlp_scratch_bytes(_capi.UW_PIPE_PAL, F, 100, B) == _capi.UW_EINVAL
