"""The C++ host compressor produces byte-identical sections to the oracle
encoder, its validator rejects corrupted blobs, and blobs round-trip through
serialization.  Host code only, no device."""
import numpy as np
import pytest

import mlp_matmul_amd as uw
from oracle import codec
import workloads

SEC = ("sm", "stream", "glen", "tile_off", "tile_vbase", "vexp", "bitmap", "nib")


def _same_as_oracle(w, threads=0):
    ref = codec.encode(w)
    b = uw.compress(w, emit_palette=True, threads=threads)
    inf = b.info()
    assert inf.rows == ref.R and inf.cols == ref.C
    assert inf.palette_size == ref.P
    assert list(inf.palette)[:ref.P] == list(ref.palette)
    assert list(inf.lengths) == list(ref.lengths)
    coded = [s for s in range(16) if ref.lengths[s]]
    assert [inf.codes[s] for s in coded] == [int(ref.codes[s]) for s in coded]
    assert inf.verbatim_groups == ref.V
    assert list(inf.hist) == list(ref.hist)
    for name in SEC:
        got = b.section(name)
        exp = getattr(ref, name)
        assert got.dtype == exp.dtype, name
        assert np.array_equal(got, exp), name
    assert inf.huffman_form_bytes == codec.huffman_form_bytes(ref)
    assert inf.palette_form_bytes == codec.palette_form_bytes(ref)
    # decode table: entry v names the codeword prefixing the lmax-bit string v
    lsym, llen, lmax = codec.decode_lut(ref.lengths, ref.codes)
    dl = b.section("dlut")
    if lmax:
        covered = llen > 0
        assert np.array_equal(dl[covered] >> 4, lsym[covered])
        assert np.array_equal(dl[covered] & 15, llen[covered])
    _check_multi_symbol_table(b.section("mlut"), lsym, llen, lmax)
    b.validate()
    return b, ref


def _check_multi_symbol_table(ml, lsym, llen, lmax):
    """Entry v of the 12-bit multi-symbol table must hold exactly the codewords
    that the oracle's one-codeword table decodes one after another from the
    string v while each lies wholly inside it, at most four: their total
    length (bits 0-7), four times their count (bits 8-15) and their symbols
    (4 bits each from bit 16).  Strings the oracle's table does not cover
    (possible only with one coded symbol) are checked up to that point."""
    assert ml.dtype == np.uint32 and ml.size == 4096
    if lmax == 0:
        assert not ml.any()
        return
    v = np.arange(4096, dtype=np.int64)
    used = np.zeros_like(v)
    n = np.zeros_like(v)
    syms = np.zeros_like(v)
    alive = np.ones(v.size, bool)
    covered = np.ones(v.size, bool)
    for _ in range(4):
        rest = (v << used) & 0xFFF
        idx = rest >> (12 - lmax) if lmax <= 12 else rest << (lmax - 12)
        ln = llen[idx]
        covered &= ~(alive & (ln == 0))
        take = alive & (ln > 0) & (used + ln <= 12)
        syms = np.where(take, syms | (lsym[idx] << (16 + 4 * n)), syms)
        used = np.where(take, used + ln, used)
        n = np.where(take, n + 1, n)
        alive &= take
    got = ml.astype(np.int64)
    assert np.array_equal(got[covered], (used | (4 * n) << 8 | syms)[covered])
    # uncovered strings: the symbols decoded before the gap agree
    keep = (1 << 16) * ((1 << (4 * n)) - 1)
    assert ((got >> 8 & 0xFF)[~covered] >= 4 * n[~covered]).all()
    assert np.array_equal((got & keep)[~covered], syms[~covered])
    # with two or more coded symbols the code is complete: every string decodes
    if (llen > 0).any() and len(set(lsym[llen > 0].tolist())) >= 2:
        assert covered.all()


def test_small_workload_identical():
    w, _ = workloads.small_matrix()
    _same_as_oracle(w)


@pytest.mark.parametrize("wl,m,shape", [(2, 0, (1024, 4096)), (2, 2, (256, 14336)), (4, 0, (512, 4096)),
                                         (4, 2, (128, 14336)), (5, 1, (512, 4096))])
def test_layer_distributions_identical(wl, m, shape):
    _same_as_oracle(workloads.layer_weight(wl, 2, m, shape=shape))


@pytest.mark.parametrize("threads", [1, 3, 8])
def test_thread_count_does_not_change_bytes(threads):
    w = workloads.layer_weight(2, 0, 0, shape=(300, 4096))
    _same_as_oracle(w, threads=threads)


def _bits(sign, e, m):
    return ((np.asarray(sign, np.uint16) << 15) | (np.asarray(e, np.uint16) << 7)
            | np.asarray(m, np.uint16)).astype(np.uint16)


@pytest.mark.parametrize("case", ["single", "sixteen", "spread", "random", "special", "partial", "tiny", "empty"])
def test_edge_cases_identical(case):
    rng = np.random.default_rng(42)
    if case == "single":
        w = _bits(rng.integers(0, 2, (9, 128)), 119, rng.integers(0, 128, (9, 128)))
    elif case == "sixteen":
        w = _bits(rng.integers(0, 2, (16, 256)), rng.integers(100, 116, (16, 256)), rng.integers(0, 128, (16, 256)))
    elif case == "spread":
        w = _bits(rng.integers(0, 2, (16, 256)), rng.integers(90, 122, (16, 256)), rng.integers(0, 128, (16, 256)))
    elif case == "random":
        w = workloads.random_bf16_bits(3, 64 * 300).reshape(150, 128)
    elif case == "special":
        w = workloads.gaussian_weights(rng, 40, 192, 0.02)
        flat = w.ravel()
        sp = np.array([0, 0x8000, 1, 0x807F, 0x7F80, 0xFF80, 0x7FC0, 0x7F81, 0xFFFF], np.uint16)
        flat[rng.choice(flat.size, sp.size * 4, replace=False)] = np.tile(sp, 4)
    elif case == "partial":
        w = workloads.gaussian_weights(rng, 65, 64, 0.02, 0.02, 1.0)
    elif case == "tiny":
        w = workloads.gaussian_weights(rng, 1, 64, 0.02)
    else:
        w = np.zeros((0, 64), np.uint16)
    _same_as_oracle(w)


def test_golden_examples_through_cpp(golden_dir):
    import json
    import os
    ex = json.load(open(os.path.join(golden_dir, "codec_worked_examples.json")))
    for name, e in ex.items():
        w = np.array([int(h, 16) for h in e["bf16_hex"]], np.uint16).reshape(e["rows"], e["cols"])
        b = uw.compress(w)
        assert b.section("stream").tobytes().hex() == e["stream_hex"], name
        assert b.section("nib").tobytes().hex() == e["nib_hex"], name
        assert b.section("vexp").tobytes().hex() == e["vexp_hex"], name


def test_attention_shape_identical():
    """The second workload (an attention projection, 1024x4096): same bytes as
    the oracle encoder."""
    _same_as_oracle(workloads.attention_weight(0, "k"))


def test_long_tile_identical():
    """Geometric exponent frequencies give 15-bit codewords and one tile far
    longer than the average (more than 4 KiB of stream): same bytes as the
    oracle encoder, and the longest tile is what the blob reports."""
    b, ref = _same_as_oracle(workloads.geometric_exponent_matrix())
    inf = b.info()
    assert inf.lmax == 15 and inf.verbatim_groups == 0
    assert inf.max_tile_bytes == int(np.diff(ref.tile_off.astype(np.int64)).max()) > 4096


def test_rejects_bad_shape():
    with pytest.raises(uw.UnweightError):
        uw.compress(np.zeros((2, 96), np.uint16))


def test_serialize_roundtrip_and_add_palette():
    w, _ = workloads.small_matrix()
    b = uw.compress(w, emit_palette=False)
    assert b.section("nib").size == 0
    data = b.serialize()
    assert data[:4] == b"UWF2" and len(data) % 256 == 0
    b2 = uw.Blob.deserialize(data)
    for name in SEC:
        assert np.array_equal(b.section(name), b2.section(name)), name
    assert np.array_equal(b.section("dlut"), b2.section("dlut"))
    assert np.array_equal(b.section("mlut"), b2.section("mlut"))
    b2.add_palette()
    assert np.array_equal(b2.section("nib"), codec.encode(w).nib)
    b3 = uw.Blob.deserialize(b2.serialize())
    assert np.array_equal(b3.section("nib"), b2.section("nib"))


def _corrupt(data, off, value):
    d = bytearray(data)
    d[off] = value
    return bytes(d)


def _section_offset(data, idx):
    import struct
    sizes = struct.unpack_from("<8Q", data, 72)
    pos = 256
    for s in range(idx):
        pos = (pos + 255) // 256 * 256 + sizes[s]
    return (pos + 255) // 256 * 256, sizes[idx]


def test_validator_rejects_corruption():
    w, _ = workloads.small_matrix()
    data = uw.compress(w).serialize()
    uw.Blob.deserialize(data)    # intact blob passes
    bad = [
        _corrupt(data, 0, ord("X")),                   # magic
        _corrupt(data, 56, 14),                        # a code length -> Kraft sum != 1
        _corrupt(data, 32, 17),                        # palette size
    ]
    off, n = _section_offset(data, 2)                  # GLEN: change one group's bit length
    bad.append(_corrupt(data, off + 4, data[off + 4] ^ 0x10))
    off, n = _section_offset(data, 3)                  # TILE_OFF not monotone / wrong size
    bad.append(_corrupt(data, off + 5, 0xFF))
    off, n = _section_offset(data, 6)                  # BITMAP: flag a coded group verbatim
    bmp = np.frombuffer(data[off:off + n], np.uint64)
    t = int(np.nonzero(bmp != np.uint64(0xFFFFFFFFFFFFFFFF))[0][0])
    word = int(bmp[t])
    free_bit = next(i for i in range(64) if not (word >> i) & 1)
    d = bytearray(data)
    d[off + 8 * t + free_bit // 8] |= 1 << (free_bit % 8)
    bad.append(bytes(d))
    bad.append(data[:len(data) // 2])                  # truncated
    for k, blob in enumerate(bad):
        with pytest.raises(uw.UnweightError) as ei:
            uw.Blob.deserialize(blob)
        assert ei.value.code == -3, k


def test_plan_table_roundtrip(tmp_path):
    uw.plan_clear()
    uw.plan_set(14336, 4096, 1, uw.UW_PIPE_DIRECT, uw.UW_KERNEL_GEMV, 1)
    uw.plan_set(4096, 14336, 256, uw.UW_PIPE_PAL, uw.UW_KERNEL_MFMA, 4)
    assert uw.plan_lookup(14336, 4096, 1) == (uw.UW_PIPE_DIRECT, uw.UW_KERNEL_GEMV, 1)
    assert uw.plan_lookup(1, 64, 1) is None
    p = tmp_path / "plan.txt"
    uw.plan_save(p)
    uw.plan_clear()
    assert uw.plan_count() == 0
    uw.plan_load(p)
    assert uw.plan_count() == 2
    assert uw.plan_lookup(4096, 14336, 256) == (uw.UW_PIPE_PAL, uw.UW_KERNEL_MFMA, 4)
    with pytest.raises(uw.UnweightError):
        uw.plan_set(1, 64, 1, 7, 0, 1)
    with pytest.raises(uw.UnweightError):
        uw.plan_set(1, 64, 1, uw.UW_PIPE_BF16, 0, 1)
    uw.plan_set(14336, 4096, 1, uw.UW_PIPE_HUFF, uw.UW_KERNEL_AUTO, 1)      # the autotuner may pick it
    assert uw.plan_lookup(14336, 4096, 1) == (uw.UW_PIPE_HUFF, uw.UW_KERNEL_AUTO, 1)
    uw.plan_clear()


def test_plan_file_device_key(tmp_path):
    """A plan file names the device it was tuned on; another device's plan,
    a file without that line and a malformed entry are refused and leave the
    table as it was."""
    uw.plan_clear()
    uw.plan_set(4096, 14336, 16, uw.UW_PIPE_DIRECT, uw.UW_KERNEL_SKINNY, 1)
    p = tmp_path / "plan.txt"
    uw.plan_save(p)
    head, *entries = p.read_text().splitlines()
    magic, device = head.split()
    assert magic == "uwplan-v2" and device                # "none" here, "<arch>/<cus>cu" on a GPU
    assert entries == [f"4096 14336 16 {uw.UW_PIPE_DIRECT} {uw.UW_KERNEL_SKINNY} 1"]
    other = tmp_path / "other.txt"
    other.write_text("uwplan-v2 gfx000:test/1cu\n1 64 1 4 0 1\n")
    no_head = tmp_path / "nohead.txt"
    no_head.write_text("1 64 1 4 0 1\n")
    bad = tmp_path / "bad.txt"
    bad.write_text(f"uwplan-v2 {device}\n1 64 1 4 0 1\n1 64 2 9 0 1\n")
    for path, code in ((other, -5), (no_head, -3), (bad, -3)):
        with pytest.raises(uw.UnweightError) as ei:
            uw.plan_load(path)
        assert ei.value.code == code, path.name
        assert uw.plan_count() == 1
    uw.plan_clear()
    uw.plan_load(p)
    assert uw.plan_lookup(4096, 14336, 16) == (uw.UW_PIPE_DIRECT, uw.UW_KERNEL_SKINNY, 1)
    uw.plan_clear()


@pytest.mark.parametrize("lengths", [
    list(range(1, 15)) + [15, 15],                                  # the one 16-symbol shape reaching 15 bits
    [2, 2, 2] + list(range(3, 14)) + [14, 14],
    list(range(1, 13)) + [14, 14, 14, 14],
    list(range(1, 11)) + [12, 12, 13, 13, 13, 13],
])
def test_long_codewords_fill_the_top_of_the_decode_table(lengths):
    """The decoders keep only the last 64 entries of the single-symbol table
    in LDS for windows whose first codeword is longer than the 12-bit
    multi-symbol index.  That relies on canonical codes: the longest codes
    are numerically the largest, so such windows are the top lmax-bit values,
    at most 16 codes x 2^(15-13) = 64 of them.  Checked here on the tables
    the host builds, for 16-symbol codes with 13-15-bit codewords."""
    assert len(lengths) == 16 and sum(2.0 ** -l for l in lengths) == 1.0
    # exponent 100+s repeated 2^(15 - len) times: dyadic counts, for which an
    # optimal code has these lengths
    counts = [2 ** (15 - l) for l in lengths]
    exps = np.repeat(np.arange(100, 116, dtype=np.uint16), counts)
    w = ((exps << 7) | (np.arange(exps.size, dtype=np.uint16) & 0x7F)).astype(np.uint16)
    w = np.random.default_rng(5).permutation(w).reshape(-1, 256)
    b = uw.compress(w)
    L = b.info().lmax
    assert L == max(lengths) and sorted(b.info().lengths[:16]) == sorted(lengths)
    mlut = np.frombuffer(b.section("mlut"), np.uint32)
    v = np.arange(1 << L)
    long_first = mlut[v >> (L - 12)] == 0                        # first codeword over 12 bits
    assert long_first.any()
    lo = int(v[long_first].min())
    assert lo >= (1 << L) - 64
    assert long_first[lo:].all()                                 # one run up to the top


def test_version_one_images_are_rejected():
    """Format version 2 pads coded groups to 4 bits and stores one-byte group
    lengths; an image of the 16-bit-length version 1 is refused, not misread."""
    w, _ = workloads.small_matrix()
    data = bytearray(uw.compress(w).serialize())
    assert data[:4] == b"UWF2"
    data[:4] = b"UWF1"
    with pytest.raises(uw.UnweightError, match="version 1") as ei:
        uw.Blob.deserialize(bytes(data))
    assert ei.value.code == -3          # UW_EFORMAT
