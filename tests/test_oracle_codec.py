"""Pins for the oracle codec beyond the hand-worked examples.

* lossless: decode(encode(W)) == W bit for bit (the page reports bit-identical
  outputs), through both decoders and the direct-palette reconstruction, on
  the workloads' distributions and on edge cases (one exponent, > 16 spread
  exponents, all-verbatim, +-0 / subnormal / Inf / NaN payloads, partial
  last tile, empty);
* the sign/mantissa plane is the input with the exponent removed;
* the palette is the top 16 exponents by count and covers >= 99% (page:
  "How to compress model weights effectively");
* verbatim groups are exactly those holding an out-of-palette exponent, at
  the rate 1 - (1 - q)^64 that independent outliers predict;
* the exponent histogram matches the closed form for a rounded normal;
* section sizes follow the closed-form accounting, and the three decode
  modes write 2 : 1 : 0.5 bytes per weight ("Four ways to use compressed
  weights": exponent-only halves and palette quarters the write-back).
"""
import numpy as np
import pytest
from scipy import stats

from oracle import codec
import workloads


def _roundtrip(w, sequential=False):
    c = codec.encode(w)
    assert np.array_equal(codec.decode_parallel(c, "full"), w)
    if sequential:
        assert np.array_equal(codec.decode_sequential(c, "full"), w)
    assert np.array_equal(codec.reconstruct_from_palette(c), w)
    exps = ((w >> 7) & 0xFF).astype(np.uint8)
    assert np.array_equal(codec.decode_parallel(c, "exp"), exps)
    assert np.array_equal(codec.reconstruct_from_exponents(exps, c.sm, *w.shape), w)
    assert np.array_equal(codec.decode_parallel(c, "pal"), c.nib)
    return c


def test_roundtrip_small_workload_both_decoders():
    w, _ = workloads.small_matrix()
    c = _roundtrip(w, sequential=True)
    assert np.array_equal(codec.decode_sequential(c, "pal"), c.nib)


@pytest.mark.parametrize("wl,m,shape", [(2, 0, (512, 4096)), (2, 2, (256, 14336)),
                                         (4, 1, (512, 4096)), (5, 2, (128, 14336))])
def test_roundtrip_layer_distributions(wl, m, shape):
    w = workloads.layer_weight(wl, 1, m, shape=shape)
    _roundtrip(w)


def test_bitstring_encoder_agrees_on_small_workload():
    w, _ = workloads.small_matrix()
    c = codec.encode(w)
    e, _ = codec.split_fields(w.ravel())
    tiles = codec.encode_stream_bitstring(c, e)
    for t, bits in enumerate(tiles):
        got = bytes(int(bits[i:i + 8], 2) for i in range(0, len(bits), 8))
        assert got == c.stream[c.tile_off[t]:c.tile_off[t + 1]].tobytes()


def _bits(sign, e, m):
    return ((np.asarray(sign, np.uint16) << 15) | (np.asarray(e, np.uint16) << 7)
            | np.asarray(m, np.uint16)).astype(np.uint16)


def test_edge_single_exponent():
    rng = np.random.default_rng(1)
    w = _bits(rng.integers(0, 2, (7, 128)), 120, rng.integers(0, 128, (7, 128)))
    c = _roundtrip(w, sequential=True)
    assert c.P == 1 and c.V == 0 and c.lengths[0] == 1 and c.lengths[1:].sum() == 0


def test_edge_exactly_16_exponents_no_verbatim():
    rng = np.random.default_rng(2)
    w = _bits(rng.integers(0, 2, (16, 256)), rng.integers(100, 116, (16, 256)),
              rng.integers(0, 128, (16, 256)))
    c = _roundtrip(w, sequential=True)
    assert c.P == 16 and c.V == 0


def test_edge_spread_exponents_mostly_verbatim():
    rng = np.random.default_rng(3)
    w = _bits(rng.integers(0, 2, (16, 256)), rng.integers(90, 122, (16, 256)),
              rng.integers(0, 128, (16, 256)))
    c = _roundtrip(w, sequential=True)
    assert c.V > 0.9 * c.G


def test_edge_uniform_random_bits_all_verbatim():
    w = workloads.random_bf16_bits(4, 64 * 200).reshape(100, 128)
    c = _roundtrip(w, sequential=True)
    assert c.V == c.G
    assert c.stream.size == 0 and int(c.tile_off[-1]) == 0
    assert not c.nib.any()


def test_edge_special_values_and_nan_payloads():
    rng = np.random.default_rng(5)
    w = workloads.gaussian_weights(rng, 40, 192, 0.02)
    specials = np.array([0x0000, 0x8000, 0x0001, 0x807F, 0x0040, 0x7F80, 0xFF80,
                         0x7FC0, 0x7F81, 0xFFFF, 0x7FA5, 0x0080, 0x7F7F], np.uint16)
    flat = w.ravel()
    pos = rng.choice(flat.size, size=specials.size * 3, replace=False)
    flat[pos] = np.tile(specials, 3)
    _roundtrip(w, sequential=True)


@pytest.mark.parametrize("R,C", [(3, 192), (65, 64), (1, 64 * 64 + 64), (5, 64 * 13)])
def test_edge_partial_last_tile(R, C):
    w = workloads.gaussian_weights(np.random.default_rng(R * C), R, C, 0.02, 0.01, 1.0)
    c = _roundtrip(w, sequential=True)
    assert c.T == (R * C // 64 + 63) // 64


def test_edge_empty():
    w = np.zeros((0, 128), np.uint16)
    c = codec.encode(w)
    assert c.G == 0 and c.T == 0 and c.stream.size == 0
    assert list(c.tile_off) == [0] and list(c.tile_vbase) == [0]
    assert codec.decode_parallel(c, "full").shape == (0, 128)


def test_rejects_cols_not_multiple_of_64():
    with pytest.raises(ValueError):
        codec.encode(np.zeros((2, 100), np.uint16))


# ------------------------------------------------------------------ properties
@pytest.fixture(scope="module")
def small():
    w, _ = workloads.small_matrix()
    return w, codec.encode(w)


def test_sm_plane_is_input_without_exponent(small):
    w, c = small
    flat = w.ravel().astype(np.uint32)
    assert np.array_equal(c.sm.astype(np.uint32), ((flat & 0x8000) >> 8) | (flat & 0x7F))


def test_palette_is_top16_and_covers_99pct(small):
    w, c = small
    e = ((w.ravel() >> 7) & 0xFF)
    counts = np.bincount(e, minlength=256)
    assert np.array_equal(counts, c.hist)
    in_pal = set(int(x) for x in c.palette)
    least_in = min(counts[E] for E in in_pal)
    assert all(counts[E] <= least_in for E in range(256) if E not in in_pal)
    cover = sum(counts[E] for E in in_pal) / e.size
    assert cover >= 0.99


@pytest.mark.parametrize("wl,m", [(2, 0), (4, 2), (5, 1)])
def test_palette_coverage_on_layer_distributions(wl, m):
    w = workloads.layer_weight(wl, 0, m, shape=(512, 4096) if m != 2 else (128, 14336))
    c = codec.encode(w)
    cover = c.hist[c.palette].sum() / w.size
    assert cover >= 0.99


def test_verbatim_groups_exactly_the_out_of_palette_ones(small):
    w, c = small
    e = ((w.ravel() >> 7) & 0xFF).reshape(-1, 64)
    pal = set(int(x) for x in c.palette)
    expect = np.array([any(int(x) not in pal for x in row) for row in e])
    assert np.array_equal(codec.group_flags(c), expect)
    # the verbatim exponents are those groups' exponent bytes, in group order
    assert np.array_equal(c.vexp.reshape(-1, 64), e[expect])
    # and the coded bit count of a verbatim group is zero
    assert not c.glen[expect].any()


def test_verbatim_rate_matches_independent_outliers(small):
    w, c = small
    q = 1.0 - c.hist[c.palette].sum() / w.size
    pred = 1.0 - (1.0 - q) ** 64
    obs = c.V / c.G
    sd = np.sqrt(pred * (1 - pred) / c.G)
    assert abs(obs - pred) < 5 * sd


def _exponent_prob(E, sigma):
    """P(bf16 exponent byte == E) for N(0, sigma) rounded to nearest bf16.

    A normal bf16 with exponent byte E spans [2^(E-127), 2^(E-126)); values
    from half an ulp below 2^(E-127) round up into it and values from half an
    ulp below 2^(E-126) round up out of it: ulp = 2^(E-134).
    """
    lo = 2.0 ** (E - 127) * (1 - 2.0 ** -9)
    hi = 2.0 ** (E - 126) * (1 - 2.0 ** -9)
    return 2 * (stats.norm.cdf(hi / sigma) - stats.norm.cdf(lo / sigma))


@pytest.mark.parametrize("which", ["small", "layer2"])
def test_histogram_matches_closed_form(which):
    if which == "small":
        w, _ = workloads.small_matrix()
        sigma, p, s = 0.02, 1e-3, 1.0
    else:
        w = workloads.layer_weight(2, 0, 0, shape=(1024, 4096))
        sigma, p, s = 0.02, 5e-4, 0.5
    hist = codec.exponent_histogram(((w >> 7) & 0xFF).ravel())
    n = w.size
    expected = np.array([(1 - p) * _exponent_prob(E, sigma) + p * _exponent_prob(E, s)
                         for E in range(256)]) * n
    keep = expected >= 20
    # lump the sparse tails into one bin
    obs = np.append(hist[keep], hist[~keep].sum())
    exp_ = np.append(expected[keep], n - expected[keep].sum())
    chi2 = ((obs - exp_) ** 2 / exp_).sum()
    dof = obs.size - 1
    assert chi2 < stats.chi2.ppf(1 - 1e-4, dof), (chi2, dof)


def test_size_accounting_closed_form(small):
    w, c = small
    N, G, T, V = c.N, c.G, c.T, c.V
    # stream bytes from the code side: each coded group's code bits (its
    # exponents' code lengths summed) rounded up to a multiple of 4, per tile
    # rounded up to whole bytes
    e = ((w.ravel() >> 7) & 0xFF).reshape(-1, 64)
    sym_of = {int(E): s for s, E in enumerate(c.palette)}
    vf = codec.group_flags(c)
    gbits = np.array([0 if vf[g] else sum(int(c.lengths[sym_of[int(x)]]) for x in e[g]) for g in range(G)])
    assert int(gbits.sum()) == int((c.freq * c.lengths).sum())
    gpad = (gbits + 3) // 4 * 4
    assert np.array_equal(c.glen.astype(np.int64) * 4, gpad)
    tile_bits = [int(gpad[t * 64:(t + 1) * 64].sum()) for t in range(T)]
    stream_bytes = sum((b + 7) // 8 for b in tile_bits)
    # GLEN is one byte per group
    expect = (codec.HEADER_BYTES + N + stream_bytes + G + 64 * V + 8 * T + 2 * 4 * (T + 1))
    assert codec.huffman_form_bytes(c) == expect
    assert codec.palette_form_bytes(c) == codec.HEADER_BYTES + N + N // 2 + 64 * V + 8 * T + 4 * (T + 1)


def test_decode_mode_output_bytes_per_weight(small):
    w, c = small
    full = codec.decode_parallel(c, "full")
    exp_ = codec.decode_parallel(c, "exp")
    pal = codec.decode_parallel(c, "pal")
    assert full.nbytes == 2 * w.size
    assert exp_.nbytes == w.size
    assert pal.nbytes * 2 == w.size


def test_pal_mode_zero_on_verbatim_groups(small):
    w, c = small
    nib = codec.decode_parallel(c, "pal")
    idx = np.empty(c.N, np.uint8)
    idx[0::2], idx[1::2] = nib & 15, nib >> 4
    idx = idx.reshape(-1, 64)
    vf = codec.group_flags(c)
    assert not idx[vf].any()
    e = ((w.ravel() >> 7) & 0xFF).reshape(-1, 64)
    assert np.array_equal(c.palette[idx[~vf]], e[~vf])


def test_compression_ratio_near_page_figure(small):
    # the page reports about 30% smaller MLP weights; plausibility only
    w, c = small
    saved = 1 - codec.huffman_form_bytes(c) / (2 * w.size)
    assert 0.25 < saved < 0.36


def test_group_of_longest_codes_fills_the_length_byte():
    """Frequencies 32 * Fibonacci force a code 15 deep; a group made only of
    the two 15-bit codewords is 64 * 15 = 960 bits, already a multiple of 4,
    the largest group length: 240 in the one-byte GLEN.  It round-trips."""
    fib = [1, 1]
    while len(fib) < 16:
        fib.append(fib[-1] + fib[-2])
    counts = [32 * f for f in fib]                   # symbol k gets exponent 100 + k
    exps = np.repeat(np.arange(100, 116), counts)
    # the two rarest classes (32 each) first: one group of longest codes
    order = np.concatenate([np.nonzero(exps < 102)[0], np.nonzero(exps >= 102)[0]])
    exps = exps[order]
    pad = (-exps.size) % 64
    exps = np.concatenate([exps, np.full(pad, 115)])
    w = ((exps.astype(np.uint16) << 7) | (np.arange(exps.size) % 128).astype(np.uint16)).reshape(1, -1)
    c = codec.encode(w)
    assert int(c.lengths.max()) == 15
    rare = [s for s, E in enumerate(c.palette) if E in (100, 101)]
    assert all(int(c.lengths[s]) == 15 for s in rare)
    assert int(c.glen[0]) == 240 and int(c.glen.max()) == 240
    assert np.array_equal(codec.decode_parallel(c, "full"), w)
    assert np.array_equal(codec.decode_sequential(c, "full"), w)
