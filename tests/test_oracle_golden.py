"""Oracle codec vs hand-worked examples (tests/golden/codec_worked_examples.json).

Each example was worked out by hand from the format readings of the Unweight
page ("How to compress model weights effectively": raw sign/mantissa,
Huffman-coded exponent over a top-16 palette, verbatim 64-element rows); the
derivation is written out in the fixture.  A dropped term, a flipped bit
order, a wrong canonical assignment or a misplaced nibble changes bytes here.
"""
import json
import os

import numpy as np
import pytest

from oracle import codec

pytestmark = pytest.mark.filterwarnings("ignore")


def _load(golden_dir):
    with open(os.path.join(golden_dir, "codec_worked_examples.json")) as f:
        return json.load(f)


@pytest.fixture(scope="module")
def examples(golden_dir):
    return _load(golden_dir)


NAMES = ["three_symbols", "verbatim_group", "single_exponent", "group_padding"]


def _matrix(ex):
    vals = np.array([int(h, 16) for h in ex["bf16_hex"]], dtype=np.uint16)
    return vals.reshape(ex["rows"], ex["cols"])


@pytest.mark.parametrize("name", NAMES)
def test_sections_match_hand_derivation(examples, name):
    ex = examples[name]
    w = _matrix(ex)
    c = codec.encode(w)
    assert list(c.palette) == ex["palette"]
    assert list(c.lengths) == ex["lengths"]
    coded = [s for s, L in enumerate(ex["lengths"]) if L]
    assert [int(c.codes[s]) for s in coded] == [ex["codes"][s] for s in coded]
    assert list(c.glen) == ex["glen"]
    assert c.stream.tobytes().hex() == ex["stream_hex"]
    assert list(c.tile_off) == ex["tile_off"]
    assert list(c.tile_vbase) == ex["tile_vbase"]
    assert c.vexp.tobytes().hex() == ex["vexp_hex"]
    assert [int(b) for b in c.bitmap] == ex["bitmap"]
    assert c.nib.tobytes().hex() == ex["nib_hex"]
    assert list(c.freq[:16]) == ex["freq"]
    nz = {str(E): int(n) for E, n in enumerate(c.hist) if n}
    assert nz == ex["hist_nonzero"]
    # sign/mantissa plane: sign bit to bit 7, mantissa kept in bits 6..0
    sm_expect = [((int(h, 16) >> 8) & 0x80) | (int(h, 16) & 0x7F) for h in ex["bf16_hex"]]
    assert list(c.sm) == sm_expect


@pytest.mark.parametrize("name", NAMES)
@pytest.mark.parametrize("decoder", ["sequential", "parallel"])
def test_worked_examples_decode(examples, name, decoder):
    ex = examples[name]
    w = _matrix(ex)
    c = codec.encode(w)
    dec = getattr(codec, "decode_" + decoder)
    assert np.array_equal(dec(c, "full"), w)
    exps = ((w >> 7) & 0xFF).astype(np.uint8)
    assert np.array_equal(dec(c, "exp"), exps)
    assert dec(c, "pal").tobytes().hex() == ex["nib_hex"]


def test_bitstring_encoder_matches_on_examples(examples):
    for name in NAMES:
        ex = examples[name]
        w = _matrix(ex)
        c = codec.encode(w)
        e, _ = codec.split_fields(w.ravel())
        tiles = codec.encode_stream_bitstring(c, e)
        bits = "".join(tiles)
        got = bytes(int(bits[i:i + 8], 2) for i in range(0, len(bits), 8)).hex()
        assert got == ex["stream_hex"]
