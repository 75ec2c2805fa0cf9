"""Oracle codec: the compressed at-rest format and its three decode modes.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What the Unweight page fixes (Cloudflare, "Unweight: how we compressed an LLM
22% without sacrificing quality"):
  * "How to compress model weights effectively": a bf16 value is 1 sign bit,
    8 exponent bits and 7 mantissa bits.  Sign and mantissa are kept raw; only
    the exponent byte is entropy coded with a Huffman code.  The 16 most
    frequent exponents form a palette; a 64-element row that holds any
    exponent outside that palette is stored as-is, so the hot loop checks once
    per row and never per element.
  * "Four ways to use compressed weights": decoders produce either the full
    bf16 matrix, only the exponent bytes (half the write-back), or 4-bit
    palette indices (a quarter); the direct-palette form is that 4-bit form
    produced once at load time.

Readings taken where the page is silent:
  * a "64-element row" is 64 consecutive elements along a storage row
    (in-features), so C % 64 == 0 is required; it is called a *group*;
  * the palette is per matrix, ordered by (descending count, ascending
    exponent); the palette index is that rank;
  * the Huffman alphabet is the palette index; frequencies are counted over
    the non-verbatim groups only, which are the only ones coded;
  * Huffman tree: min-heap keyed (weight, id), leaf id = symbol index,
    internal ids 16, 17, ... in creation order; a lone coded symbol gets
    length 1; codes are canonical, assigned in (length, symbol) order, and
    written MSB-first;
  * the stream is cut into tiles of 64 groups that start on a byte boundary;
    each coded group's bits are followed by zero bits up to a multiple of 4
    bits, and that padded length, in 4-bit units, is stored in one byte per
    group (at most 64 * 15 / 4 = 240) so that 64 lanes can find their start
    bits by a prefix sum; tile byte offsets and verbatim counts before each
    tile are u32 tables; a u64 bitmap per tile flags verbatim groups, whose
    64 raw exponent bytes go to a separate array;
  * the sign/mantissa byte is (sign << 7) | mantissa;
  * the 4-bit form puts element i in byte i // 2, low nibble for even i, and
    holds 0 for every element of a verbatim group.
"""
from __future__ import annotations

import heapq
from dataclasses import dataclass, field

import numpy as np

GROUP = 64          # elements per verbatim decision ("64-element row")
TILE = 64           # groups per independently addressable stream tile
PALETTE_MAX = 16    # palette size: 4-bit indices
GLEN_UNIT = 4       # bits: coded groups are padded to, and measured in, this unit


# ------------------------------------------------------------------ field split
def split_fields(bits: np.ndarray):
    """bf16 bits -> (exponent byte, sign/mantissa byte).

    exponent = bits 14..7; sign/mantissa = sign in bit 7, mantissa in bits 6..0.
    """
    b = np.asarray(bits, dtype=np.uint16)
    e = ((b >> 7) & 0xFF).astype(np.uint8)
    sm = (((b >> 8) & 0x80) | (b & 0x7F)).astype(np.uint8)
    return e, sm


def join_fields(e: np.ndarray, sm: np.ndarray) -> np.ndarray:
    """Inverse of split_fields."""
    e16 = np.asarray(e).astype(np.uint16)
    s16 = np.asarray(sm).astype(np.uint16)
    return (((s16 & 0x80) << 8) | (e16 << 7) | (s16 & 0x7F)).astype(np.uint16)


# ------------------------------------------------------------- palette, flags
def exponent_histogram(e: np.ndarray) -> np.ndarray:
    """Count of each of the 256 exponent values."""
    return np.bincount(np.asarray(e, dtype=np.uint8).ravel(), minlength=256).astype(np.int64)


def top16_palette(hist: np.ndarray) -> np.ndarray:
    """The (at most) 16 most frequent exponents, by (-count, exponent)."""
    present = [E for E in range(256) if hist[E] > 0]
    present.sort(key=lambda E: (-int(hist[E]), E))
    return np.array(present[:PALETTE_MAX], dtype=np.uint8)


def palette_index_table(palette: np.ndarray) -> np.ndarray:
    """256-entry map exponent -> palette index, -1 when out of palette."""
    idx = np.full(256, -1, dtype=np.int64)
    for s, E in enumerate(palette):
        idx[int(E)] = s
    return idx


def verbatim_flags(e: np.ndarray, palette: np.ndarray) -> np.ndarray:
    """True for every 64-element group holding an exponent outside the palette."""
    idx = palette_index_table(palette)[np.asarray(e).ravel()]
    return (idx.reshape(-1, GROUP) < 0).any(axis=1)


def symbol_frequencies(e: np.ndarray, palette: np.ndarray, vflag: np.ndarray) -> np.ndarray:
    """Occurrences of each palette index over the non-verbatim groups."""
    sym = palette_index_table(palette)[np.asarray(e).ravel()].reshape(-1, GROUP)
    coded = sym[~vflag].ravel()
    return np.bincount(coded, minlength=PALETTE_MAX).astype(np.int64)[:PALETTE_MAX]


# -------------------------------------------------------------------- Huffman
def huffman_code_lengths(freq) -> np.ndarray:
    """Textbook Huffman code lengths for up to 16 symbols.

    Merge the two lightest nodes until one remains; a symbol's length is its
    leaf depth.  Ties are broken by the heap key (weight, id): leaves have
    id = symbol, merged nodes get ids 16, 17, ... in creation order.
    Symbols of zero frequency get length 0 (no codeword); a single coded
    symbol gets length 1.
    """
    freq = [int(f) for f in freq]
    n = len(freq)
    lengths = np.zeros(n, dtype=np.int64)
    live = [s for s in range(n) if freq[s] > 0]
    if not live:
        return lengths
    if len(live) == 1:
        lengths[live[0]] = 1
        return lengths
    heap = [(freq[s], s) for s in live]
    heapq.heapify(heap)
    parent = {}
    next_id = PALETTE_MAX
    while len(heap) > 1:
        w1, a = heapq.heappop(heap)
        w2, b = heapq.heappop(heap)
        parent[a] = next_id
        parent[b] = next_id
        heapq.heappush(heap, (w1 + w2, next_id))
        next_id += 1
    for s in live:
        depth, node = 0, s
        while node in parent:
            node = parent[node]
            depth += 1
        lengths[s] = depth
    return lengths


def canonical_codes(lengths) -> np.ndarray:
    """Canonical codewords: symbols ordered by (length, symbol); each next code
    is the previous plus one, shifted left by the growth in length."""
    lengths = [int(x) for x in lengths]
    order = sorted((L, s) for s, L in enumerate(lengths) if L > 0)
    codes = np.zeros(len(lengths), dtype=np.int64)
    code, prev = 0, None
    for L, s in order:
        if prev is not None:
            code = (code + 1) << (L - prev)
        codes[s] = code
        prev = L
    return codes


# ------------------------------------------------------------ the at-rest form
@dataclass
class Compressed:
    """One compressed matrix.  Section dtypes are the on-disk ones."""
    R: int
    C: int
    palette: np.ndarray          # uint8[P]
    lengths: np.ndarray          # int64[16], 0 = no codeword
    codes: np.ndarray            # int64[16]
    sm: np.ndarray               # uint8[N]   sign/mantissa plane
    stream: np.ndarray           # uint8[S]   Huffman stream, tiles byte aligned
    glen: np.ndarray             # uint8[G]   padded coded bits of each group / 4 (0 if verbatim)
    tile_off: np.ndarray         # uint32[T+1] byte offset of each tile's stream
    tile_vbase: np.ndarray       # uint32[T+1] verbatim groups before each tile
    vexp: np.ndarray             # uint8[64 V] raw exponents of verbatim groups
    bitmap: np.ndarray           # uint64[T]  bit g%64 of word g//64 = verbatim
    nib: np.ndarray              # uint8[N/2] palette indices, 2 per byte
    hist: np.ndarray = field(repr=False, default=None)
    freq: np.ndarray = field(repr=False, default=None)
    vflag: np.ndarray = field(repr=False, default=None)

    @property
    def N(self):
        return self.R * self.C

    @property
    def G(self):
        return self.N // GROUP

    @property
    def T(self):
        return (self.G + TILE - 1) // TILE

    @property
    def V(self):
        return int(self.vexp.size // GROUP)

    @property
    def P(self):
        return int(self.palette.size)

    @property
    def lmax(self):
        return int(max(self.lengths.max(initial=0), 0))


def _check_shape(bits):
    b = np.asarray(bits, dtype=np.uint16)
    if b.ndim != 2:
        raise ValueError("weights must be a 2-D [rows, cols] array of bf16 bits")
    R, C = b.shape
    if C % GROUP != 0:
        raise ValueError("cols must be a multiple of 64")
    return b, R, C


def element_symbols(e: np.ndarray, palette: np.ndarray, vflag: np.ndarray) -> np.ndarray:
    """Palette index of every element; 0 for elements of verbatim groups."""
    sym = palette_index_table(palette)[np.asarray(e).ravel()].reshape(-1, GROUP)
    sym[vflag] = 0
    return sym.ravel()


def pack_nibbles(sym: np.ndarray) -> np.ndarray:
    """Two 4-bit indices per byte: element 2j low nibble, 2j+1 high nibble."""
    s = np.asarray(sym, dtype=np.uint8)
    return (s[0::2] | (s[1::2] << 4)).astype(np.uint8)


def encode(bits) -> Compressed:
    """Compress a [R, C] bf16 matrix (C % 64 == 0) into the at-rest form."""
    b, R, C = _check_shape(bits)
    N = R * C
    G = N // GROUP
    T = (G + TILE - 1) // TILE
    e, sm = split_fields(b.ravel())
    hist = exponent_histogram(e)
    palette = top16_palette(hist)
    vflag = verbatim_flags(e, palette) if G else np.zeros(0, dtype=bool)
    freq = symbol_frequencies(e, palette, vflag) if G else np.zeros(PALETTE_MAX, np.int64)
    lengths = huffman_code_lengths(np.pad(freq, (0, PALETTE_MAX - freq.size)))
    codes = canonical_codes(lengths)
    sym = element_symbols(e, palette, vflag) if G else np.zeros(0, np.int64)

    # per-element code length; verbatim groups contribute nothing
    L = lengths[sym].reshape(-1, GROUP) if G else np.zeros((0, GROUP), np.int64)
    L = np.where(vflag[:, None], 0, L)
    gbits = L.sum(axis=1)                                   # code bits of each group
    gpad = -(-gbits // GLEN_UNIT) * GLEN_UNIT               # padded to a 4-bit boundary
    # tiles start on byte boundaries
    tile_bits = np.add.reduceat(gpad, np.arange(0, G, TILE)) if G else np.zeros(0, np.int64)
    tile_bytes = (tile_bits + 7) // 8
    tile_off = np.concatenate([[0], np.cumsum(tile_bytes)]).astype(np.int64)
    # start bit of every element: its tile's first bit + the padded lengths of
    # the groups before it in the tile + the code bits before it in its group
    Lf = L.ravel()
    tile_of_elem = np.arange(N) // (GROUP * TILE)
    g_excl = np.cumsum(gpad) - gpad
    g_in_tile = g_excl - g_excl[(np.arange(G) // TILE) * TILE] if G else np.zeros(0, np.int64)
    in_group = (np.cumsum(L, axis=1) - L).ravel()
    start = tile_off[tile_of_elem] * 8 + np.repeat(g_in_tile, GROUP) + in_group
    total_bits = int(tile_off[-1]) * 8
    bitv = np.zeros(total_bits, dtype=np.uint8)
    cf = codes[sym] if N else np.zeros(0, np.int64)
    for k in range(int(lengths.max(initial=0))):
        sel = Lf > k
        bitv[start[sel] + k] = (cf[sel] >> (Lf[sel] - 1 - k)) & 1
    stream = np.packbits(bitv) if total_bits else np.zeros(0, np.uint8)

    vper_tile = np.add.reduceat(vflag.astype(np.int64), np.arange(0, G, TILE)) if G else np.zeros(0, np.int64)
    tile_vbase = np.concatenate([[0], np.cumsum(vper_tile)]).astype(np.int64)
    vexp = e.reshape(-1, GROUP)[vflag].ravel() if G else np.zeros(0, np.uint8)
    bitmap = np.zeros(T, dtype=np.uint64)
    for g in np.nonzero(vflag)[0]:
        bitmap[g // TILE] |= np.uint64(1) << np.uint64(g % TILE)
    nib = pack_nibbles(sym) if N else np.zeros(0, np.uint8)

    return Compressed(
        R=R, C=C, palette=palette, lengths=lengths, codes=codes,
        sm=sm.astype(np.uint8), stream=stream.astype(np.uint8),
        glen=(gpad // GLEN_UNIT).astype(np.uint8), tile_off=tile_off.astype(np.uint32),
        tile_vbase=tile_vbase.astype(np.uint32), vexp=vexp.astype(np.uint8),
        bitmap=bitmap, nib=nib, hist=hist, freq=freq, vflag=vflag)


def encode_stream_bitstring(comp: Compressed, e: np.ndarray) -> list:
    """Per-tile stream as '0'/'1' strings, one symbol at a time (small inputs).

    A second, loop-by-loop statement of the tile stream used to cross-check
    ``encode`` on small matrices.
    """
    sym_of = palette_index_table(comp.palette)
    tiles = []
    for t in range(comp.T):
        s = []
        for g in range(t * TILE, min((t + 1) * TILE, comp.G)):
            if comp.vflag[g]:
                continue
            gs = []
            for i in range(g * GROUP, (g + 1) * GROUP):
                k = sym_of[int(e[i])]
                L = int(comp.lengths[k])
                gs.append(format(int(comp.codes[k]), f"0{L}b"))
            gbits = "".join(gs)
            s.append(gbits + "0" * (-len(gbits) % GLEN_UNIT))
        bits = "".join(s)
        bits += "0" * (-len(bits) % 8)
        tiles.append(bits)
    return tiles


# ------------------------------------------------------------------- decoding
MODES = ("full", "exp", "pal")


def group_flags(comp: Compressed) -> np.ndarray:
    """Verbatim flag of every group, read back from the per-tile bitmap."""
    g = np.arange(comp.G)
    word = comp.bitmap[g // TILE] if comp.G else np.zeros(0, np.uint64)
    return ((word >> (g % TILE).astype(np.uint64)) & np.uint64(1)).astype(bool)


def _verbatim_slot(comp: Compressed, g: int) -> int:
    """Rank of verbatim group g among all verbatim groups, from the tile base
    count plus the flagged groups before it in its tile's bitmap word."""
    t, j = divmod(g, TILE)
    below = int(comp.bitmap[t]) & ((1 << j) - 1)
    return int(comp.tile_vbase[t]) + bin(below).count("1")


def _assemble(comp: Compressed, exps: np.ndarray, syms: np.ndarray, mode: str):
    if mode == "full":
        return join_fields(exps, comp.sm).reshape(comp.R, comp.C)
    if mode == "exp":
        return exps.astype(np.uint8).reshape(comp.R, comp.C)
    if mode == "pal":
        return pack_nibbles(syms)
    raise ValueError(mode)


def decode_sequential(comp: Compressed, mode: str = "full"):
    """Bit-by-bit decoder: walks each tile's stream from its first byte and
    matches growing bit strings against the codeword table.  Uses neither the
    per-group lengths nor a lookup table; meant for small matrices."""
    table = {}
    for s in range(PALETTE_MAX):
        L = int(comp.lengths[s])
        if L:
            table[(L, int(comp.codes[s]))] = s
    stream = comp.stream
    exps = np.zeros(comp.N, dtype=np.uint8)
    syms = np.zeros(comp.N, dtype=np.uint8)
    for t in range(comp.T):
        pos = int(comp.tile_off[t]) * 8
        for g in range(t * TILE, min((t + 1) * TILE, comp.G)):
            base = g * GROUP
            if (int(comp.bitmap[t]) >> (g % TILE)) & 1:
                v = _verbatim_slot(comp, g)
                exps[base:base + GROUP] = comp.vexp[v * GROUP:(v + 1) * GROUP]
                continue
            for i in range(GROUP):
                code, L = 0, 0
                while True:
                    bit = (int(stream[pos >> 3]) >> (7 - (pos & 7))) & 1
                    pos += 1
                    code = (code << 1) | bit
                    L += 1
                    if (L, code) in table:
                        s = table[(L, code)]
                        break
                    if L > 16:
                        raise ValueError("invalid code in stream")
                syms[base + i] = s
                exps[base + i] = comp.palette[s]
            pos += -pos % GLEN_UNIT          # the group's zero padding (tiles start byte aligned)
    return _assemble(comp, exps, syms, mode)


def decode_lut(lengths, codes):
    """Table indexed by the next lmax stream bits -> (symbol, code length)."""
    lmax = int(max(lengths.max(initial=0), 0))
    sym = np.zeros(1 << lmax, dtype=np.int64)
    ln = np.zeros(1 << lmax, dtype=np.int64)
    for s in range(PALETTE_MAX):
        L = int(lengths[s])
        if L:
            lo = int(codes[s]) << (lmax - L)
            sym[lo:lo + (1 << (lmax - L))] = s
            ln[lo:lo + (1 << (lmax - L))] = L
    return sym, ln, lmax


def group_start_bits(comp: Compressed) -> np.ndarray:
    """First stream bit of every group: its tile's byte offset times 8 plus the
    padded lengths of the groups before it in the same tile."""
    G = comp.G
    gl = comp.glen.astype(np.int64) * GLEN_UNIT
    tile_of = np.arange(G) // TILE
    incl = np.cumsum(gl)
    tile_first = np.concatenate([[0], incl])[np.arange(0, G, TILE)] if G else np.zeros(0, np.int64)
    return comp.tile_off.astype(np.int64)[tile_of] * 8 + (incl - gl) - tile_first[tile_of]


def decode_parallel(comp: Compressed, mode: str = "full"):
    """Group-parallel decoder: every group starts at its own bit (from the
    per-group lengths) and all groups advance one symbol per step through a
    2^lmax lookup table.  Same result as ``decode_sequential``."""
    N, G = comp.N, comp.G
    exps = np.zeros(N, dtype=np.uint8)
    syms = np.zeros(N, dtype=np.uint8)
    if G == 0:
        return _assemble(comp, exps, syms, mode)
    vflag = group_flags(comp)
    coded = np.nonzero(~vflag)[0]
    if coded.size:
        lsym, llen, lmax = decode_lut(comp.lengths, comp.codes)
        s = np.concatenate([comp.stream, np.zeros(4, np.uint8)]).astype(np.int64)
        pos = group_start_bits(comp)[coded]
        out = np.zeros((coded.size, GROUP), dtype=np.int64)
        for i in range(GROUP):
            byte = pos >> 3
            window = (s[byte] << 16) | (s[byte + 1] << 8) | s[byte + 2]
            peek = (window >> (24 - lmax - (pos & 7))) & ((1 << lmax) - 1)
            out[:, i] = lsym[peek]
            pos = pos + llen[peek]
        sy = syms.reshape(G, GROUP)
        ex = exps.reshape(G, GROUP)
        sy[coded] = out
        ex[coded] = comp.palette[out]
    for g in np.nonzero(vflag)[0]:
        v = _verbatim_slot(comp, int(g))
        exps[g * GROUP:(g + 1) * GROUP] = comp.vexp[v * GROUP:(v + 1) * GROUP]
    return _assemble(comp, exps, syms, mode)


def reconstruct_from_palette(comp: Compressed) -> np.ndarray:
    """bf16 bits rebuilt from the direct-palette form (4-bit indices + sign/
    mantissa + verbatim exponents), as the reconstructive matmul does on chip."""
    N, G = comp.N, comp.G
    lo = comp.nib & 0x0F
    hi = comp.nib >> 4
    idx = np.empty(N, dtype=np.uint8)
    idx[0::2] = lo
    idx[1::2] = hi
    pal = np.zeros(PALETTE_MAX, dtype=np.uint8)
    pal[:comp.P] = comp.palette
    exps = pal[idx]
    for g in np.nonzero(group_flags(comp))[0]:
        v = _verbatim_slot(comp, int(g))
        exps[g * GROUP:(g + 1) * GROUP] = comp.vexp[v * GROUP:(v + 1) * GROUP]
    return join_fields(exps, comp.sm).reshape(comp.R, comp.C)


def reconstruct_from_exponents(e: np.ndarray, sm: np.ndarray, R: int, C: int) -> np.ndarray:
    """bf16 bits rebuilt from a decoded exponent plane and the sign/mantissa plane."""
    return join_fields(np.asarray(e).ravel(), np.asarray(sm).ravel()).reshape(R, C)


# ---------------------------------------------------------------- accounting
HEADER_BYTES = 256

SECTION_NAMES = ("sm", "stream", "glen", "tile_off", "tile_vbase", "vexp", "bitmap", "nib")


def section_bytes(comp: Compressed) -> dict:
    return {n: int(getattr(comp, n).nbytes) for n in SECTION_NAMES}


def huffman_form_bytes(comp: Compressed) -> int:
    """At-rest bytes of the Huffman form (everything but the 4-bit indices)."""
    sb = section_bytes(comp)
    return HEADER_BYTES + sum(v for k, v in sb.items() if k != "nib")


def palette_form_bytes(comp: Compressed) -> int:
    """At-rest bytes of the direct-palette form the fused matmul reads."""
    sb = section_bytes(comp)
    return HEADER_BYTES + sb["sm"] + sb["nib"] + sb["vexp"] + sb["bitmap"] + sb["tile_vbase"]
