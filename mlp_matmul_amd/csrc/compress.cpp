// Host compressor for the lossless exponent codec, plus blob access,
// serialization and validation.
//
// Method: Cloudflare, "Unweight: how we compressed an LLM 22% without
// sacrificing quality", section "How to compress model weights effectively":
// sign and mantissa of each bf16 weight stay raw, the exponent byte is Huffman
// coded over the 16 most frequent exponents of the matrix, and a 64-element
// row holding any other exponent is kept verbatim so the decoder branches once
// per row.  The 4-bit palette form is the one "Four ways to use compressed
// weights" makes at load time for the direct-palette pipeline.
//
// Byte layout choices the page leaves open (palette order, Huffman tie-break,
// canonical order, bit order, 64-group byte-aligned tiles with per-group bit
// lengths, verbatim bitmap/base tables, nibble order) are the ones described
// in unweight.h; the compressor is deterministic, so a given matrix always
// produces the same bytes.
#include <algorithm>
#include <cstring>
#include <functional>
#include <new>
#include <queue>
#include <thread>
#include <utility>

#include "uw_internal.h"

namespace {

using uw::kGroup;
using uw::kTile;

int resolve_threads(int threads) {
    if (threads > 0) return threads;
    unsigned hc = std::thread::hardware_concurrency();
    return hc ? int(hc) : 1;
}

// Run f(begin, end) over [0, n) split into contiguous chunks, one per thread.
void parallel_for(int64_t n, int threads, const std::function<void(int64_t, int64_t, int)>& f) {
    if (n <= 0) return;
    int t = int(std::min<int64_t>(resolve_threads(threads), n));
    if (t <= 1) {
        f(0, n, 0);
        return;
    }
    std::vector<std::thread> pool;
    pool.reserve(t);
    for (int i = 0; i < t; ++i) {
        int64_t b = n * i / t, e = n * (i + 1) / t;
        pool.emplace_back([&f, b, e, i] { f(b, e, i); });
    }
    for (auto& th : pool) th.join();
}

// Textbook Huffman lengths: merge the two lightest nodes, keyed (weight, id);
// leaves have id = symbol, merged nodes ids 16, 17, ... in creation order.
void huffman_lengths(const uint64_t freq[16], uint8_t len[16]) {
    std::memset(len, 0, 16);
    int live[16], nlive = 0;
    for (int s = 0; s < 16; ++s)
        if (freq[s] > 0) live[nlive++] = s;
    if (nlive == 0) return;
    if (nlive == 1) {
        len[live[0]] = 1;
        return;
    }
    using Node = std::pair<uint64_t, int>;
    std::priority_queue<Node, std::vector<Node>, std::greater<Node>> heap;
    int parent[64];
    std::fill(parent, parent + 64, -1);
    for (int i = 0; i < nlive; ++i) heap.push({freq[live[i]], live[i]});
    int next = 16;
    while (heap.size() > 1) {
        Node a = heap.top();
        heap.pop();
        Node b = heap.top();
        heap.pop();
        parent[a.second] = next;
        parent[b.second] = next;
        heap.push({a.first + b.first, next});
        ++next;
    }
    for (int i = 0; i < nlive; ++i) {
        int d = 0, node = live[i];
        while (parent[node] >= 0) {
            node = parent[node];
            ++d;
        }
        len[live[i]] = uint8_t(d);
    }
}

}  // namespace

namespace uw {

void canonical_codes(const uint8_t lengths[16], uint16_t codes[16]) {
    std::memset(codes, 0, 16 * sizeof(uint16_t));
    std::pair<int, int> order[16];
    int n = 0;
    for (int s = 0; s < 16; ++s)
        if (lengths[s]) order[n++] = {lengths[s], s};
    std::sort(order, order + n);
    uint32_t code = 0;
    int prev = -1;
    for (int i = 0; i < n; ++i) {
        if (prev >= 0) code = (code + 1) << (order[i].first - prev);
        codes[order[i].second] = uint16_t(code);
        prev = order[i].first;
    }
}

void build_dlut(uw_blob& b) {
    int L = b.lmax;
    size_t n = size_t(1) << L;
    // entries no codeword reaches (possible only with one coded symbol)
    // decode as symbol 0 of length max(L, 1) so a corrupt stream still advances
    b.dlut.assign(std::max<size_t>(n, 2), uint8_t(std::max(L, 1)));
    for (int s = 0; s < 16; ++s) {
        int l = b.lengths[s];
        if (!l) continue;
        size_t lo = size_t(b.codes[s]) << (L - l);
        size_t cnt = size_t(1) << (L - l);
        for (size_t v = lo; v < lo + cnt; ++v) b.dlut[v] = uint8_t((s << 4) | l);
    }
    b.dlut.resize(n);
}

void build_mlut(uw_blob& b) {
    const int L = b.lmax;
    const uint32_t mask = (1u << kMlutBits) - 1;
    b.mlut.assign(size_t(1) << kMlutBits, 0u);
    if (L == 0) return;
    for (uint32_t v = 0; v <= mask; ++v) {
        // apply the decode table to the bits not yet used (zero filled past
        // the string's end) while the codeword it names ends inside the string
        uint32_t used = 0, n = 0, syms = 0;
        while (n < 4) {
            const uint32_t rest = (v << used) & mask;
            const uint32_t idx = L <= kMlutBits ? rest >> (kMlutBits - L) : rest << (L - kMlutBits);
            const uint32_t ent = b.dlut[idx], len = ent & 15u;
            if (len == 0 || used + len > uint32_t(kMlutBits)) break;
            syms |= (ent >> 4) << (16 + 4 * n);
            used += len;
            ++n;
        }
        b.mlut[v] = used | ((4 * n) << 8) | syms;
    }
}

void build_nibbles(uw_blob& b, const uint8_t* e, int threads) {
    int8_t idx_of[256];
    std::memset(idx_of, -1, sizeof(idx_of));
    for (int s = 0; s < b.P; ++s) idx_of[b.palette[s]] = int8_t(s);
    b.nib.assign(size_t(b.N / 2), 0);
    parallel_for(b.G, threads, [&](int64_t g0, int64_t g1, int) {
        for (int64_t g = g0; g < g1; ++g) {
            bool verb = (b.bitmap[g / kTile] >> (g % kTile)) & 1;
            uint8_t* out = b.nib.data() + g * (kGroup / 2);
            if (verb) continue;  // zeros
            const uint8_t* eg = e + g * kGroup;
            for (int j = 0; j < kGroup; j += 2)
                out[j / 2] = uint8_t(idx_of[eg[j]] | (idx_of[eg[j + 1]] << 4));
        }
    });
    b.has_nib = true;
}

}  // namespace uw

extern "C" {

int uw_version(void) { return (1 << 16) | 1; }

int uw_compress(const uint16_t* w, int64_t rows, int64_t cols, const uw_opts* opts, uw_blob** out) {
    uw::clear_error();
    if (!out) return uw::fail(UW_EINVAL, "uw_compress: out is NULL");
    *out = nullptr;
    if (rows < 0 || cols < 0) return uw::fail(UW_EINVAL, "uw_compress: negative size");
    if (cols % kGroup) return uw::fail(UW_EINVAL, "uw_compress: cols must be a multiple of 64");
    if (cols && rows > INT64_MAX / cols) return uw::fail(UW_EINVAL, "uw_compress: size overflow");
    int64_t N = rows * cols;
    if (N && !w) return uw::fail(UW_EINVAL, "uw_compress: w is NULL");
    int threads = opts ? opts->threads : 0;
    bool emit_pal = opts && opts->emit_palette;

    uw_blob* b = new (std::nothrow) uw_blob;
    if (!b) return uw::fail(UW_ENOMEM, "uw_compress: out of host memory");
    try {
        b->rows = rows;
        b->cols = cols;
        b->N = N;
        b->G = N / kGroup;
        b->T = (b->G + kTile - 1) / kTile;
        const int64_t G = b->G, T = b->T;
        int nt = int(std::min<int64_t>(resolve_threads(threads), std::max<int64_t>(T, 1)));

        // 1. field split and exponent histogram
        std::vector<uint8_t> e(static_cast<size_t>(N));
        b->sm.resize(size_t(N));
        std::vector<std::vector<uint64_t>> hist_t(nt, std::vector<uint64_t>(256, 0));
        parallel_for(T, nt, [&](int64_t t0, int64_t t1, int tid) {
            uint64_t* h = hist_t[tid].data();
            int64_t i0 = t0 * kTile * kGroup, i1 = std::min<int64_t>(N, t1 * kTile * kGroup);
            for (int64_t i = i0; i < i1; ++i) {
                uint16_t v = w[i];
                uint8_t ex = uint8_t((v >> 7) & 0xFF);
                e[i] = ex;
                b->sm[i] = uint8_t(((v >> 8) & 0x80) | (v & 0x7F));
                ++h[ex];
            }
        });
        for (auto& h : hist_t)
            for (int k = 0; k < 256; ++k) b->hist[k] += h[k];

        // 2. palette: the 16 most frequent exponents by (-count, exponent)
        std::vector<std::pair<uint64_t, int>> present;
        for (int k = 0; k < 256; ++k)
            if (b->hist[k]) present.push_back({b->hist[k], k});
        std::sort(present.begin(), present.end(), [](auto a, auto c) {
            return a.first != c.first ? a.first > c.first : a.second < c.second;
        });
        b->P = int32_t(std::min<size_t>(present.size(), 16));
        int8_t idx_of[256];
        std::memset(idx_of, -1, sizeof(idx_of));
        for (int s = 0; s < b->P; ++s) {
            b->palette[s] = uint8_t(present[s].second);
            idx_of[present[s].second] = int8_t(s);
        }

        // 3. verbatim flags and symbol frequencies over coded groups
        std::vector<uint8_t> vflag(size_t(G), 0);
        std::vector<std::vector<uint64_t>> freq_t(nt, std::vector<uint64_t>(16, 0));
        parallel_for(T, nt, [&](int64_t t0, int64_t t1, int tid) {
            uint64_t* f = freq_t[tid].data();
            for (int64_t g = t0 * kTile; g < std::min<int64_t>(G, t1 * kTile); ++g) {
                const uint8_t* eg = e.data() + g * kGroup;
                bool verb = false;
                for (int j = 0; j < kGroup; ++j) verb |= idx_of[eg[j]] < 0;
                vflag[g] = verb;
                if (!verb)
                    for (int j = 0; j < kGroup; ++j) ++f[idx_of[eg[j]]];
            }
        });
        uint64_t freq[16] = {};
        for (auto& f : freq_t)
            for (int s = 0; s < 16; ++s) freq[s] += f[s];

        // 4. Huffman code lengths and canonical codes
        huffman_lengths(freq, b->lengths);
        uw::canonical_codes(b->lengths, b->codes);
        b->lmax = 0;
        for (int s = 0; s < 16; ++s) b->lmax = std::max<int32_t>(b->lmax, b->lengths[s]);

        // 5. per-group bit lengths, tile offsets, verbatim bases, bitmap
        b->glen.assign(size_t(G), 0);
        b->bitmap.assign(size_t(T), 0);
        std::vector<uint64_t> tile_bits(size_t(T), 0);
        std::vector<uint32_t> tile_v(size_t(T), 0);
        parallel_for(T, nt, [&](int64_t t0, int64_t t1, int) {
            for (int64_t t = t0; t < t1; ++t) {
                uint64_t bits = 0;
                for (int64_t g = t * kTile; g < std::min<int64_t>(G, (t + 1) * kTile); ++g) {
                    if (vflag[g]) {
                        b->bitmap[t] |= uint64_t(1) << (g % kTile);
                        ++tile_v[t];
                        continue;
                    }
                    const uint8_t* eg = e.data() + g * kGroup;
                    uint32_t gl = 0;
                    for (int j = 0; j < kGroup; ++j) gl += b->lengths[idx_of[eg[j]]];
                    gl = (gl + 3u) & ~3u;                    // padded to a 4-bit boundary
                    b->glen[g] = uint8_t(gl / 4u);           // <= 64 * 15 / 4 = 240
                    bits += gl;
                }
                tile_bits[t] = bits;
            }
        });
        b->tile_off.assign(size_t(T + 1), 0);
        b->tile_vbase.assign(size_t(T + 1), 0);
        uint64_t off = 0, vb = 0;
        for (int64_t t = 0; t < T; ++t) {
            b->tile_off[t] = uint32_t(off);
            b->tile_vbase[t] = uint32_t(vb);
            off += (tile_bits[t] + 7) / 8;
            vb += tile_v[t];
        }
        if (off > UINT32_MAX) {
            delete b;
            return uw::fail(UW_EUNSUPPORTED, "uw_compress: stream over 4 GiB");
        }
        b->tile_off[T] = uint32_t(off);
        b->tile_vbase[T] = uint32_t(vb);
        b->V = int64_t(vb);

        // 6. encode every tile's stream, MSB-first, zero-padded to a byte
        b->stream.assign(size_t(off), 0);
        b->vexp.assign(size_t(vb) * kGroup, 0);
        parallel_for(T, nt, [&](int64_t t0, int64_t t1, int) {
            for (int64_t t = t0; t < t1; ++t) {
                uint8_t* o = b->stream.data() + b->tile_off[t];
                uint64_t acc = 0;
                int nacc = 0;
                size_t pos = 0;
                uint64_t vslot = b->tile_vbase[t];
                for (int64_t g = t * kTile; g < std::min<int64_t>(G, (t + 1) * kTile); ++g) {
                    const uint8_t* eg = e.data() + g * kGroup;
                    if (vflag[g]) {
                        std::memcpy(b->vexp.data() + vslot * kGroup, eg, kGroup);
                        ++vslot;
                        continue;
                    }
                    uint32_t gbits = 0;
                    for (int j = 0; j < kGroup; ++j) {
                        int s = idx_of[eg[j]];
                        int L = b->lengths[s];
                        acc = (acc << L) | b->codes[s];
                        nacc += L;
                        gbits += uint32_t(L);
                        while (nacc >= 8) {
                            o[pos++] = uint8_t(acc >> (nacc - 8));
                            nacc -= 8;
                        }
                    }
                    // zero bits up to the group's 4-bit boundary (groups start on one)
                    const int padb = int((4u - (gbits & 3u)) & 3u);
                    acc <<= padb;
                    nacc += padb;
                    while (nacc >= 8) {
                        o[pos++] = uint8_t(acc >> (nacc - 8));
                        nacc -= 8;
                    }
                }
                if (nacc > 0) o[pos++] = uint8_t(acc << (8 - nacc));
            }
        });

        // 7. optional direct-palette nibbles, decode table
        if (emit_pal) uw::build_nibbles(*b, e.data(), nt);
        uw::build_dlut(*b);
        uw::build_mlut(*b);
    } catch (const std::bad_alloc&) {
        delete b;
        return uw::fail(UW_ENOMEM, "uw_compress: out of host memory");
    }
    *out = b;
    return UW_OK;
}

int uw_blob_add_palette(uw_blob* b) {
    uw::clear_error();
    if (!b) return uw::fail(UW_EINVAL, "uw_blob_add_palette: NULL blob");
    if (b->has_nib) return UW_OK;
    try {
        // exponents rebuilt from the Huffman form on the host
        std::vector<uint8_t> e(size_t(b->N), 0);
        for (int64_t t = 0; t < b->T; ++t) {
            const uint8_t* s = b->stream.data() + b->tile_off[t];
            uint64_t bitpos = 0, nbits = uint64_t(b->tile_off[t + 1] - b->tile_off[t]) * 8;
            for (int64_t g = t * kTile; g < std::min<int64_t>(b->G, (t + 1) * kTile); ++g) {
                if ((b->bitmap[t] >> (g % kTile)) & 1) continue;  // nibbles stay 0
                for (int j = 0; j < kGroup; ++j) {
                    uint32_t peek = 0;
                    for (int k = 0; k < b->lmax; ++k) {
                        uint64_t p = bitpos + k;
                        uint32_t bit = p < nbits ? (s[p >> 3] >> (7 - (p & 7))) & 1 : 0;
                        peek = (peek << 1) | bit;
                    }
                    uint8_t ent = b->dlut[peek];
                    e[g * kGroup + j] = b->palette[ent >> 4];
                    bitpos += ent & 15;
                }
                bitpos = (bitpos + 3) & ~uint64_t(3);   // the group's zero padding
            }
        }
        uw::build_nibbles(*b, e.data(), 0);
    } catch (const std::bad_alloc&) {
        return uw::fail(UW_ENOMEM, "uw_blob_add_palette: out of host memory");
    }
    return UW_OK;
}

void uw_blob_free(uw_blob* b) { delete b; }

int uw_blob_info(const uw_blob* b, uw_info* info) {
    uw::clear_error();
    if (!b || !info) return uw::fail(UW_EINVAL, "uw_blob_info: NULL argument");
    std::memset(info, 0, sizeof(*info));
    info->rows = b->rows;
    info->cols = b->cols;
    info->groups = b->G;
    info->tiles = b->T;
    info->verbatim_groups = b->V;
    info->palette_size = b->P;
    info->lmax = b->lmax;
    std::memcpy(info->palette, b->palette, 16);
    std::memcpy(info->lengths, b->lengths, 16);
    std::memcpy(info->codes, b->codes, sizeof(b->codes));
    std::memcpy(info->hist, b->hist, sizeof(b->hist));
    uint64_t* sb = info->section_bytes;
    sb[UW_SEC_SM] = b->sm.size();
    sb[UW_SEC_STREAM] = b->stream.size();
    sb[UW_SEC_GLEN] = b->glen.size();
    sb[UW_SEC_TILE_OFF] = b->tile_off.size() * 4;
    sb[UW_SEC_TILE_VBASE] = b->tile_vbase.size() * 4;
    sb[UW_SEC_VEXP] = b->vexp.size();
    sb[UW_SEC_BITMAP] = b->bitmap.size() * 8;
    sb[UW_SEC_NIB] = b->has_nib ? b->nib.size() : 0;
    sb[UW_SEC_DLUT] = b->dlut.size();
    sb[UW_SEC_MLUT] = b->mlut.size() * 4;
    info->huffman_form_bytes = uw::kHeaderBytes + sb[UW_SEC_SM] + sb[UW_SEC_STREAM] + sb[UW_SEC_GLEN] +
                               sb[UW_SEC_TILE_OFF] + sb[UW_SEC_TILE_VBASE] + sb[UW_SEC_VEXP] +
                               sb[UW_SEC_BITMAP];
    info->palette_form_bytes = uw::kHeaderBytes + sb[UW_SEC_SM] + b->N / 2 + sb[UW_SEC_VEXP] +
                               sb[UW_SEC_BITMAP] + sb[UW_SEC_TILE_VBASE];
    info->has_palette = b->has_nib;
    uint32_t mt = 0;
    for (size_t t = 0; t + 1 < b->tile_off.size(); ++t) mt = std::max(mt, b->tile_off[t + 1] - b->tile_off[t]);
    info->max_tile_bytes = mt;
    return UW_OK;
}

int uw_blob_section(const uw_blob* b, int sec, const void** ptr, uint64_t* bytes) {
    uw::clear_error();
    if (!b || !ptr || !bytes) return uw::fail(UW_EINVAL, "uw_blob_section: NULL argument");
    const void* p = nullptr;
    uint64_t n = 0;
    switch (sec) {
        case UW_SEC_SM: p = b->sm.data(); n = b->sm.size(); break;
        case UW_SEC_STREAM: p = b->stream.data(); n = b->stream.size(); break;
        case UW_SEC_GLEN: p = b->glen.data(); n = b->glen.size(); break;
        case UW_SEC_TILE_OFF: p = b->tile_off.data(); n = b->tile_off.size() * 4; break;
        case UW_SEC_TILE_VBASE: p = b->tile_vbase.data(); n = b->tile_vbase.size() * 4; break;
        case UW_SEC_VEXP: p = b->vexp.data(); n = b->vexp.size(); break;
        case UW_SEC_BITMAP: p = b->bitmap.data(); n = b->bitmap.size() * 8; break;
        case UW_SEC_NIB:
            if (b->has_nib) { p = b->nib.data(); n = b->nib.size(); }
            break;
        case UW_SEC_DLUT: p = b->dlut.data(); n = b->dlut.size(); break;
        case UW_SEC_MLUT: p = b->mlut.data(); n = b->mlut.size() * 4; break;
        default: return uw::fail(UW_EINVAL, "uw_blob_section: unknown section");
    }
    *ptr = n ? p : nullptr;
    *bytes = n;
    return UW_OK;
}

// ----------------------------------------------------------------- serialize
// Header (little-endian, 256 bytes):
//   0 "UWF2"  4 u32 version(2)  8 i64 rows  16 i64 cols  24 i64 V
//   32 u32 P  36 u32 lmax  40 u8 palette[16]  56 u8 lengths[16]
//   72 u64 bytes of sections SM..NIB [8]  136 u32 flags (bit 0: NIB stored)
// Sections follow in enum order, each at a 256-byte aligned offset.
namespace {
constexpr int kStored = UW_SEC_NIB + 1;
uint64_t align256(uint64_t x) { return (x + 255) & ~uint64_t(255); }
}  // namespace

int uw_blob_serialize(const uw_blob* b, void* buf, uint64_t cap, uint64_t* need) {
    uw::clear_error();
    if (!b || !need) return uw::fail(UW_EINVAL, "uw_blob_serialize: NULL argument");
    const void* ptrs[kStored];
    uint64_t sizes[kStored];
    uint64_t total = uw::kHeaderBytes;
    for (int s = 0; s < kStored; ++s) {
        uw_blob_section(b, s, &ptrs[s], &sizes[s]);
        total = align256(total) + sizes[s];
    }
    total = align256(total);
    *need = total;
    if (!buf) return UW_OK;
    if (cap < total) return uw::fail(UW_EINVAL, "uw_blob_serialize: buffer too small");
    uint8_t* o = static_cast<uint8_t*>(buf);
    std::memset(o, 0, size_t(total));
    std::memcpy(o, "UWF2", 4);
    uint32_t ver = 2, P = uint32_t(b->P), L = uint32_t(b->lmax), flags = b->has_nib ? 1u : 0u;
    std::memcpy(o + 4, &ver, 4);
    std::memcpy(o + 8, &b->rows, 8);
    std::memcpy(o + 16, &b->cols, 8);
    std::memcpy(o + 24, &b->V, 8);
    std::memcpy(o + 32, &P, 4);
    std::memcpy(o + 36, &L, 4);
    std::memcpy(o + 40, b->palette, 16);
    std::memcpy(o + 56, b->lengths, 16);
    std::memcpy(o + 72, sizes, 8 * kStored);
    std::memcpy(o + 136, &flags, 4);
    uint64_t pos = uw::kHeaderBytes;
    for (int s = 0; s < kStored; ++s) {
        pos = align256(pos);
        if (sizes[s]) std::memcpy(o + pos, ptrs[s], size_t(sizes[s]));
        pos += sizes[s];
    }
    return UW_OK;
}

int uw_blob_deserialize(const void* buf, uint64_t bytes, uw_blob** out) {
    uw::clear_error();
    if (!buf || !out) return uw::fail(UW_EINVAL, "uw_blob_deserialize: NULL argument");
    *out = nullptr;
    const uint8_t* in = static_cast<const uint8_t*>(buf);
    if (bytes < uw::kHeaderBytes || std::memcmp(in, "UWF2", 4) != 0)
        return uw::fail(UW_EFORMAT, std::memcmp(in, "UWF1", 4) == 0 && bytes >= 4
                                        ? "uw_blob_deserialize: format version 1 (16-bit group lengths) is not read; "
                                          "compress the weights again"
                                        : "uw_blob_deserialize: bad magic");
    uint32_t ver, P, L, flags;
    uint64_t sizes[kStored];
    uw_blob* b = new (std::nothrow) uw_blob;
    if (!b) return uw::fail(UW_ENOMEM, "uw_blob_deserialize: out of host memory");
    std::memcpy(&ver, in + 4, 4);
    std::memcpy(&b->rows, in + 8, 8);
    std::memcpy(&b->cols, in + 16, 8);
    std::memcpy(&b->V, in + 24, 8);
    std::memcpy(&P, in + 32, 4);
    std::memcpy(&L, in + 36, 4);
    std::memcpy(b->palette, in + 40, 16);
    std::memcpy(b->lengths, in + 56, 16);
    std::memcpy(sizes, in + 72, 8 * kStored);
    std::memcpy(&flags, in + 136, 4);
    auto bad = [&](const char* m) {
        delete b;
        return uw::fail(UW_EFORMAT, m);
    };
    if (ver != 2) return bad("uw_blob_deserialize: unknown version");
    if (b->rows < 0 || b->cols < 0 || b->cols % kGroup) return bad("uw_blob_deserialize: bad shape");
    if (b->cols && b->rows > (int64_t(1) << 40) / b->cols) return bad("uw_blob_deserialize: bad shape");
    if (P > 16 || L > uint32_t(uw::kMaxCodeLen)) return bad("uw_blob_deserialize: bad palette/lmax");
    b->P = int32_t(P);
    b->lmax = int32_t(L);
    b->N = b->rows * b->cols;
    b->G = b->N / kGroup;
    b->T = (b->G + kTile - 1) / kTile;
    b->has_nib = flags & 1;
    uint64_t pos = uw::kHeaderBytes;
    try {
        for (int s = 0; s < kStored; ++s) {
            pos = align256(pos);
            if (sizes[s] > bytes || pos > bytes - sizes[s]) return bad("uw_blob_deserialize: truncated");
            const uint8_t* p = in + pos;
            uint64_t n = sizes[s];
            auto need_mult = [&](uint64_t m) { return n % m == 0; };
            switch (s) {
                case UW_SEC_SM: b->sm.assign(p, p + n); break;
                case UW_SEC_STREAM: b->stream.assign(p, p + n); break;
                case UW_SEC_GLEN:
                    b->glen.resize(n);
                    if (n) std::memcpy(b->glen.data(), p, n);
                    break;
                case UW_SEC_TILE_OFF:
                    if (!need_mult(4)) return bad("uw_blob_deserialize: TILE_OFF size");
                    b->tile_off.resize(n / 4);
                    if (n) std::memcpy(b->tile_off.data(), p, n);
                    break;
                case UW_SEC_TILE_VBASE:
                    if (!need_mult(4)) return bad("uw_blob_deserialize: TILE_VBASE size");
                    b->tile_vbase.resize(n / 4);
                    if (n) std::memcpy(b->tile_vbase.data(), p, n);
                    break;
                case UW_SEC_VEXP: b->vexp.assign(p, p + n); break;
                case UW_SEC_BITMAP:
                    if (!need_mult(8)) return bad("uw_blob_deserialize: BITMAP size");
                    b->bitmap.resize(n / 8);
                    if (n) std::memcpy(b->bitmap.data(), p, n);
                    break;
                case UW_SEC_NIB: b->nib.assign(p, p + n); break;
            }
            pos += n;
        }
    } catch (const std::bad_alloc&) {
        delete b;
        return uw::fail(UW_ENOMEM, "uw_blob_deserialize: out of host memory");
    }
    // the code lengths are checked (at most 15, Kraft sum 1) before the
    // canonical codes and the decode tables are derived from them
    int rc = uw_validate(b);
    if (rc != UW_OK) {
        delete b;
        return rc;
    }
    uw::canonical_codes(b->lengths, b->codes);
    uw::build_dlut(*b);
    uw::build_mlut(*b);
    *out = b;
    return UW_OK;
}

// ------------------------------------------------------------------ validate
int uw_validate(const uw_blob* b) {
    uw::clear_error();
    if (!b) return uw::fail(UW_EINVAL, "uw_validate: NULL blob");
    auto bad = [](const std::string& m) { return uw::fail(UW_EFORMAT, "uw_validate: " + m); };
    if (b->rows < 0 || b->cols < 0 || b->cols % kGroup) return bad("cols not a multiple of 64");
    if (b->N != b->rows * b->cols || b->G != b->N / kGroup || b->T != (b->G + kTile - 1) / kTile)
        return bad("inconsistent sizes");
    if (b->P < 0 || b->P > 16) return bad("palette size over 16");
    if (int64_t(b->sm.size()) != b->N) return bad("SM size");
    if (int64_t(b->glen.size()) != b->G) return bad("GLEN size");
    if (int64_t(b->tile_off.size()) != b->T + 1 || int64_t(b->tile_vbase.size()) != b->T + 1)
        return bad("tile table size");
    if (int64_t(b->bitmap.size()) != b->T) return bad("BITMAP size");
    if (b->has_nib && int64_t(b->nib.size()) != b->N / 2) return bad("NIB size");
    // code lengths: only palette symbols, <= 15, Kraft equality (or one code of length 1)
    int ncoded = 0, lmax = 0;
    uint64_t kraft = 0;  // in units of 2^-15
    for (int s = 0; s < 16; ++s) {
        int l = b->lengths[s];
        if (!l) continue;
        if (s >= b->P) return bad("code for a symbol outside the palette");
        if (l > uw::kMaxCodeLen) return bad("code length over 15");
        ++ncoded;
        lmax = std::max(lmax, l);
        kraft += uint64_t(1) << (uw::kMaxCodeLen - l);
    }
    if (lmax != b->lmax) return bad("lmax does not match the code lengths");
    if (ncoded >= 2 && kraft != (uint64_t(1) << uw::kMaxCodeLen)) return bad("Kraft sum is not 1");
    if (ncoded == 1 && lmax != 1) return bad("single code must have length 1");
    int minlen = 16;
    for (int s = 0; s < 16; ++s)
        if (b->lengths[s]) minlen = std::min<int>(minlen, b->lengths[s]);
    // tile tables
    if (b->tile_off[0] != 0 || b->tile_vbase[0] != 0) return bad("tables must start at 0");
    if (uint64_t(b->tile_off[b->T]) != b->stream.size()) return bad("TILE_OFF[T] != stream bytes");
    if (int64_t(b->tile_vbase[b->T]) != b->V || int64_t(b->vexp.size()) != b->V * kGroup)
        return bad("verbatim count mismatch");
    for (int64_t t = 0; t < b->T; ++t) {
        if (b->tile_off[t + 1] < b->tile_off[t]) return bad("TILE_OFF not monotone");
        uint64_t pc = uint64_t(__builtin_popcountll(b->bitmap[t]));
        if (b->tile_vbase[t + 1] < b->tile_vbase[t] || b->tile_vbase[t + 1] - b->tile_vbase[t] != pc)
            return bad("bitmap popcount != TILE_VBASE step");
        int64_t g0 = t * kTile, g1 = std::min<int64_t>(b->G, g0 + kTile);
        if (g1 - g0 < kTile && (b->bitmap[t] >> (g1 - g0)) != 0) return bad("bitmap bit past the last group");
        uint64_t bits = 0;
        for (int64_t g = g0; g < g1; ++g) {
            bool verb = (b->bitmap[t] >> (g - g0)) & 1;
            const uint32_t gl = 4u * b->glen[g];     // padded bits
            if (verb) {
                if (gl) return bad("verbatim group with coded bits");
                continue;
            }
            if (!ncoded || gl < uint32_t(64 * minlen) || gl > uint32_t(64 * lmax))
                return bad("group bit length out of range");
            bits += gl;
        }
        if ((bits + 7) / 8 != uint64_t(b->tile_off[t + 1] - b->tile_off[t]))
            return bad("tile bytes do not match its group bit lengths");
    }
    if (b->has_nib)
        for (int64_t g = 0; g < b->G; ++g)
            if ((b->bitmap[g / kTile] >> (g % kTile)) & 1)
                for (int j = 0; j < kGroup / 2; ++j)
                    if (b->nib[g * (kGroup / 2) + j]) return bad("nonzero nibbles in a verbatim group");
    return UW_OK;
}

}  // extern "C"
