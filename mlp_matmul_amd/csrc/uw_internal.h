// Internal declarations shared by the host translation units of libunweight.
#pragma once

#include <cstdint>
#include <string>
#include <vector>

#include "unweight.h"

namespace uw {

constexpr int kGroup = 64;       // elements per verbatim decision
constexpr int kTile = 64;        // groups per stream tile
constexpr int kPaletteMax = 16;  // 4-bit palette indices
constexpr int kMaxCodeLen = 15;  // 16 symbols -> Huffman depth <= 15
constexpr uint64_t kHeaderBytes = 256;

// Record a message for uw_last_error() and return the code.
int fail(int code, const std::string& msg);
void clear_error();

// The current HIP device: its ordinal (-1 when no device can be selected) and
// an identity for tuned plans, "<gcnArchName>/<compute units>cu" ("none"
// without a device).  Defined with the HIP entry points.
int current_device();
std::string device_key(int ordinal);

}  // namespace uw

struct uw_blob {
    int64_t rows = 0, cols = 0;
    int64_t N = 0, G = 0, T = 0, V = 0;
    int32_t P = 0, lmax = 0;
    uint8_t palette[16] = {};
    uint8_t lengths[16] = {};
    uint16_t codes[16] = {};
    uint64_t hist[256] = {};
    bool has_nib = false;
    std::vector<uint8_t> sm, stream, vexp, nib, dlut;
    std::vector<uint32_t> mlut;
    std::vector<uint8_t> glen;     // padded coded bits of each group / 4
    std::vector<uint32_t> tile_off, tile_vbase;
    std::vector<uint64_t> bitmap;
};

namespace uw {
// Canonical codewords from code lengths (symbols in (length, symbol) order).
void canonical_codes(const uint8_t lengths[16], uint16_t codes[16]);
// Decode table of 2^lmax entries: (symbol << 4) | length.
void build_dlut(uw_blob& b);
// Multi-symbol table over 12-bit strings (layout in unweight.h), built from
// the decode table; requires build_dlut first.
constexpr int kMlutBits = 12;
void build_mlut(uw_blob& b);
// Direct-palette nibbles from the exponent of every element.
void build_nibbles(uw_blob& b, const uint8_t* e, int threads);
}  // namespace uw
