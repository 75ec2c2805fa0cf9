// Tile-parallel Huffman decoder for gfx950: full bf16, exponent-only and
// palette-transcode outputs.
//
// Method: Cloudflare, "Unweight: how we compressed an LLM 22% without
// sacrificing quality", section "Four ways to use compressed weights": the
// full Huffman decode rebuilds bf16 for a plain matmul, the exponent-only
// decode writes half as many bytes back, the palette transcode writes 4-bit
// indices (a quarter) and is also how the direct-palette form is made at load
// time.  Verbatim 64-element rows ("How to compress model weights
// effectively") are copied from the raw exponent array.
//
// Mapping to CDNA4: one wavefront per tile of 64 groups, one lane per group.
// The wave copies the tile's stream bytes into LDS with coalesced dword loads;
// each lane finds its group's first bit by a wave prefix sum of the per-group
// bit lengths, then walks 64 codewords through a 64-bit window and a 2^lmax
// byte lookup table held in LDS.  Symbols are kept as packed nibbles in
// registers and written out with 16-byte stores per lane.
#include "device_common.h"
#include "kernels.h"

namespace uwk {

namespace {

constexpr int kDecWaves = 4;

__device__ __forceinline__ uint32_t load_word(const uint8_t* s, uint32_t w, uint64_t nbytes) {
    uint64_t b = uint64_t(w) * 4;
    if (b + 4 <= nbytes) return reinterpret_cast<const uint32_t*>(s)[w];
    uint32_t v = 0;
    for (int i = 0; i < 4; ++i)
        if (b + i < nbytes) v |= uint32_t(s[b + i]) << (8 * i);
    return v;
}

__device__ __forceinline__ uint32_t pal_byte(const DecodeArgs& a, int i) { return uwk::pal_byte(a.pal, uint32_t(i)); }

template <int MODE>
__global__ __launch_bounds__(256) void decode_kernel(DecodeArgs a) {
    extern __shared__ uint32_t lds[];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int lmax = a.lmax;
    const uint32_t lut_bytes = 1u << lmax;
    const uint32_t lut_words = (lut_bytes + 3) / 4;
    uint32_t* lut_w = lds;
    uint32_t* ptab = lds + lut_words;          // 256 entries indexed by a nibble pair
    uint32_t* buf = ptab + 256 + wave * a.buf_words;

    // code table -> LDS
    if (lut_bytes >= 4) {
        for (uint32_t i = tid; i < lut_words; i += 256) lut_w[i] = reinterpret_cast<const uint32_t*>(a.dlut)[i];
    } else if (tid == 0) {
        uint32_t v = 0;
        for (uint32_t i = 0; i < lut_bytes; ++i) v |= uint32_t(a.dlut[i]) << (8 * i);
        lut_w[0] = v;
    }
    // nibble pair -> (FULL) two exponents in bf16 position, (EXP) two exponent bytes
    {
        uint32_t lo = pal_byte(a, tid & 15), hi = pal_byte(a, tid >> 4);
        ptab[tid] = MODE == MODE_FULL ? (lo << 7) | (hi << 23) : lo | (hi << 8);
    }
    __syncthreads();
    const uint8_t* lutb = reinterpret_cast<const uint8_t*>(lut_w);
    const uint32_t lim = uint32_t(a.buf_words) - 1;
    const int rs = 64 - (lmax > 0 ? lmax : 1);

    for (int64_t tb = int64_t(blockIdx.x) * kDecWaves; tb < a.T; tb += int64_t(gridDim.x) * kDecWaves) {
        const int64_t t = tb + wave;
        const bool tile_ok = t < a.T;
        uint32_t off0 = 0, off1 = 0, vbase = 0;
        uint64_t word = 0;
        if (tile_ok) {
            off0 = a.tile_off[t];
            off1 = a.tile_off[t + 1];
            word = a.bitmap[t];
            vbase = a.tile_vbase[t];
        }
        // stage the tile's stream (dword aligned) plus two zero words
        const uint32_t w0 = off0 >> 2;
        uint32_t nw = tile_ok ? ((off1 + 3) >> 2) - w0 : 0;
        nw = min(nw, uint32_t(a.buf_words) - 2);
        for (uint32_t i = lane; i < nw + 2; i += 64) buf[i] = i < nw ? load_word(a.stream, w0 + i, a.stream_bytes) : 0u;
        __syncthreads();

        const int64_t g = t * 64 + lane;
        const bool gvalid = tile_ok && g < a.G;
        const uint32_t gl = gvalid ? a.glen[g] : 0u;
        uint32_t incl = gl;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            uint32_t v = __shfl_up(incl, d, 64);
            if (lane >= d) incl += v;
        }
        const uint32_t start = incl - gl + ((off0 & 3u) << 3);
        const bool verb = (word >> lane) & 1ull;

        if (gvalid && !verb) {
            uint32_t wp = start >> 5;
            const uint32_t sh = start & 31;
            uint64_t win = (uint64_t(bswap32(buf[min(wp, lim)])) << 32) | bswap32(buf[min(wp + 1, lim)]);
            win <<= sh;
            int avail = 64 - int(sh);
            wp += 2;
            uint32_t nib[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
            for (int j = 0; j < 64; ++j) {
                if (avail < 32) {
                    win |= uint64_t(bswap32(buf[min(wp, lim)])) << (32 - avail);
                    ++wp;
                    avail += 32;
                }
                const uint32_t ent = lutb[uint32_t(win >> rs)];
                const uint32_t len = ent & 15u;
                nib[j >> 3] |= (ent >> 4) << (4 * (j & 7));
                win <<= len;
                avail -= int(len);
            }
            if (MODE == MODE_PAL) {
                uint8_t* o = static_cast<uint8_t*>(a.out) + g * 32;
                store16(o, u32x4_t{nib[0], nib[1], nib[2], nib[3]});
                store16(o + 16, u32x4_t{nib[4], nib[5], nib[6], nib[7]});
            } else if (MODE == MODE_EXP) {
                uint8_t* o = static_cast<uint8_t*>(a.out) + g * 64;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    uint32_t d[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int k = q * 8 + i * 2;   // nibble-pair bytes k, k+1
                        const uint32_t b0 = (nib[k >> 2] >> (8 * (k & 3))) & 0xFFu;
                        const uint32_t b1 = (nib[(k + 1) >> 2] >> (8 * ((k + 1) & 3))) & 0xFFu;
                        d[i] = ptab[b0] | (ptab[b1] << 16);
                    }
                    store16(o + 16 * q, u32x4_t{d[0], d[1], d[2], d[3]});
                }
            } else {
                const uint8_t* smg = a.sm + g * 64;
                uint16_t* o = static_cast<uint16_t*>(a.out) + g * 64;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const u32x4_t s4 = load_stream16(smg + 16 * q);
                    uint32_t d[8];
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        const int k = q * 8 + i;       // nibble-pair byte k = elements 2k, 2k+1
                        const uint32_t nb = (nib[k >> 2] >> (8 * (k & 3))) & 0xFFu;
                        d[i] = (i & 1) ? join_pair<1>(s4[i >> 1], ptab[nb]) : join_pair<0>(s4[i >> 1], ptab[nb]);
                    }
                    store16(o + 16 * q, u32x4_t{d[0], d[1], d[2], d[3]});
                    store16(o + 16 * q + 8, u32x4_t{d[4], d[5], d[6], d[7]});
                }
            }
        } else if (gvalid) {
            const uint32_t slot = verbatim_slot(word, uint32_t(lane), vbase);
            const uint8_t* vx = a.vexp + uint64_t(slot) * 64;
            if (MODE == MODE_PAL) {
                uint8_t* o = static_cast<uint8_t*>(a.out) + g * 32;
                store16(o, u32x4_t{0, 0, 0, 0});
                store16(o + 16, u32x4_t{0, 0, 0, 0});
            } else if (MODE == MODE_EXP) {
                uint8_t* o = static_cast<uint8_t*>(a.out) + g * 64;
#pragma unroll
                for (int q = 0; q < 4; ++q) store16(o + 16 * q, load16(vx + 16 * q));
            } else {
                const uint8_t* smg = a.sm + g * 64;
                uint16_t* o = static_cast<uint16_t*>(a.out) + g * 64;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const u32x4_t s4 = load_stream16(smg + 16 * q);
                    const u32x4_t e4 = load16(vx + 16 * q);
                    uint32_t d[8];
#pragma unroll
                    for (int i = 0; i < 8; ++i)
                        d[i] = (i & 1) ? join_pair<1>(s4[i >> 1], exp_pair<1>(e4[i >> 1]))
                                       : join_pair<0>(s4[i >> 1], exp_pair<0>(e4[i >> 1]));
                    store16(o + 16 * q, u32x4_t{d[0], d[1], d[2], d[3]});
                    store16(o + 16 * q + 8, u32x4_t{d[4], d[5], d[6], d[7]});
                }
            }
        }
        __syncthreads();
    }
}

}  // namespace

size_t decode_lds_bytes(int lmax, int* buf_words) {
    // a tile holds at most 64 groups x 64 codes x lmax bits = 512*lmax bytes;
    // +1 word for a misaligned start, +2 zero words for the lookahead window
    const int bw = 128 * (lmax > 0 ? lmax : 1) + 4;
    if (buf_words) *buf_words = bw;
    const size_t lut_words = ((size_t(1) << lmax) + 3) / 4;
    return (lut_words + 256 + size_t(kDecWaves) * bw) * 4;
}

hipError_t launch_decode(int mode, const DecodeArgs& a0, hipStream_t s) {
    DecodeArgs a = a0;
    const size_t lds = decode_lds_bytes(a.lmax, &a.buf_words);
    const int64_t blocks = (a.T + kDecWaves - 1) / kDecWaves;
    const unsigned grid = unsigned(blocks < 1024 ? (blocks > 0 ? blocks : 1) : 1024);
    if (a.T == 0) return hipSuccess;
    switch (mode) {
        case MODE_FULL: decode_kernel<MODE_FULL><<<grid, 256, lds, s>>>(a); break;
        case MODE_EXP: decode_kernel<MODE_EXP><<<grid, 256, lds, s>>>(a); break;
        default: decode_kernel<MODE_PAL><<<grid, 256, lds, s>>>(a); break;
    }
    return hipGetLastError();
}

}  // namespace uwk
