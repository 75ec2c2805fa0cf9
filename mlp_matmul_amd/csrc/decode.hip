// Tile-parallel Huffman decoder for gfx950: full bf16, exponent-only and
// palette-transcode outputs, and the decode inside a batch-1 matmul.
//
// Method: Cloudflare, "Unweight: how we compressed an LLM 22% without
// sacrificing quality", section "Four ways to use compressed weights": the
// full Huffman decode rebuilds bf16 for a plain matmul, the exponent-only
// decode writes half as many bytes back, the palette transcode writes 4-bit
// indices (a quarter) and is also how the direct-palette form is made at load
// time.  Verbatim 64-element rows ("How to compress model weights
// effectively") are copied from the raw exponent array.
//
// Mapping to CDNA4: one wavefront per tile of 64 groups, one lane per group,
// eight wavefronts per workgroup sharing the lookup tables in LDS.  The wave
// copies the tile's stream into LDS with 16-byte loads issued together
// (byte-swapped so each word reads MSB-first), and each lane finds its
// group's first bit by a wave prefix sum of the per-group bit lengths.  A
// lane then decodes its 64 codewords several at a time: a 32-bit window at
// its bit position (one funnel shift of two LDS words) indexes a 4096-entry
// multi-symbol table that yields up to four symbols, their count and their
// total length per lookup (about 3.7 symbols for these codes, so ~19
// lookups per group instead of 64).  Codewords longer than the 12-bit index
// fall back to the single-symbol table.  Symbols are appended to a 64-bit
// accumulator whose words go to a per-lane LDS slot.  The output phase then
// walks the tile in element order, 8 elements per lane and 512 per wave
// instruction, so that exponent and bf16 stores (and the sign/mantissa
// loads) are contiguous across the wave; it maps palette indices to
// exponents through an LDS table of nibble pairs (full bf16) or with byte
// permutes of the palette held in registers (exponent-only, where it
// measured faster: the lookup loop already keeps LDS busy).  The stream buffer is sized by the
// matrix's longest tile, which keeps LDS per wave small enough for several
// workgroups per CU.
//
// The fourth mode decodes inside a batch-1 matmul (Huffman stream straight
// from HBM, no decoded plane written): the output phase's element walk
// rebuilds each lane's 8 weights in registers, multiplies them with the
// matching activations (v_dot2, fp32) and keeps two sums per lane, for the
// first and the second row the tile touches (a tile is 4096 elements, so at
// most two rows when rows have at least 4096 columns); two wave sums give
// the tile's partials, which a second kernel adds up per row in tile order
// (deterministic).  This goes past the page's four pipelines: decode and
// matmul in one pass, reading the Huffman form (the smallest) once.
#include "device_common.h"
#include "kernels.h"

namespace uwk {

namespace {

constexpr int kDecWaves = 8;
constexpr int kMlutEntries = 4096;      // 12-bit index
constexpr int kTailWords = 16;          // the last 64 single-symbol entries, bytes
constexpr int kSlot = 9;                // LDS words per lane: 64 nibbles + one overflow word
constexpr int kStageRounds = 4;         // 16-byte loads per lane issued before one wait

typedef uint32_t u32x4_a4 __attribute__((ext_vector_type(4), aligned(4)));

__device__ __forceinline__ uint32_t load_word(const uint8_t* s, uint32_t w, uint64_t nbytes) {
    uint64_t b = uint64_t(w) * 4;
    if (b + 4 <= nbytes) return reinterpret_cast<const uint32_t*>(s)[w];
    uint32_t v = 0;
    for (int i = 0; i < 4; ++i)
        if (b + i < nbytes) v |= uint32_t(s[b + i]) << (8 * i);
    return v;
}

__device__ __forceinline__ uint32_t pal_byte(const DecodeArgs& a, int i) { return uwk::pal_byte(a.pal, uint32_t(i)); }

// Orders this wave's LDS accesses around a point: LDS operations of one
// wavefront complete in program order, so only the compiler must not move
// accesses across it.
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

typedef __attribute__((address_space(3))) uint32_t lds_u32;

// LDS word at a byte address
__device__ __forceinline__ uint32_t lds_ld(uint32_t addr) {
    return *reinterpret_cast<const lds_u32*>(static_cast<uintptr_t>(addr));
}
__device__ __forceinline__ void lds_st(uint32_t addr, uint32_t v) {
    *reinterpret_cast<lds_u32*>(static_cast<uintptr_t>(addr)) = v;
}

// Stream word w (any index; words outside [0, nbytes) read as zero bytes)
__device__ __forceinline__ uint32_t load_word_any(const uint8_t* s, int64_t w, uint64_t nbytes) {
    return w < 0 ? 0u : load_word(s, uint32_t(w), nbytes);
}

template <int MODE>
__global__ __launch_bounds__(64 * kDecWaves, 6) void decode_kernel(DecodeArgs a) {
    extern __shared__ uint32_t lds[];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: tile metadata in scalar loads
    const int lmax = a.lmax;
    const uint32_t bw = uint32_t(a.buf_words);   // multiple of 4
    // LDS: the multi-symbol table (at address 0), the nibble-pair table and
    // the single-symbol table's tail shared by the workgroup, then per wave
    // [stream buffer | 64 symbol slots]
    const uint32_t wave_words = bw + 64 * kSlot;
    uint32_t* mlut = lds;
    uint32_t* ptab = lds + kMlutEntries;
    uint8_t* tail = reinterpret_cast<uint8_t*>(ptab + 256);
    uint32_t* buf = ptab + 256 + kTailWords + wave * wave_words;
    // byte addresses; the empty asm keeps the wave's base one opaque scalar
    // so that each window read needs a single address instruction
    uint32_t buf_a = uint32_t((kMlutEntries + 256 + kTailWords + wave * wave_words) * 4);
    asm("" : "+s"(buf_a));
    const uint32_t slots_a = buf_a + bw * 4;
    const uint32_t ptab_a = kMlutEntries * 4;

    const int fb_shift = 32 - (lmax > 0 ? lmax : 1);
    const bool vec_ok = a.stream_bytes >= 16;
    const int64_t N = a.G * 64;
    const int64_t S = int64_t(gridDim.x) * kDecWaves;     // tile stride of a wave

    for (int i = tid; i < kMlutEntries / 4; i += 64 * kDecWaves)
        reinterpret_cast<u32x4_t*>(mlut)[i] = reinterpret_cast<const u32x4_t*>(a.mlut)[i];
    if ((MODE == MODE_FULL || MODE == MODE_GEMV) && tid < 256) {
        // nibble pair -> two exponents in bf16 position
        uint32_t lo = pal_byte(a, tid & 15), hi = pal_byte(a, tid >> 4);
        ptab[tid] = (lo << 7) | (hi << 23);
    }
    // A window whose first codeword is longer than the 12-bit index starts
    // with one of the longest, numerically largest canonical codes, so its
    // lmax-bit value lies in the top of the single-symbol table: at most 16
    // codes of 13-15 bits cover at most 16 * 4 = 64 such values.  That tail
    // is kept here, so the fallback is an LDS read, not a global load.
    const uint32_t dlut_n = 1u << lmax;
    const uint32_t tail_base = dlut_n > 64u ? dlut_n - 64u : 0u;
    if (tid < 64) tail[tid] = tail_base + uint32_t(tid) < dlut_n ? a.dlut[tail_base + uint32_t(tid)] : uint8_t(0);
    // EXP output: four palette indices (one per byte) -> their exponent
    // bytes with v_perm on the 16 palette bytes held in four uniform words
    // (selectors 0-7 pick a byte; 12 and 13 give 0x00 and 0xFF, the mask
    // choosing entries 8-15)
    const uint32_t P0 = __builtin_amdgcn_readfirstlane(a.pal[0]), P1 = __builtin_amdgcn_readfirstlane(a.pal[1]);
    const uint32_t P2 = __builtin_amdgcn_readfirstlane(a.pal[2]), P3 = __builtin_amdgcn_readfirstlane(a.pal[3]);
    auto pal4 = [&](uint32_t x) {
        const uint32_t sel = x & 0x07070707u;
        const uint32_t lo8 = __builtin_amdgcn_perm(P1, P0, sel), hi8 = __builtin_amdgcn_perm(P3, P2, sel);
        const uint32_t m = __builtin_amdgcn_perm(0u, 0u, ((x >> 3) & 0x01010101u) | 0x0C0C0C0Cu);
        return (hi8 & m) | (lo8 & ~m);
    };
    __syncthreads();

    // waves take tiles independently (no workgroup barrier in the loop)
    for (int64_t t = int64_t(blockIdx.x) * kDecWaves + wave; t < a.T; t += S) {
        const uint32_t off0 = a.tile_off[t], off1 = a.tile_off[t + 1], vbase = a.tile_vbase[t];
        const uint64_t word = a.bitmap[t];
        const int64_t g = t * 64 + lane;
        const bool gvalid = g < a.G;
        // padded bits of the lane's group (the next group starts there); the
        // load is unconditional and its use too (lanes past the last group
        // read the tile's first byte and mask it), so the compiler cannot
        // move the load, and the wait for it, into a branch
        const uint32_t gl0 = (a.glen + t * 64)[gvalid ? uint32_t(lane) : 0u];
        const uint32_t gl = (4u * gl0) & (0u - uint32_t(gvalid));
        const bool verb = (word >> lane) & 1ull;
        // output phase: lane handles elements 512k + 8*lane .. +7 of the tile
        const int64_t e0 = t * 4096 + 8 * lane;
        // the tile's first two verbatim groups (if any), one element per lane;
        // a third and later ones (rare) are loaded when written
        const uint64_t w1 = word & (word - 1);
        const uint32_t vg0 = word ? uint32_t(__builtin_ctzll(word)) : 64u;
        const uint32_t vg1 = w1 ? uint32_t(__builtin_ctzll(w1)) : 64u;
        uint32_t ve0 = 0, ve1 = 0, vs0 = 0, vs1 = 0;
        if (MODE != MODE_PAL && word && t * 64 + vg0 < a.G) {
            ve0 = a.vexp[uint64_t(vbase) * 64 + lane];
            if (MODE == MODE_FULL || MODE == MODE_GEMV) vs0 = a.sm[(t * 64 + vg0) * 64 + lane];
            if (w1 && t * 64 + vg1 < a.G) {
                ve1 = a.vexp[uint64_t(vbase + 1) * 64 + lane];
                if (MODE == MODE_FULL || MODE == MODE_GEMV) vs1 = a.sm[(t * 64 + vg1) * 64 + lane];
            }
        }

        // stage stream words w0-1 .. w0+nw into buf[0 .. nw+1]: a lead word
        // (never decisive: the window of bit position p reads words
        // (p+31)/32 and the next one), the tile, one lookahead word; words
        // past the tile only ever feed codewords that are discarded
        const uint32_t w0 = off0 >> 2;
        const uint32_t nw = off1 > off0 ? ((off1 + 3) >> 2) - w0 : 0;
        const uint32_t need = min(nw + 2, bw);
        wave_lds_sync();     // the previous tile's reads of buf and slots are done
        auto stage = [&](uint32_t base) {
            u32x4_t v[kStageRounds];
#pragma unroll
            for (int r = 0; r < kStageRounds; ++r) {
                const int64_t wi = int64_t(w0) - 1 + base + 256 * r + 4 * lane;
                const bool fast = vec_ok && wi >= 0 && uint64_t(wi) * 4 + 16 <= a.stream_bytes;
                // no access at all for lanes past the stream (it may be empty and NULL)
                v[r] = fast ? *reinterpret_cast<const u32x4_a4*>(a.stream + uint64_t(wi) * 4) : u32x4_t{0, 0, 0, 0};
            }
#pragma unroll
            for (int r = 0; r < kStageRounds; ++r) {
                const uint32_t i = base + 256 * r + 4 * lane;
                if (i < need) {
                    const int64_t wi = int64_t(w0) - 1 + i;
                    if (!(vec_ok && wi >= 0 && uint64_t(wi) * 4 + 16 <= a.stream_bytes)) {   // stream ends
#pragma unroll 1
                        for (int k = 0; k < 4; ++k) v[r][k] = load_word_any(a.stream, wi + k, a.stream_bytes);
                    }
                    *reinterpret_cast<u32x4_t*>(buf + i) =
                        u32x4_t{bswap32(v[r][0]), bswap32(v[r][1]), bswap32(v[r][2]), bswap32(v[r][3])};
                }
            }
        };
        // one pass covers 4 KiB, every tile of these codes; longer ones loop
        stage(0);
        for (uint32_t base = 256 * kStageRounds; base < need; base += 256 * kStageRounds) stage(base);
        wave_lds_sync();
        // FULL: the sign/mantissa bytes of the lane's output elements go out
        // now and arrive during the lookups
        u32x2_t smv[8];
        if (MODE == MODE_FULL || MODE == MODE_GEMV) {
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const int64_t e = e0 + 512 * k;
                smv[k] = load_stream8(a.sm + (e < N ? e : 0));
            }
        }

        uint32_t incl = gl;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            uint32_t v = __shfl_up(incl, d, 64);
            if (lane >= d) incl += v;
        }

        // q = 31 + bit position from buf[1]; nc4 = 4 x symbols decoded (256 = done).
        // A lane makes at most 64 lookups of at most 255 bits each (entries
        // carry 8-bit lengths), so clamping its start once keeps every window
        // read inside this wave's buffer and slots; for a consistent stream
        // the clamp never binds.
        // q carries the buffer's LDS address (x 8, a multiple of 32, so its
        // low five bits are unchanged): the window's word address is then
        // (q >> 3) & ~3 with no add.
        uint32_t q = min(incl - gl + ((off0 & 3u) << 3) + 31, (bw + 64u) * 32u) + buf_a * 8u;
        uint32_t nc4 = (gvalid && !verb && lmax > 0) ? 0u : 256u;
        uint32_t oa = slots_a + lane * (kSlot * 4);
        uint32_t cur = 0;                   // the slot word being filled, 8 nibbles
        while (nc4 < 256u) {
            const uint32_t wa = (q >> 3) & ~3u;
            const uint32_t win = __builtin_amdgcn_alignbit(lds_ld(wa), lds_ld(wa + 4), ~q);
            uint32_t e = lds_ld((win >> 18) & 0x3FFCu);      // table entry win>>20
            if (e == 0) {                   // first codeword longer than 12 bits
                const uint32_t d = tail[((win >> fb_shift) - tail_base) & 63u];
                e = (d & 15u) | (4u << 8) | ((d >> 4) << 16);
            }
            q += e & 0xFFu;
            // append up to 4 nibbles at bit s of the word and store it; when
            // they run past bit 31 (then s >= 16) the word is complete and
            // its overflow, syms >> (32 - s), starts the next one
            const uint32_t syms = e >> 16, s = nc4 & 31u;
            cur |= syms << s;
            lds_st(oa, cur);
            const uint32_t nn = nc4 + ((e >> 8) & 0xFFu);
            const bool done = ((nn ^ nc4) & 32u) != 0;
            const uint32_t spill = __builtin_amdgcn_alignbit(0u, syms, 32u - s);
            cur = done ? spill : cur;
            oa += done ? 4u : 0u;
            nc4 = nn;
        }

        if (MODE == MODE_PAL) {
            // own slot: 32 contiguous bytes per lane
            if (gvalid) {
                const uint32_t sa = slots_a + lane * (kSlot * 4);
                uint32_t nib[8];
#pragma unroll
                for (int k = 0; k < 8; ++k) nib[k] = verb ? 0u : lds_ld(sa + 4 * k);
                uint8_t* out = static_cast<uint8_t*>(a.out) + g * 32;
                store16(out, u32x4_t{nib[0], nib[1], nib[2], nib[3]});
                store16(out + 16, u32x4_t{nib[4], nib[5], nib[6], nib[7]});
            }
        } else {
            wave_lds_sync();     // slots are read across lanes
            // GEMV: the tile's elements before `rsplit` lie in its first row
            // (starting at column c_first), the rest in the next row
            float acc0 = 0.f, acc1 = 0.f;
            uint32_t rsplit = 0, c_first = 0;      // cols < 2^31; tile-relative positions < 4096
            if (MODE == MODE_GEMV) {
                const int64_t cf = (t * 4096) % a.C;
                c_first = uint32_t(cf);
                rsplit = uint32_t(a.C - cf < 4096 ? a.C - cf : 4096);
            }
            // non-verbatim groups: 8 elements per lane, 512 per instruction
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const uint32_t gi = 8 * k + (lane >> 3);
                const int64_t e = e0 + 512 * k;
                if (e >= N || ((word >> gi) & 1ull)) continue;
                const uint32_t nw32 = lds_ld(slots_a + gi * (kSlot * 4) + 4 * (lane & 7));
                if (MODE == MODE_EXP) {
                    // palette lookups in registers: even and odd elements'
                    // exponents, then interleaved into element order
                    const uint32_t ev = pal4(nw32 & 0x0F0F0F0Fu), od = pal4((nw32 >> 4) & 0x0F0F0F0Fu);
                    *reinterpret_cast<u32x2_t*>(static_cast<uint8_t*>(a.out) + e) =
                        u32x2_t{__builtin_amdgcn_perm(od, ev, 0x05010400u), __builtin_amdgcn_perm(od, ev, 0x07030602u)};
                } else {
                    uint32_t pr[4];     // ptab entries of the 4 nibble pairs
#pragma unroll
                    for (int i = 0; i < 4; ++i) pr[i] = lds_ld(ptab_a + ((nw32 >> (8 * i)) & 0xFFu) * 4);
                    const u32x2_t s8 = smv[k];
                    const u32x4_t w = u32x4_t{join_pair<0>(s8[0], pr[0]), join_pair<1>(s8[0], pr[1]),
                                              join_pair<0>(s8[1], pr[2]), join_pair<1>(s8[1], pr[3])};
                    if (MODE == MODE_GEMV) {
                        // the lane's 8 weights lie in one row (rows are whole groups)
                        const uint32_t et = 8u * uint32_t(lane) + 512u * k;      // e - t * 4096
                        const bool second = et >= rsplit;
                        const u32x4_t xv = load16(a.x + (second ? et - rsplit : c_first + et));
                        float s = dot2_bf16(w[0], xv[0], 0.f);
                        s = dot2_bf16(w[1], xv[1], s);
                        s = dot2_bf16(w[2], xv[2], s);
                        s = dot2_bf16(w[3], xv[3], s);
                        if (second) acc1 += s;
                        else acc0 += s;
                    } else {
                        store16(static_cast<uint16_t*>(a.out) + e, w);
                    }
                }
            }
            // verbatim groups: the whole wave writes one group, lane = element
            uint64_t rest = word;
            for (uint32_t r = 0; rest; ++r, rest &= rest - 1) {
                const uint32_t gi = uint32_t(__builtin_ctzll(rest));
                if (t * 64 + gi >= a.G) break;       // bits past the last group (invalid input)
                const int64_t e = (t * 64 + gi) * 64 + lane;
                uint32_t ev, sv = 0;
                if (r == 0) {
                    ev = ve0;
                    sv = vs0;
                } else if (r == 1) {
                    ev = ve1;
                    sv = vs1;
                } else {
                    ev = a.vexp[uint64_t(vbase + r) * 64 + lane];
                    if (MODE == MODE_FULL || MODE == MODE_GEMV) sv = a.sm[e];
                }
                const uint32_t wb = ((sv & 0x80u) << 8) | (ev << 7) | (sv & 0x7Fu);
                if (MODE == MODE_GEMV) {
                    // bf16 x bf16 is exact in fp32
                    const uint32_t et = gi * 64u + uint32_t(lane);           // e - t * 4096
                    const bool second = et >= rsplit;
                    const float xe = __uint_as_float(uint32_t(a.x[second ? et - rsplit : c_first + et]) << 16);
                    const float p = __uint_as_float(wb << 16) * xe;
                    if (second) acc1 += p;
                    else acc0 += p;
                } else if (MODE == MODE_EXP) {
                    static_cast<uint8_t*>(a.out)[e] = uint8_t(ev);
                } else {
                    static_cast<uint16_t*>(a.out)[e] = uint16_t(wb);
                }
            }
            if (MODE == MODE_GEMV) {
                acc0 = wave_sum(acc0);
                acc1 = wave_sum(acc1);
                if (lane == 0) {
                    float* part = static_cast<float*>(a.out);
                    if (a.C == 4096) {
                        part[t] = acc0;          // tile t is row t: the output itself
                    } else {
                        part[2 * t] = acc0;
                        part[2 * t + 1] = acc1;
                    }
                }
            }
        }
    }
}

// y[r] = sum of the partials of row r over the tiles it spans, in tile order
// (tile t's partial 0 belongs to its first row, partial 1 to the next: a
// tile starting inside row r holds r's elements in partial 0, the one it
// starts in before r holds them in partial 1).
__global__ __launch_bounds__(256) void gemv_rows_reduce(const float* __restrict__ part, int64_t R, int64_t C,
                                                        float* __restrict__ y) {
    const int64_t r = int64_t(blockIdx.x) * 256 + threadIdx.x;
    if (r >= R) return;
    const int64_t first = r * C, t0 = first >> 12, t1 = (first + C - 1) >> 12;
    float s = 0.f;
    // eight loads issued together per round (no load waits for the previous
    // one), then added in tile order
    for (int64_t tb = t0; tb <= t1; tb += 8) {
        float v[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int64_t t = tb + i;
            v[i] = t <= t1 ? part[2 * t + ((t << 12) >= first ? 0 : 1)] : 0.f;
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) s += v[i];
    }
    y[r] = s;
}

}  // namespace

size_t decode_lds_bytes(int lmax, uint32_t max_tile_bytes, int* buf_words) {
    // the longest tile, +1 word for a misaligned start, the lead word, one
    // lookahead word, rounded to whole 16-byte rows
    (void)lmax;
    const int bw = ((int(max_tile_bytes) + 3) / 4 + 3 + 3) & ~3;
    if (buf_words) *buf_words = bw;
    return (size_t(kMlutEntries) + 256 + kTailWords + size_t(kDecWaves) * (bw + 64 * kSlot)) * 4;
}

hipError_t launch_decode(int mode, const DecodeArgs& a0, hipStream_t s) {
    DecodeArgs a = a0;
    const size_t lds = decode_lds_bytes(a.lmax, a.max_tile_bytes, &a.buf_words);
    if (a.T == 0) return hipSuccess;
    // persistent grid: as many workgroups as fit on the chip at once (LDS
    // and 2048 threads per CU), each looping over tiles
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) == hipSuccess) (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    const int per_cu = std::max(1, std::min(2048 / (64 * kDecWaves), int((160u * 1024u) / lds)));
    const int64_t blocks = (a.T + kDecWaves - 1) / kDecWaves;
    const unsigned grid = unsigned(std::max<int64_t>(1, std::min<int64_t>(blocks, int64_t(cus) * per_cu)));
    const dim3 block(64 * kDecWaves);
    switch (mode) {
        case MODE_FULL: decode_kernel<MODE_FULL><<<grid, block, lds, s>>>(a); break;
        case MODE_EXP: decode_kernel<MODE_EXP><<<grid, block, lds, s>>>(a); break;
        case MODE_GEMV: launch_timed(decode_kernel<MODE_GEMV>, dim3(grid), block, lds, s, a); break;
        default: decode_kernel<MODE_PAL><<<grid, block, lds, s>>>(a); break;
    }
    return hipGetLastError();
}

hipError_t launch_decode_gemv(const DecodeArgs& a0, int64_t rows, float* y, hipStream_t s) {
    if (rows == 0) return hipSuccess;
    DecodeArgs a = a0;
    if (a.C == 4096) a.out = y;                 // one row per tile: written directly
    hipError_t e = launch_decode(MODE_GEMV, a, s);
    if (e != hipSuccess || a.C == 4096) return e;
    gemv_rows_reduce<<<unsigned((rows + 255) / 256), 256, 0, s>>>(static_cast<const float*>(a.out), rows, a.C, y);
    return hipGetLastError();
}

}  // namespace uwk
