// Skinny matmul (batch 2..64) on bf16 MFMA with weights rebuilt in the
// A-operand registers, for uncompressed, exponent-source and palette-source
// weights, and the gate/up pair of an MLP block with the SiLU product in the
// epilogue (palette source, batch up to 16).
//
// Method: Cloudflare, "Unweight: how we compressed an LLM 22% without
// sacrificing quality", "How the reconstructive matmul works": compressed
// weights go from HBM straight into on-chip reconstruction and from there into
// the matrix units; rebuilt weights never reach device memory.
//
// Mapping to CDNA4.  At small batch the matmul is still bound by the weight
// stream, so the kernel is laid out for parallelism and coalescing rather
// than reuse: a wavefront owns 16 weight rows and one K-slice (the 2, 4 or 8
// wavefronts of a workgroup split K and sum their partial tiles in LDS), so a
// Llama matrix runs thousands of wavefronts.  Per step of 128 columns, lane
// l feeds row l%16 and columns 32*(l/16)..+32 into four
// v_mfma_f32_16x16x32_bf16 (the K order inside an MFMA is a free permutation
// when A and B agree, so each lane's B fragments are the matching 8-element
// runs of the activation rows).
//   Loads.  That operand layout puts consecutive lanes on consecutive rows,
// and a 16-byte load whose lanes sit in different rows costs the L1 one
// access per lane: loaded that way, the weight planes and the activation
// fragments kept the L1 saturated (measured on MI355X at batch 16: the
// address unit stalled on it most of the kernel).  So every plane of a step
// is loaded as contiguous row runs (a 128-byte sign/mantissa row by 8 lanes
// side by side, the 4-bit row by 4, the activation rows by 16) into
// registers, written to a wave-private LDS region and read back in the MFMA
// layout, first the weight planes, then the activation tile over the same
// region; only the activation rows the batch fills are loaded.  The weights
// are rebuilt to bf16 in registers from there.  All loads of steps
// t+1..t+PD are issued before step t is rebuilt (PD + 1 register sets, no
// data-dependent branch around a load); the verbatim bitmap words and bases
// of the (at most two) tiles a lane's row segment touches are loaded once, so
// the verbatim flag and slot of every step are register arithmetic, and a
// verbatim lane's 32 raw exponents come with the step's other loads.
#include <cstdlib>

#include "device_common.h"
#include "kernels.h"

namespace uwk {

namespace {

constexpr int kKStep = 128;   // columns per wave per step
constexpr int kMaxSlice = 4096;  // columns of one wave's K-slice: its row segment spans <= 2 tiles

__device__ __forceinline__ uint32_t palb(const MatArgs& a, int i) { return pal_byte(a.pal, uint32_t(i)); }

// Weight planes of a source, each staged per step as 16 rows x bpr bytes:
// bf16 (256 bytes a row); exponents (128) + sign/mantissa (128); 4-bit
// indices (64) + sign/mantissa (128).
template <int SRC>
struct Planes {
    static constexpr int n = SRC == SRC_BF16 ? 1 : 2;
    static constexpr int bpr0 = SRC == SRC_BF16 ? 256 : (SRC == SRC_EXP ? 128 : 64);
    static constexpr int bpr1 = 128;
    static constexpr int pieces = (bpr0 + (n > 1 ? bpr1 : 0)) / 64;   // 16-byte loads per lane and row block
    // LDS bytes of one row block's planes (rows padded by 16 bytes)
    static constexpr int bytes = 16 * (bpr0 + 16) + (n > 1 ? 16 * (bpr1 + 16) : 0);
};

template <int SRC, int NB, int RB, int XQ>
struct Step {
    u32x4_t w[RB][Planes<SRC>::pieces];   // weight planes, contiguous row runs (not the MFMA layout)
    u32x4_t vx[RB][2];  // PAL: verbatim exponents (MFMA layout)
    uint32_t verb[RB];  // PAL
    u32x4_t x[XQ];      // the wave's activation tile, 16 contiguous bytes per lane and load
};

// A wave's activation tile in LDS: NB*16 batch rows x one step of columns,
// rows padded by 16 bytes (conflict-free 16-byte fragment reads and writes).
constexpr int kXS = kKStep + 8;

// Orders a wave's LDS writes before its (cross-lane) reads and vice versa.
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// 8 rebuilt bf16 pairs (16 weights) from 16 sign/mantissa bytes and exponents.
__device__ __forceinline__ void join8(const u32x4_t& sm, const uint32_t e7[8], uint32_t out[8]) {
#pragma unroll
    for (int p = 0; p < 8; ++p) out[p] = (p & 1) ? join_pair<1>(sm[p >> 1], e7[p]) : join_pair<0>(sm[p >> 1], e7[p]);
}

// KW wavefronts per workgroup split K; a wavefront owns RB blocks of 16 rows
// (sharing the activation fragments); PD steps of loads are kept in flight
// ahead of the step being rebuilt (PD + 1 register sets).
// XQ: quads of activation rows loaded per step (4*NB, or fewer when the
// batch leaves the rest of the 16-row tile empty).
// DUAL (palette source, one row block, one batch block): the gate/up pair of
// a SwiGLU MLP.  The workgroup holds 2*KW waves, the first KW on rows of the
// gate matrix (a0), the others on the same rows of the up matrix, each wave
// exactly as in a launch of its own matrix; the epilogue sums each matrix's
// K-slices in the same order and writes H[b][r] = bf16(SiLU(g) * u), and g
// and u themselves when a0.Y / up.Y are not null.
template <int SRC, int NB, int KW, int PD, int RB, int XQ, bool DUAL>
__global__ __launch_bounds__(64 * KW * (DUAL ? 2 : 1)) void mfma_gemv_kernel(MatArgs a0, MatArgs up, uint16_t* H) {
    static_assert(XQ >= 1 && XQ <= 4 * NB, "activation row quads");
    static_assert(!DUAL || (SRC == SRC_PAL && RB == 1 && NB == 1), "gate/up pair");
    constexpr int NW = KW * (DUAL ? 2 : 1);                 // waves per workgroup
    __shared__ uint32_t lut[DUAL ? 512 : 256];
    // a region per wave during the K loop, holding a step's weight planes and
    // then its activation tile; the K-slices' partial tiles afterwards
    using PL = Planes<SRC>;
    constexpr int kWBytes = RB * PL::bytes, kXTBytes = NB * 16 * kXS * 2;
    constexpr int kRegion = kWBytes > kXTBytes ? kWBytes : kXTBytes;
    constexpr int kXBytes = NW * kRegion, kPBytes = NW * RB * NB * 64 * 16;
    static_assert(kXBytes <= 150 * 1024 && kPBytes <= 150 * 1024, "LDS");
    __shared__ __align__(16) uint8_t smem[kXBytes > kPBytes ? kXBytes : kPBytes];
    auto part = reinterpret_cast<f32x4_t(*)[RB][NB][64]>(smem);
    const int tid = threadIdx.x;
    if (SRC == SRC_PAL)
        for (int i = tid; i < 256; i += 64 * NW) {
            lut[i] = (palb(a0, i & 15) << 7) | (palb(a0, i >> 4) << 23);
            if (DUAL) lut[256 + i] = (palb(up, i & 15) << 7) | (palb(up, i >> 4) << 23);
        }
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    // DUAL: the matrix of this wave (uniform) and its place in that matrix's K-split
    const int mi = DUAL ? wave / KW : 0, kwi = DUAL ? wave % KW : wave;
    const MatArgs& a = (DUAL && mi) ? up : a0;
    const uint32_t* const lutm = lut + (DUAL ? 256 * mi : 0);
    const uint32_t C = uint32_t(a.C);
    const uint32_t R = uint32_t(a.R);
    const uint32_t row0 = blockIdx.x * (16 * RB);         // first row of this workgroup
    const uint32_t nb0 = blockIdx.y * (NB * 16);          // first batch row of this tile
    const uint32_t B = uint32_t(a.B);
    const uint32_t steps = C / kKStep;
    const uint32_t s_lo = steps * kwi / KW, s_hi = steps * (kwi + 1) / KW;

    const uint32_t q = uint32_t(lane) >> 4, rl = uint32_t(lane) & 15u;
    uint32_t rowc[RB];                                    // rows past R read row 0; never stored
#pragma unroll
    for (int r = 0; r < RB; ++r) {
        const uint32_t row = row0 + 16 * r + rl;
        rowc[r] = row < R ? row : 0u;
    }
    // activation rows of the lane's tile loads (piece j: row 4j + q, 16 bytes
    // at column 8*(lane%16)); rows past the batch read row 0, their output
    // columns are never stored
    uint32_t xrow[XQ];
#pragma unroll
    for (int j = 0; j < XQ; ++j) {
        const uint32_t b = nb0 + 4 * j + q;
        xrow[j] = b < B ? b : 0u;
    }
    uint8_t* const region = smem + wave * kRegion;
    uint16_t* const xw = reinterpret_cast<uint16_t*>(region);

    // verbatim tables of the (at most two) tiles each row segment touches
    uint64_t word0[RB], word1[RB];
    uint32_t vb0[RB], vb1[RB], t0[RB];
#pragma unroll
    for (int r = 0; r < RB; ++r) {
        word0[r] = word1[r] = 0;
        vb0[r] = vb1[r] = t0[r] = 0;
        if (SRC == SRC_PAL && s_lo < s_hi) {
            const uint32_t p0 = rowc[r] * C + s_lo * kKStep, p1 = rowc[r] * C + s_hi * kKStep - 1;
            t0[r] = p0 >> 12;
            const uint32_t t1 = p1 >> 12;
            word0[r] = a.bitmap[t0[r]];
            vb0[r] = a.tile_vbase[t0[r]];
            word1[r] = a.bitmap[t1];
            vb1[r] = a.tile_vbase[t1];
        }
    }
    const uint8_t* vb_ptr = a.vexp ? a.vexp : a.sm;
    const uint16_t* wb = static_cast<const uint16_t*>(a.w);
    const uint8_t* w8 = static_cast<const uint8_t*>(a.w);

    // The weight planes of a step go out as contiguous runs of each row (the
    // MFMA layout puts consecutive lanes on consecutive rows, which would cost
    // an L1 access per lane): a plane row of bpr bytes is loaded by bpr/16
    // neighbouring lanes, 16 bytes each, piece i covering rows
    // 64i/(bpr/16).. of the block.  Plain (cache-retained) loads.
    const uint8_t* const plane0 = SRC == SRC_BF16 ? reinterpret_cast<const uint8_t*>(wb) : w8;
    auto plane_piece = [&](const uint8_t* base, int bpr, int r, int i, uint32_t s) {
        const uint32_t p = uint32_t(i) * 64u + uint32_t(lane), cpr = uint32_t(bpr) / 16u;
        const uint32_t row = p / cpr, chunk = p % cpr;
        uint32_t rowg = row0 + 16u * uint32_t(r) + row;
        rowg = rowg < R ? rowg : 0u;
        return load16(base + uint64_t(rowg) * (uint64_t(bpr) * C / kKStep) + uint64_t(s) * bpr + chunk * 16u);
    };
    auto issue = [&](uint32_t s, Step<SRC, NB, RB, XQ>& st) {
        const uint32_t k = s * kKStep + q * 32;
#pragma unroll
        for (int r = 0; r < RB; ++r) {
#pragma unroll
            for (int i = 0; i < PL::bpr0 / 64; ++i) st.w[r][i] = plane_piece(plane0, PL::bpr0, r, i, s);
            if (PL::n > 1) {
#pragma unroll
                for (int i = 0; i < PL::bpr1 / 64; ++i)
                    st.w[r][PL::bpr0 / 64 + i] = plane_piece(a.sm, PL::bpr1, r, i, s);
            }
            if (SRC == SRC_PAL) {
                const uint32_t pos = rowc[r] * C + k;
                const bool second = (pos >> 12) != t0[r];
                const uint64_t word = second ? word1[r] : word0[r];
                const uint32_t vbase = second ? vb1[r] : vb0[r];
                const uint32_t bit = (pos >> 6) & 63u;
                st.verb[r] = uint32_t(word >> bit) & 1u;
                const uint32_t slot = verbatim_slot(word, bit, vbase);
                const uint32_t voff = st.verb[r] ? slot * 64u + (pos & 63u) : 0u;
                st.vx[r][0] = load16(vb_ptr + voff);
                st.vx[r][1] = load16(vb_ptr + voff + 16);
            }
        }
        // the activation tile of the step: XQ quads of rows x 256 contiguous
        // bytes (quads past the batch are not loaded: their output columns
        // are never stored)
#pragma unroll
        for (int j = 0; j < XQ; ++j) st.x[j] = load16(a.X + xrow[j] * C + s * kKStep + 8 * rl);
        // keep every load of the step here: the scheduler must not sink one
        // into a later rebuild, whose wait would then cover it
        __builtin_amdgcn_sched_barrier(0);
    };

    f32x4_t acc[RB][NB];
#pragma unroll
    for (int r = 0; r < RB; ++r)
#pragma unroll
        for (int n = 0; n < NB; ++n) acc[r][n] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    auto compute = [&](const Step<SRC, NB, RB, XQ>& st) {
        // the weight planes through the wave's region (the previous step's
        // reads of it are done), read back in the MFMA layout: lane l, row
        // l%16, the lane's run of 32 weights
        wave_lds_sync();
#pragma unroll
        for (int r = 0; r < RB; ++r) {
            uint8_t* const rb = region + r * PL::bytes;
#pragma unroll
            for (int i = 0; i < PL::pieces; ++i) {
                const bool p1 = i >= PL::bpr0 / 64;
                const int bpr = p1 ? PL::bpr1 : PL::bpr0;
                const uint32_t pp = uint32_t(p1 ? i - PL::bpr0 / 64 : i) * 64u + uint32_t(lane);
                const uint32_t cpr = uint32_t(bpr) / 16u;
                uint8_t* const dst = rb + (p1 ? 16 * (PL::bpr0 + 16) : 0) + (pp / cpr) * (bpr + 16) + (pp % cpr) * 16u;
                *reinterpret_cast<u32x4_t*>(dst) = st.w[r][i];
            }
        }
        wave_lds_sync();
        u32x4_t wl[RB][4], sml[RB][2];
#pragma unroll
        for (int r = 0; r < RB; ++r) {
            const uint8_t* const rb = region + r * PL::bytes;
            if (SRC == SRC_BF16) {
#pragma unroll
                for (int j = 0; j < 4; ++j) wl[r][j] = *reinterpret_cast<const u32x4_t*>(rb + rl * 272u + 64u * q + 16u * j);
            } else {
                const uint8_t* const p1 = rb + 16 * (PL::bpr0 + 16);
                if (SRC == SRC_EXP) {
#pragma unroll
                    for (int j = 0; j < 2; ++j) wl[r][j] = *reinterpret_cast<const u32x4_t*>(rb + rl * 144u + 32u * q + 16u * j);
                } else {
                    wl[r][0] = *reinterpret_cast<const u32x4_t*>(rb + rl * 80u + 16u * q);
                }
#pragma unroll
                for (int j = 0; j < 2; ++j) sml[r][j] = *reinterpret_cast<const u32x4_t*>(p1 + rl * 144u + 32u * q + 16u * j);
            }
        }
        // then the activation tile over the same region, and this step's B
        // fragments: batch row 16n + l%16, the lane's K run
        wave_lds_sync();
#pragma unroll
        for (int j = 0; j < XQ; ++j) *reinterpret_cast<u32x4_t*>(xw + (4 * j + q) * kXS + 8 * rl) = st.x[j];
        wave_lds_sync();
        u32x4_t xf[4][NB];
#pragma unroll
        for (int sub = 0; sub < 4; ++sub)
#pragma unroll
            for (int n = 0; n < NB; ++n)
                xf[sub][n] = *reinterpret_cast<const u32x4_t*>(xw + (16 * n + rl) * kXS + 32 * q + 8 * sub);
#pragma unroll
        for (int r = 0; r < RB; ++r) {
            uint32_t w[16];   // 32 weights as bf16 pairs
            if (SRC == SRC_BF16) {
#pragma unroll
                for (int i = 0; i < 16; ++i) w[i] = wl[r][i >> 2][i & 3];
            } else if (SRC == SRC_EXP) {
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    uint32_t e7[8];
#pragma unroll
                    for (int p = 0; p < 8; ++p)
                        e7[p] = (p & 1) ? exp_pair<1>(wl[r][h][p >> 1]) : exp_pair<0>(wl[r][h][p >> 1]);
                    join8(sml[r][h], e7, w + 8 * h);
                }
            } else {
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    uint32_t e7[8];
#pragma unroll
                    for (int p = 0; p < 8; ++p) {
                        const uint32_t nbyte = (wl[r][0][2 * h + (p >> 2)] >> (8 * (p & 3))) & 0xFFu;
                        e7[p] = *reinterpret_cast<const uint32_t*>(reinterpret_cast<const char*>(lutm) + (nbyte << 2));
                    }
                    if (st.verb[r]) {   // a verbatim lane: raw exponents, under its own exec mask
#pragma unroll
                        for (int p = 0; p < 8; ++p)
                            e7[p] = (p & 1) ? exp_pair<1>(st.vx[r][h][p >> 1]) : exp_pair<0>(st.vx[r][h][p >> 1]);
                    }
                    join8(sml[r][h], e7, w + 8 * h);
                }
            }
#pragma unroll
            for (int sub = 0; sub < 4; ++sub) {
                const bf16x8_t A = __builtin_bit_cast(bf16x8_t, u32x4_t{w[4 * sub], w[4 * sub + 1], w[4 * sub + 2],
                                                                        w[4 * sub + 3]});
#pragma unroll
                for (int n = 0; n < NB; ++n)
                    acc[r][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, __builtin_bit_cast(bf16x8_t, xf[sub][n]),
                                                                        acc[r][n], 0, 0, 0);
            }
        }
    };

    __syncthreads();                                      // LUT ready
    // Steps past the slice re-issue its last step, so no load is conditional.
    // Each loop body holds all its steps with no exit between them (the 0..PD
    // steps left over are computed after the loop): a mid-body exit lets the
    // compiler fold identical step bodies into one with register copies,
    // which must wait for every load in flight.
    if (s_lo < s_hi) {
        const uint32_t last = s_hi - 1;
        uint32_t s = s_lo;
        if (PD == 1) {
            Step<SRC, NB, RB, XQ> s0, s1;
            issue(s_lo, s0);
            for (; s + 1 < s_hi; s += 2) {
                issue(s + 1, s1);
                compute(s0);
                issue(min(s + 2, last), s0);
                compute(s1);
            }
            if (s < s_hi) compute(s0);
        } else {
            Step<SRC, NB, RB, XQ> s0, s1, s2;
            issue(s_lo, s0);
            issue(min(s_lo + 1, last), s1);
            for (; s + 2 < s_hi; s += 3) {
                issue(s + 2, s2);
                compute(s0);
                issue(min(s + 3, last), s0);
                compute(s1);
                issue(min(s + 4, last), s1);
                compute(s2);
            }
            if (s < s_hi) compute(s0);
            if (s + 1 < s_hi) compute(s1);
        }
    }
    // sum the K-slices (their tiles overlay the activation tiles: every wave
    // is done with its own first): D layout, lane l holds batch column l%16,
    // rows 4*(l/16)..+3
    __syncthreads();
#pragma unroll
    for (int r = 0; r < RB; ++r)
#pragma unroll
        for (int n = 0; n < NB; ++n) part[wave][r][n][lane] = acc[r][n];
    __syncthreads();
    if (DUAL) {
        for (int idx = tid; idx < NB * 64; idx += 64 * NW) {
            const int n = idx / 64, l = idx % 64;
            f32x4_t g = part[0][0][n][l], u = part[KW][0][n][l];
#pragma unroll
            for (int w_ = 1; w_ < KW; ++w_) {
                g += part[w_][0][n][l];
                u += part[KW + w_][0][n][l];
            }
            const uint32_t b = nb0 + n * 16 + (l & 15);
            const uint32_t rr = row0 + 4 * (l >> 4);
            if (b < B) {
                const int64_t o = int64_t(b) * a0.R + rr;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    if (rr + i < R) {
                        if (a0.Y) a0.Y[o + i] = g[i];
                        if (up.Y) up.Y[o + i] = u[i];
                        H[o + i] = uint16_t(f32_to_bf16_rne(silu_mul1(g[i], u[i])));
                    }
                }
            }
        }
        return;
    }
    for (int idx = tid; idx < RB * NB * 64; idx += 64 * KW) {
        const int r = idx / (NB * 64), n = (idx / 64) % NB, l = idx % 64;
        f32x4_t v = part[0][r][n][l];
#pragma unroll
        for (int w_ = 1; w_ < KW; ++w_) v += part[w_][r][n][l];
        const uint32_t b = nb0 + n * 16 + (l & 15);
        const uint32_t rr = row0 + 16 * r + 4 * (l >> 4);
        if (b < B) {
            float* o = a.Y + int64_t(b) * a.R + rr;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (rr + i < R) o[i] = v[i];
        }
    }
}

struct Shape {
    int kw, pd, rb;
};

int env_int(const char* name, int dflt) {
    const char* e = getenv(name);
    return e && *e ? atoi(e) : dflt;
}

// K-split width, prefetch depth and row blocks per wavefront, as measured on
// the Llama MLP and attention shapes at batch 2..16 (UW_SKINNY_KW / _PD / _RB
// override for tuning).  The K-split is the smallest that gives about one
// 16-row block per SIMD (a 14336-row matrix: 2; 4096 rows: 4; 1024 rows: 8;
// blocks, not waves: with two blocks per wave, gate at batch 24 and 32 runs
// 24.7 and 25.7 us at split 2 against 28.7 and 29.5 us at split 4), and at
// least what keeps one wave's slice within kMaxSlice columns.  One row
// block per wave up to batch 16 (with the tiles staged through LDS a second
// block saves little activation traffic and halves the workgroups), two on
// tall matrices above (gate at batch 32: 29.6 against 30.8 us) and from
// batch 5 on matrices of 32768 rows or more, where halving the workgroups
// still leaves many per CU and each wave re-reads the activation tile for
// fewer rows (the 128256-row output projection at batch 16: 168.5 against
// 191.8 us).  Two steps in flight for long slices (>= 24 steps) at batch <= 8.
Shape choose_shape(const MatArgs& a) {
    const int64_t steps = a.C / kKStep;
    const bool two_blocks = (a.B > 16 && a.R >= 8192) || (a.B > 4 && a.R >= 32768);
    int rb = env_int("UW_SKINNY_RB", two_blocks ? 2 : 1);
    const int kw_env = env_int("UW_SKINNY_KW", 0);
    int kw = kw_env;
    if (kw <= 0) {
        const int64_t simds = 4 * int64_t(a.cus > 0 ? a.cus : 256);
        const int64_t waves_per_kw = (a.R + 16 * rb - 1) / (16 * rb) * ((a.B + 63) / 64);
        kw = 2;
        while (kw < 8 && waves_per_kw * rb * kw < simds) kw *= 2;
    }
    kw = kw <= 2 ? 2 : (kw <= 4 ? 4 : 8);
    while (kw < 8 && (steps + kw - 1) / kw * kKStep > kMaxSlice) kw *= 2;
    int pd = env_int("UW_SKINNY_PD", a.B <= 8 && steps / kw >= 24 ? 2 : 1);
    pd = pd >= 2 ? 2 : 1;
    rb = rb >= 2 ? 2 : 1;
    return {kw, pd, rb};
}

template <int SRC, int NB, int KW, int PD, int RB, bool DUAL = false>
hipError_t launch_shape(const MatArgs& a, hipStream_t s, const MatArgs& up = MatArgs{}, uint16_t* h = nullptr) {
    dim3 grid(unsigned((a.R + 16 * RB - 1) / (16 * RB)), unsigned((a.B + NB * 16 - 1) / (NB * 16)));
    const dim3 block(64 * KW * (DUAL ? 2 : 1));
    // one 16-row batch tile: load only the row quads the batch fills
    if constexpr (NB == 1) {
        if (a.B <= 4) launch_timed(mfma_gemv_kernel<SRC, NB, KW, PD, RB, 1, DUAL>, grid, block, 0, s, a, up, h);
        else if (a.B <= 8) launch_timed(mfma_gemv_kernel<SRC, NB, KW, PD, RB, 2, DUAL>, grid, block, 0, s, a, up, h);
        else launch_timed(mfma_gemv_kernel<SRC, NB, KW, PD, RB, 4, DUAL>, grid, block, 0, s, a, up, h);
    } else {
        launch_timed(mfma_gemv_kernel<SRC, NB, KW, PD, RB, 4 * NB, false>, grid, block, 0, s, a, up, h);
    }
    return hipGetLastError();
}

// Register budget (a workgroup of KW waves must fit one CU: 8 waves leave
// 256 registers a wave): four batch tiles take one step set and one row
// block, and at most four waves; two batch tiles take a third step set or a
// second row block, not both; eight waves take one step set, and a second
// row block only with one batch tile.
template <int SRC, int NB, int KW>
hipError_t launch_kw(const MatArgs& a, const Shape& sh, hipStream_t s) {
    if constexpr (NB == 4) {
        return launch_shape<SRC, 4, KW, 1, 1>(a, s);
    } else if constexpr (KW == 8) {
        if (NB == 1 && sh.rb == 2) return launch_shape<SRC, 1, 8, 1, 2>(a, s);
        return launch_shape<SRC, NB, 8, 1, 1>(a, s);
    } else {
        if (sh.rb == 1)
            return sh.pd == 1 ? launch_shape<SRC, NB, KW, 1, 1>(a, s) : launch_shape<SRC, NB, KW, 2, 1>(a, s);
        if (NB == 2 || sh.pd == 1) return launch_shape<SRC, NB, KW, 1, 2>(a, s);
        return launch_shape<SRC, NB, KW, (NB == 1 ? 2 : 1), 2>(a, s);
    }
}

template <int SRC, int NB>
hipError_t launch_nb(const MatArgs& a, const Shape& sh, hipStream_t s) {
    switch (sh.kw) {
        case 2: return launch_kw<SRC, NB, 2>(a, sh, s);
        case 4: return launch_kw<SRC, NB, 4>(a, sh, s);
        default:
            if constexpr (NB == 4) return hipErrorNotSupported;   // never chosen: see launch_src
            else return launch_kw<SRC, NB, 8>(a, sh, s);
    }
}

template <int SRC>
hipError_t launch_src(const MatArgs& a, hipStream_t s) {
    const Shape sh = choose_shape(a);
    if (a.B <= 16) return launch_nb<SRC, 1>(a, sh, s);
    // 64-column batch tiles at most four waves wide; 32-column ones otherwise
    if (a.B <= 32 || sh.kw > 4) return launch_nb<SRC, 2>(a, sh, s);
    return launch_nb<SRC, 4>(a, sh, s);
}

}  // namespace

// Supported when the K-slices are whole 128-column steps and, split 8 ways at
// most, each slice spans at most 4096 columns (so a lane's row segment
// touches at most two tiles).
// Gate/up pair (palette sources): the LDS-DMA kernel's pair where the
// library prefers it (batch 3-32 on tall matrices); else this kernel's pair:
// batch <= 16 (above it the separate launches take two row blocks per wave
// on tall matrices and measured faster than this pair: Llama gate/up at
// batch 32, 61.8 against 67.9 us), and the K-split the library takes for one
// of the matrices at most 4 (so a workgroup holds at most 8 waves; small
// matrices that split 8 ways are left to separate launches).
namespace {
bool staged_pair_supported(const MatArgs& g, const MatArgs& u) {
    return g.R == u.R && g.C == u.C && g.B == u.B && g.B >= 1 && g.B <= 16 && g.C > 0 && g.C % kKStep == 0 &&
           mfma_gemv_supported(g) && choose_shape(g).kw <= 4;
}
}  // namespace

bool mfma_gemv_gateup_supported(const MatArgs& g, const MatArgs& u) {
    if (g.R == u.R && g.C == u.C && g.B == u.B && skinny_dma_pair_preferred(g)) return true;   // the DMA pair
    return staged_pair_supported(g, u);
}

// This kernel's pair splits K as the library does for one of its matrices,
// so its g and u equal what separate launches of this kernel give, bit for
// bit; the DMA pair likewise equals single launches of the DMA kernel.
hipError_t launch_mfma_gemv_gateup(const MatArgs& g, const MatArgs& u, uint16_t* h, hipStream_t s) {
    if (g.R == 0) return hipSuccess;
    if (skinny_dma_pair_preferred(g)) {
        const hipError_t e = launch_skinny_dma_gateup(g, u, h, s);
        if (e != hipErrorNotSupported) return e;
    }
    if (!staged_pair_supported(g, u)) return hipErrorNotSupported;
    const Shape sh = choose_shape(g);
    const int kw = sh.kw;
    if (kw <= 2)
        return sh.pd == 1 ? launch_shape<SRC_PAL, 1, 2, 1, 1, true>(g, s, u, h)
                          : launch_shape<SRC_PAL, 1, 2, 2, 1, true>(g, s, u, h);
    return sh.pd == 1 ? launch_shape<SRC_PAL, 1, 4, 1, 1, true>(g, s, u, h)
                      : launch_shape<SRC_PAL, 1, 4, 2, 1, true>(g, s, u, h);
}

bool mfma_gemv_supported(const MatArgs& a) {
    const int64_t steps = a.C / kKStep;
    return a.C > 0 && a.C % kKStep == 0 && (steps + 7) / 8 * kKStep <= kMaxSlice;
}

hipError_t launch_mfma_gemv(int src, const MatArgs& a, hipStream_t s) {
    if (a.R == 0 || a.B == 0) return hipSuccess;
    if (src == SRC_PAL && skinny_dma_forced() && skinny_dma_supported(a)) {
        const hipError_t e = launch_skinny_dma(a, s);
        if (e != hipErrorNotSupported) return e;
    }
    switch (src) {
        case SRC_BF16: return launch_src<SRC_BF16>(a, s);
        case SRC_EXP: return launch_src<SRC_EXP>(a, s);
        default: return launch_src<SRC_PAL>(a, s);
    }
}

}  // namespace uwk
