// Skinny matmul (batch 2..64) on bf16 MFMA with weights rebuilt in the
// A-operand registers, for uncompressed, exponent-source and palette-source
// weights.
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
// Llama matrix runs several thousand wavefronts.  Per step of 128 columns,
// lane l holds 32 consecutive weights of row l%16 (columns 32*(l/16)..+32):
// their compressed bytes are loaded with 16-byte loads, rebuilt to bf16 in
// registers and fed, 8 at a time, as the A operand of four
// v_mfma_f32_16x16x32_bf16.  The K order inside an MFMA is a free
// permutation when A and B agree, so each lane's B fragments are the
// matching 8-element runs of the activation rows, read straight from L2 (the
// activations of a launch are a few hundred KiB and stay cache resident).
// All loads of steps t+1..t+PD are issued before step t is rebuilt (PD + 1
// register sets, no data-dependent branch around a load); the verbatim bitmap words and
// bases of the (at most two) tiles a lane's row segment touches are loaded
// once, so the verbatim flag and slot of every step are register arithmetic
// and a verbatim lane's 32 raw exponents come with the step's other loads.
#include <cstdlib>

#include "device_common.h"
#include "kernels.h"

namespace uwk {

namespace {

constexpr int kKStep = 128;   // columns per wave per step
constexpr int kMaxSlice = 4096;  // columns of one wave's K-slice: its row segment spans <= 2 tiles

__device__ __forceinline__ uint32_t palb(const MatArgs& a, int i) { return pal_byte(a.pal, uint32_t(i)); }

template <int SRC, int NB, int RB, int XQ>
struct Step {
    u32x4_t w[RB][4];   // BF16: 32 weights; EXP: w[.][0..1] = exponents; PAL: w[.][0] = nibbles
    u32x4_t sm[RB][2];  // EXP, PAL: sign/mantissa bytes
    u32x4_t vx[RB][2];  // PAL: verbatim exponents
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
template <int SRC, int NB, int KW, int PD, int RB, int XQ>
__global__ __launch_bounds__(64 * KW) void mfma_gemv_kernel(MatArgs a) {
    static_assert(XQ >= 1 && XQ <= 4 * NB, "activation row quads");
    __shared__ uint32_t lut[256];
    // per-wave activation tiles during the K loop; the K-slices' partial
    // tiles afterwards
    constexpr int kXBytes = KW * NB * 16 * kXS * 2, kPBytes = KW * RB * NB * 64 * 16;
    __shared__ __align__(16) uint8_t smem[kXBytes > kPBytes ? kXBytes : kPBytes];
    auto part = reinterpret_cast<f32x4_t(*)[RB][NB][64]>(smem);
    const int tid = threadIdx.x;
    if (SRC == SRC_PAL)
        for (int i = tid; i < 256; i += 64 * KW) lut[i] = (palb(a, i & 15) << 7) | (palb(a, i >> 4) << 23);
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const uint32_t C = uint32_t(a.C);
    const uint32_t R = uint32_t(a.R);
    const uint32_t row0 = blockIdx.x * (16 * RB);         // first row of this workgroup
    const uint32_t nb0 = blockIdx.y * (NB * 16);          // first batch row of this tile
    const uint32_t B = uint32_t(a.B);
    const uint32_t steps = C / kKStep;
    const uint32_t s_lo = steps * wave / KW, s_hi = steps * (wave + 1) / KW;

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
    uint16_t* const xw = reinterpret_cast<uint16_t*>(smem) + wave * (NB * 16 * kXS);

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

    // Plain (cache-retained) loads: a step reads half of each 128-byte line of
    // the 4-bit plane and the next step the other half.
    auto issue = [&](uint32_t s, Step<SRC, NB, RB, XQ>& st) {
        const uint32_t k = s * kKStep + q * 32;
#pragma unroll
        for (int r = 0; r < RB; ++r) {
            const uint32_t pos = rowc[r] * C + k;
            if (SRC == SRC_BF16) {
#pragma unroll
                for (int i = 0; i < 4; ++i) st.w[r][i] = load16(wb + pos + 8 * i);
            } else if (SRC == SRC_EXP) {
                st.w[r][0] = load16(w8 + pos);
                st.w[r][1] = load16(w8 + pos + 16);
                st.sm[r][0] = load16(a.sm + pos);
                st.sm[r][1] = load16(a.sm + pos + 16);
            } else {
                st.w[r][0] = load16(w8 + pos / 2);
                st.sm[r][0] = load16(a.sm + pos);
                st.sm[r][1] = load16(a.sm + pos + 16);
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
        // stage the activation tile (the previous step's fragment reads are
        // done), then read this step's B fragments: batch row 16n + l%16,
        // the lane's K run
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
                for (int i = 0; i < 16; ++i) w[i] = st.w[r][i >> 2][i & 3];
            } else if (SRC == SRC_EXP) {
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    uint32_t e7[8];
#pragma unroll
                    for (int p = 0; p < 8; ++p)
                        e7[p] = (p & 1) ? exp_pair<1>(st.w[r][h][p >> 1]) : exp_pair<0>(st.w[r][h][p >> 1]);
                    join8(st.sm[r][h], e7, w + 8 * h);
                }
            } else {
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    uint32_t e7[8];
#pragma unroll
                    for (int p = 0; p < 8; ++p) {
                        const uint32_t nbyte = (st.w[r][0][2 * h + (p >> 2)] >> (8 * (p & 3))) & 0xFFu;
                        e7[p] = *reinterpret_cast<const uint32_t*>(reinterpret_cast<const char*>(lut) + (nbyte << 2));
                    }
                    if (__builtin_amdgcn_ballot_w64(st.verb[r] != 0)) {   // rare: raw exponents for verbatim lanes
#pragma unroll
                        for (int p = 0; p < 8; ++p) {
                            const uint32_t er =
                                (p & 1) ? exp_pair<1>(st.vx[r][h][p >> 1]) : exp_pair<0>(st.vx[r][h][p >> 1]);
                            e7[p] = st.verb[r] ? er : e7[p];
                        }
                    }
                    join8(st.sm[r][h], e7, w + 8 * h);
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

// K-split width, prefetch depth and row blocks per wavefront (measured on
// the Llama MLP shapes at batch 2..64; UW_SKINNY_KW / _PD / _RB override for
// tuning).  The slice of one wave must stay within kMaxSlice columns, which
// sets the smallest K-split; two row blocks per wave halve the activation
// traffic but also the number of workgroups, so only tall matrices take them.
Shape choose_shape(const MatArgs& a) {
    const int64_t steps = a.C / kKStep;
    int kw = env_int("UW_SKINNY_KW", 2);
    int pd = env_int("UW_SKINNY_PD", 1);
    int rb = env_int("UW_SKINNY_RB", a.R >= 8192 && a.B <= 32 ? 2 : 1);
    kw = kw <= 2 ? 2 : (kw <= 4 ? 4 : (kw <= 8 ? 8 : 16));
    while (kw < 8 && (steps + kw - 1) / kw * kKStep > kMaxSlice) kw *= 2;
    pd = pd >= 2 ? 2 : 1;
    rb = rb >= 2 ? 2 : 1;
    return {kw, pd, rb};
}

template <int SRC, int NB, int KW, int PD, int RB>
hipError_t launch_shape(const MatArgs& a, hipStream_t s) {
    dim3 grid(unsigned((a.R + 16 * RB - 1) / (16 * RB)), unsigned((a.B + NB * 16 - 1) / (NB * 16)));
    // one 16-row batch tile: load only the row quads the batch fills
    if (NB == 1 && a.B <= 4) launch_timed(mfma_gemv_kernel<SRC, NB, KW, PD, RB, 1>, grid, dim3(64 * KW), 0, s, a);
    else if (NB == 1 && a.B <= 8) launch_timed(mfma_gemv_kernel<SRC, NB, KW, PD, RB, 2>, grid, dim3(64 * KW), 0, s, a);
    else launch_timed(mfma_gemv_kernel<SRC, NB, KW, PD, RB, 4 * NB>, grid, dim3(64 * KW), 0, s, a);
    return hipGetLastError();
}

// Register budget: four batch tiles take one step set and one row block;
// two batch tiles take a third step set or a second row block, not both.
template <int SRC, int NB, int KW>
hipError_t launch_kw(const MatArgs& a, const Shape& sh, hipStream_t s) {
    // sixteen waves per workgroup: one batch tile, one row block, one step set
    // (128 registers at most)
    if constexpr (KW == 16) {
        return launch_shape<SRC, 1, 16, 1, 1>(a, s);
    } else {
        if (NB == 4) return launch_shape<SRC, NB, KW, 1, 1>(a, s);
        constexpr int kNB = NB == 4 ? 1 : NB;             // keeps the instantiations below well formed
        if (sh.rb == 1)
            return sh.pd == 1 ? launch_shape<SRC, kNB, KW, 1, 1>(a, s) : launch_shape<SRC, kNB, KW, 2, 1>(a, s);
        if (NB == 2 || sh.pd == 1) return launch_shape<SRC, kNB, KW, 1, 2>(a, s);
        return launch_shape<SRC, kNB, KW, (NB == 1 ? 2 : 1), 2>(a, s);
    }
}

template <int SRC, int NB>
hipError_t launch_nb(const MatArgs& a, const Shape& sh, hipStream_t s) {
    switch (sh.kw) {
        case 2: return launch_kw<SRC, NB, 2>(a, sh, s);
        case 4: return launch_kw<SRC, NB, 4>(a, sh, s);
        case 8: return launch_kw<SRC, NB, 8>(a, sh, s);
        default:
            if constexpr (NB == 1) return launch_kw<SRC, NB, 16>(a, sh, s);
            else return launch_kw<SRC, NB, 8>(a, sh, s);
    }
}

template <int SRC>
hipError_t launch_src(const MatArgs& a, hipStream_t s) {
    const Shape sh = choose_shape(a);
    if (a.B <= 16) return launch_nb<SRC, 1>(a, sh, s);
    if (a.B <= 32) return launch_nb<SRC, 2>(a, sh, s);
    return launch_nb<SRC, 4>(a, sh, s);
}

}  // namespace

// Supported when the K-slices are whole 128-column steps and, split 8 ways at
// most, each slice spans at most 4096 columns (so a lane's row segment
// touches at most two tiles).
bool mfma_gemv_supported(const MatArgs& a) {
    const int64_t steps = a.C / kKStep;
    return a.C > 0 && a.C % kKStep == 0 && (steps + 7) / 8 * kKStep <= kMaxSlice;
}

hipError_t launch_mfma_gemv(int src, const MatArgs& a, hipStream_t s) {
    if (a.R == 0 || a.B == 0) return hipSuccess;
    switch (src) {
        case SRC_BF16: return launch_src<SRC_BF16>(a, s);
        case SRC_EXP: return launch_src<SRC_EXP>(a, s);
        default: return launch_src<SRC_PAL>(a, s);
    }
}

}  // namespace uwk
