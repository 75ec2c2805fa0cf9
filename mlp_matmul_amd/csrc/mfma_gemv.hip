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
// than reuse: a wavefront owns 16 weight rows and one K-slice (the four
// wavefronts of a workgroup split K and sum their partial tiles in LDS), so a
// Llama matrix runs several thousand wavefronts.  Per step of 128 columns,
// lane l holds 32 consecutive weights of row l%16 (columns 32*(l/16)..+32):
// their compressed bytes are loaded with 16-byte loads, rebuilt to bf16 in
// registers and fed, 8 at a time, as the A operand of four
// v_mfma_f32_16x16x32_bf16.  The K order inside an MFMA is a free
// permutation when A and B agree, so each lane's B fragments are the
// matching 8-element runs of the activation rows, read straight from L2 (the
// activations of a launch are a few hundred KiB and stay cache resident).
// All loads of step t+1 are issued before step t is rebuilt (two register
// sets, no data-dependent branch around a load); the verbatim bitmap words and
// bases of the (at most two) tiles a lane's row segment touches are loaded
// once, so the verbatim flag and slot of every step are register arithmetic
// and a verbatim lane's 32 raw exponents come with the step's other loads.
#include <cstdlib>

#include "device_common.h"
#include "kernels.h"

namespace uwk {

namespace {

constexpr int kKStep = 128;   // columns per wave per step
constexpr int kKW = 4;        // wavefronts per workgroup, each a K-slice

__device__ __forceinline__ uint32_t palb(const MatArgs& a, int i) {
    return (a.pal[i >> 2] >> (8 * (i & 3))) & 0xFFu;
}

template <int SRC, int NB>
struct Step {
    u32x4_t w[4];       // BF16: 32 weights; EXP: w[0..1] = exponents; PAL: w[0] = nibbles
    u32x4_t sm[2];      // EXP, PAL: sign/mantissa bytes
    u32x4_t vx[2];      // PAL: verbatim exponents
    uint32_t verb;      // PAL
    u32x4_t x[4][NB];   // B fragments: substep s, 16-column block nb
};

// 8 rebuilt bf16 pairs (16 weights) from 16 sign/mantissa bytes and exponents.
__device__ __forceinline__ void join8(const u32x4_t& sm, const uint32_t e7[8], uint32_t out[8]) {
#pragma unroll
    for (int p = 0; p < 8; ++p) out[p] = (p & 1) ? join_pair<1>(sm[p >> 1], e7[p]) : join_pair<0>(sm[p >> 1], e7[p]);
}

template <int SRC, int NB>
__global__ __launch_bounds__(256) void mfma_gemv_kernel(MatArgs a) {
    __shared__ uint32_t lut[256];
    __shared__ f32x4_t part[kKW][NB][64];
    const int tid = threadIdx.x;
    if (SRC == SRC_PAL) lut[tid] = (palb(a, tid & 15) << 7) | (palb(a, tid >> 4) << 23);
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const uint32_t C = uint32_t(a.C);
    const uint32_t rb = blockIdx.x;                       // 16-row block
    const uint32_t nb0 = blockIdx.y * (NB * 16);          // first batch row of this tile
    const int B = int(a.B);
    const uint32_t steps = C / kKStep;
    const uint32_t s_lo = steps * wave / kKW, s_hi = steps * (wave + 1) / kKW;

    const uint32_t q = uint32_t(lane) >> 4, rl = uint32_t(lane) & 15u;
    const uint32_t row = rb * 16 + rl;
    const bool row_ok = row < uint32_t(a.R);
    const uint32_t rowc = row_ok ? row : 0u;              // rows past R read row 0; never stored
    // B rows past the batch read row 0; their output columns are never stored
    uint32_t xrow[NB];
#pragma unroll
    for (int n = 0; n < NB; ++n) {
        const uint32_t b = nb0 + n * 16 + rl;
        xrow[n] = b < uint32_t(B) ? b : 0u;
    }

    // verbatim tables of the (at most two) tiles this lane's row segment touches
    uint64_t word0 = 0, word1 = 0;
    uint32_t vb0 = 0, vb1 = 0, t0 = 0;
    if (SRC == SRC_PAL && s_lo < s_hi) {
        const uint32_t p0 = rowc * C + s_lo * kKStep, p1 = rowc * C + s_hi * kKStep - 1;
        t0 = p0 >> 12;
        const uint32_t t1 = p1 >> 12;
        word0 = a.bitmap[t0];
        vb0 = a.tile_vbase[t0];
        word1 = a.bitmap[t1];
        vb1 = a.tile_vbase[t1];
    }
    const uint8_t* vb_ptr = a.vexp ? a.vexp : a.sm;
    const uint16_t* wb = static_cast<const uint16_t*>(a.w);
    const uint8_t* w8 = static_cast<const uint8_t*>(a.w);

    auto issue = [&](uint32_t s, Step<SRC, NB>& st) {
        const uint32_t k = s * kKStep + q * 32;
        const uint32_t pos = rowc * C + k;
        if (SRC == SRC_BF16) {
#pragma unroll
            for (int i = 0; i < 4; ++i) st.w[i] = load_stream16(wb + pos + 8 * i);
        } else if (SRC == SRC_EXP) {
            st.w[0] = load_stream16(w8 + pos);
            st.w[1] = load_stream16(w8 + pos + 16);
            st.sm[0] = load_stream16(a.sm + pos);
            st.sm[1] = load_stream16(a.sm + pos + 16);
        } else {
            st.w[0] = load_stream16(w8 + pos / 2);
            st.sm[0] = load_stream16(a.sm + pos);
            st.sm[1] = load_stream16(a.sm + pos + 16);
            const bool second = (pos >> 12) != t0;
            const uint64_t word = second ? word1 : word0;
            const uint32_t vbase = second ? vb1 : vb0;
            const uint32_t bit = (pos >> 6) & 63u;
            st.verb = uint32_t(word >> bit) & 1u;
            const uint32_t slot = verbatim_slot(word, bit, vbase);
            const uint32_t voff = st.verb ? slot * 64u + (pos & 63u) : 0u;
            st.vx[0] = load16(vb_ptr + voff);
            st.vx[1] = load16(vb_ptr + voff + 16);
        }
#pragma unroll
        for (int sub = 0; sub < 4; ++sub)
#pragma unroll
            for (int n = 0; n < NB; ++n) st.x[sub][n] = load16(a.X + xrow[n] * C + k + 8 * sub);
    };

    f32x4_t acc[NB];
#pragma unroll
    for (int n = 0; n < NB; ++n) acc[n] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    auto compute = [&](const Step<SRC, NB>& st) {
        uint32_t w[16];   // 32 weights as bf16 pairs
        if (SRC == SRC_BF16) {
#pragma unroll
            for (int i = 0; i < 16; ++i) w[i] = st.w[i >> 2][i & 3];
        } else if (SRC == SRC_EXP) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                uint32_t e7[8];
#pragma unroll
                for (int p = 0; p < 8; ++p) e7[p] = (p & 1) ? exp_pair<1>(st.w[h][p >> 1]) : exp_pair<0>(st.w[h][p >> 1]);
                join8(st.sm[h], e7, w + 8 * h);
            }
        } else {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                uint32_t e7[8];
#pragma unroll
                for (int p = 0; p < 8; ++p) {
                    const uint32_t nbyte = (st.w[0][2 * h + (p >> 2)] >> (8 * (p & 3))) & 0xFFu;
                    e7[p] = *reinterpret_cast<const uint32_t*>(reinterpret_cast<const char*>(lut) + (nbyte << 2));
                }
                if (__builtin_amdgcn_ballot_w64(st.verb != 0)) {     // rare: raw exponents for verbatim lanes
#pragma unroll
                    for (int p = 0; p < 8; ++p) {
                        const uint32_t er = (p & 1) ? exp_pair<1>(st.vx[h][p >> 1]) : exp_pair<0>(st.vx[h][p >> 1]);
                        e7[p] = st.verb ? er : e7[p];
                    }
                }
                join8(st.sm[h], e7, w + 8 * h);
            }
        }
#pragma unroll
        for (int sub = 0; sub < 4; ++sub) {
            const bf16x8_t A = __builtin_bit_cast(bf16x8_t, u32x4_t{w[4 * sub], w[4 * sub + 1], w[4 * sub + 2],
                                                                    w[4 * sub + 3]});
#pragma unroll
            for (int n = 0; n < NB; ++n)
                acc[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, __builtin_bit_cast(bf16x8_t, st.x[sub][n]),
                                                                 acc[n], 0, 0, 0);
        }
    };

    Step<SRC, NB> cur, nxt;
    __syncthreads();                                      // LUT ready
    if (s_lo < s_hi) {
        issue(s_lo, cur);
        for (uint32_t s = s_lo; s < s_hi; s += 2) {
            issue(min(s + 1, s_hi - 1), nxt);             // last step re-issued: no conditional load
            compute(cur);
            if (s + 1 >= s_hi) break;
            issue(min(s + 2, s_hi - 1), cur);
            compute(nxt);
        }
    }
    // sum the K-slices: D layout, lane l holds batch column l%16, rows 4*(l/16)..+3
#pragma unroll
    for (int n = 0; n < NB; ++n) part[wave][n][lane] = acc[n];
    __syncthreads();
    for (int idx = tid; idx < NB * 64; idx += 256) {
        const int n = idx / 64, l = idx % 64;
        f32x4_t v = part[0][n][l];
#pragma unroll
        for (int w_ = 1; w_ < kKW; ++w_) v += part[w_][n][l];
        const uint32_t b = nb0 + n * 16 + (l & 15);
        const uint32_t r = rb * 16 + 4 * (l >> 4);
        if (b < uint32_t(B)) {
            float* o = a.Y + int64_t(b) * a.R + r;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (r + i < uint32_t(a.R)) o[i] = v[i];
        }
    }
}

template <int SRC, int NB>
hipError_t launch_nb(const MatArgs& a, hipStream_t s) {
    dim3 grid(unsigned((a.R + 15) / 16), unsigned((a.B + NB * 16 - 1) / (NB * 16)));
    launch_timed(mfma_gemv_kernel<SRC, NB>, grid, dim3(256), 0, s, a);
    return hipGetLastError();
}

template <int SRC>
hipError_t launch_src(const MatArgs& a, hipStream_t s) {
    if (a.B <= 16) return launch_nb<SRC, 1>(a, s);
    if (a.B <= 32) return launch_nb<SRC, 2>(a, s);
    return launch_nb<SRC, 4>(a, s);
}

}  // namespace

// Supported when the K-slices are whole 128-column steps and each slice spans at
// most 4096 columns (so a lane's row segment touches at most two tiles).
bool mfma_gemv_supported(const MatArgs& a) {
    const int64_t steps = a.C / kKStep;
    return a.C > 0 && a.C % kKStep == 0 && (steps + kKW - 1) / kKW * kKStep <= 4096;
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
