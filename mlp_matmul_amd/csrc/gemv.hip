// Wavefront-reduction GEMV for small batches (B <= 16) on gfx950, over
// uncompressed bf16 weights or with on-chip weight reconstruction.
//
// Method: Cloudflare, "Unweight: how we compressed an LLM 22% without
// sacrificing quality".  "How the reconstructive matmul works": the kernel
// reads compressed weights, rebuilds bf16 on chip and multiplies, so rebuilt
// weights never go back to device memory.  "The GPU memory bottleneck": at
// small batch every token streams all weights, so the kernel is bound by HBM
// bandwidth and the fewer bytes it reads the faster it runs.
//
// Mapping to CDNA4: a wavefront owns one output row; per step each lane
// takes 16 consecutive weights (the wave covers 1024 contiguous weights, so
// every load instruction is fully coalesced), rebuilds them as 8 packed bf16
// pairs and accumulates with v_dot2_f32_bf16 per activation row; the 64
// partial sums are reduced across the wave at the end.
//   palette source: a 256-entry LDS table maps a byte of two 4-bit indices to
//     both exponents already in bf16 position; one v_perm and one v_and_or
//     merge them with the sign/mantissa bytes.  A lane whose 64-element
//     group is flagged in the bitmap takes its exponents from the verbatim
//     array instead (checked once per 16 weights, never per element).
//   exponent source: v_perm spreads two exponent bytes into place.
#include "device_common.h"
#include "kernels.h"

namespace uwk {

namespace {

constexpr int kSlab = 1024;   // weights per wave per step: 64 lanes x 16

__device__ __forceinline__ uint32_t palb(const MatArgs& a, int i) {
    return (a.pal[i >> 2] >> (8 * (i & 3))) & 0xFFu;
}

// Load the compressed (or raw) data of 16 consecutive weights of row-major
// position `pos` (multiple of 16).
template <int SRC>
struct Chunk {
    u32x4_t d0, d1;       // BF16: 8 dwords of weights; EXP: d0 = exponents; PAL: d0.xy = nibbles
    u32x4_t sm;           // EXP, PAL
    bool verb;
    uint64_t word;
    uint32_t vbase;
};

template <int SRC>
__device__ __forceinline__ void load_chunk(const MatArgs& a, int64_t pos, Chunk<SRC>& c) {
    if (SRC == SRC_BF16) {
        const uint16_t* w = static_cast<const uint16_t*>(a.w) + pos;
        c.d0 = load_stream16(w);
        c.d1 = load_stream16(w + 8);
    } else if (SRC == SRC_EXP) {
        c.d0 = load_stream16(static_cast<const uint8_t*>(a.w) + pos);
        c.sm = load_stream16(a.sm + pos);
    } else {
        const u32x2_t n = load_stream8(static_cast<const uint8_t*>(a.w) + pos / 2);
        c.d0 = u32x4_t{n[0], n[1], 0u, 0u};
        c.sm = load_stream16(a.sm + pos);
        const int64_t g = pos >> 6;
        c.word = a.bitmap[g >> 6];
        c.verb = (c.word >> (g & 63)) & 1ull;
    }
}

// Rebuild the 8 bf16 pairs of a chunk.
template <int SRC>
__device__ __forceinline__ void rebuild(const MatArgs& a, const Chunk<SRC>& c, int64_t pos, const uint32_t* lut,
                                        uint32_t w[8]) {
    if (SRC == SRC_BF16) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            w[i] = c.d0[i];
            w[4 + i] = c.d1[i];
        }
    } else if (SRC == SRC_EXP) {
#pragma unroll
        for (int p = 0; p < 8; ++p)
            w[p] = (p & 1) ? join_pair<1>(c.sm[p >> 1], exp_pair<1>(c.d0[p >> 1]))
                           : join_pair<0>(c.sm[p >> 1], exp_pair<0>(c.d0[p >> 1]));
    } else {
        uint32_t e7[8];
#pragma unroll
        for (int p = 0; p < 8; ++p) e7[p] = lut[(c.d0[p >> 2] >> (8 * (p & 3))) & 0xFFu];
        if (c.verb) {
            const int64_t g = pos >> 6;
            const uint32_t slot = verbatim_slot(c.word, uint32_t(g & 63), a.tile_vbase[g >> 6]);
            const u32x4_t v = load16(a.vexp + uint64_t(slot) * 64 + (pos & 63));
#pragma unroll
            for (int p = 0; p < 8; ++p) e7[p] = (p & 1) ? exp_pair<1>(v[p >> 1]) : exp_pair<0>(v[p >> 1]);
        }
#pragma unroll
        for (int p = 0; p < 8; ++p)
            w[p] = (p & 1) ? join_pair<1>(c.sm[p >> 1], e7[p]) : join_pair<0>(c.sm[p >> 1], e7[p]);
    }
}

template <int SRC, int MB, int UNR>
__global__ __launch_bounds__(256) void gemv_kernel(MatArgs a) {
    __shared__ uint32_t lut[256];
    if (SRC == SRC_PAL) {
        const int t = threadIdx.x;
        lut[t] = (palb(a, t & 15) << 7) | (palb(a, t >> 4) << 23);
        __syncthreads();
    }
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t r = int64_t(blockIdx.x) * 4 + wave;
    if (r >= a.R) return;
    const int64_t C = a.C;
    const int B = int(a.B);
    const int64_t row = r * C;
    float acc[MB];
#pragma unroll
    for (int b = 0; b < MB; ++b) acc[b] = 0.f;

    for (int64_t k0 = 0; k0 < C; k0 += int64_t(kSlab) * UNR) {
        Chunk<SRC> ch[UNR];
        bool ok[UNR];
#pragma unroll
        for (int u = 0; u < UNR; ++u) {
            const int64_t k = k0 + u * kSlab + lane * 16;
            ok[u] = k < C;
            if (ok[u]) load_chunk<SRC>(a, row + k, ch[u]);
        }
#pragma unroll
        for (int u = 0; u < UNR; ++u) {
            const int64_t k = k0 + u * kSlab + lane * 16;
            uint32_t w[8];
            if (ok[u]) rebuild<SRC>(a, ch[u], row + k, lut, w);
#pragma unroll
            for (int b = 0; b < MB; ++b) {
                if (!ok[u] || b >= B) continue;
                const uint16_t* xp = a.X + int64_t(b) * C + k;
                const u32x4_t x0 = load16(xp), x1 = load16(xp + 8);
                float s = acc[b];
                s = dot2_bf16(w[0], x0[0], s);
                s = dot2_bf16(w[1], x0[1], s);
                s = dot2_bf16(w[2], x0[2], s);
                s = dot2_bf16(w[3], x0[3], s);
                s = dot2_bf16(w[4], x1[0], s);
                s = dot2_bf16(w[5], x1[1], s);
                s = dot2_bf16(w[6], x1[2], s);
                s = dot2_bf16(w[7], x1[3], s);
                acc[b] = s;
            }
        }
    }
#pragma unroll
    for (int b = 0; b < MB; ++b) {
        if (b >= B) continue;
        const float v = wave_sum(acc[b]);
        if (lane == 0) a.Y[int64_t(b) * a.R + r] = v;
    }
}

template <int SRC>
hipError_t launch_src(const MatArgs& a, hipStream_t s) {
    const unsigned grid = unsigned((a.R + 3) / 4);
    if (a.B <= 1) gemv_kernel<SRC, 1, 4><<<grid, 256, 0, s>>>(a);
    else if (a.B <= 2) gemv_kernel<SRC, 2, 4><<<grid, 256, 0, s>>>(a);
    else if (a.B <= 4) gemv_kernel<SRC, 4, 2><<<grid, 256, 0, s>>>(a);
    else if (a.B <= 8) gemv_kernel<SRC, 8, 2><<<grid, 256, 0, s>>>(a);
    else gemv_kernel<SRC, 16, 1><<<grid, 256, 0, s>>>(a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemv(int src, const MatArgs& a, hipStream_t s) {
    if (a.R == 0 || a.B == 0) return hipSuccess;
    switch (src) {
        case SRC_BF16: return launch_src<SRC_BF16>(a, s);
        case SRC_EXP: return launch_src<SRC_EXP>(a, s);
        default: return launch_src<SRC_PAL>(a, s);
    }
}

}  // namespace uwk
