// bf16 MFMA matmul on gfx950 over uncompressed weights or with on-chip
// weight reconstruction, for batches from 16 up (any batch works).
//
// Method: Cloudflare, "Unweight: how we compressed an LLM 22% without
// sacrificing quality", "How the reconstructive matmul works": compressed
// weights are read from HBM, rebuilt as bf16 on chip and handed straight to
// the matrix units; rebuilt weights never return to device memory.  "Why no
// single pipeline wins": at large batch the matmul runs long enough to absorb
// the reconstruction work.
//
// Mapping to CDNA4 (the page's Hopper producer/consumer TMA + WGMMA design is
// not used): v_mfma_f32_16x16x32_bf16 takes its A operand as 8 consecutive-K
// bf16 per lane (lane l -> row l%16, K slice l/16).  Each lane therefore loads
// the compressed bytes of 16 consecutive weights of one row straight from HBM,
// rebuilds them in registers and feeds two MFMAs; no LDS round trip for the
// weights.  The activations, shared by every wave of the workgroup, are staged
// through double-buffered LDS with a padded row stride (no bank conflicts on
// the 16-byte B-operand reads).  A wave owns 32 rows x NB*16 batch columns.
// The K order inside an MFMA is a free permutation as long as A and B agree,
// so a lane's K slice is 16 contiguous weights split over two MFMAs.
#include "device_common.h"
#include "kernels.h"

namespace uwk {

namespace {

constexpr int kKB = 64;           // K per pipeline step
constexpr int kXS = kKB + 8;      // LDS row stride of the activation tile (bf16)

__device__ __forceinline__ uint32_t palb(const MatArgs& a, int i) { return pal_byte(a.pal, uint32_t(i)); }

template <int SRC>
struct AFrag {
    u32x4_t d0, d1, sm;
    uint64_t word;
    bool verb, ok;
};

template <int SRC>
__device__ __forceinline__ void load_a(const MatArgs& a, int64_t row, int64_t k, AFrag<SRC>& f) {
    f.ok = row < a.R;
    if (!f.ok) return;
    const int64_t pos = row * a.C + k;
    if (SRC == SRC_BF16) {
        const uint16_t* w = static_cast<const uint16_t*>(a.w) + pos;
        f.d0 = load_stream16(w);
        f.d1 = load_stream16(w + 8);
    } else if (SRC == SRC_EXP) {
        f.d0 = load_stream16(static_cast<const uint8_t*>(a.w) + pos);
        f.sm = load_stream16(a.sm + pos);
    } else {
        const u32x2_t n = load_stream8(static_cast<const uint8_t*>(a.w) + pos / 2);
        f.d0 = u32x4_t{n[0], n[1], 0u, 0u};
        f.sm = load_stream16(a.sm + pos);
        const int64_t g = pos >> 6;
        f.word = a.bitmap[g >> 6];
        f.verb = (f.word >> (g & 63)) & 1ull;
    }
}

// 16 weights -> two bf16x8 MFMA operands (elements 0-7, 8-15).
template <int SRC>
__device__ __forceinline__ void rebuild_a(const MatArgs& a, const AFrag<SRC>& f, int64_t row, int64_t k,
                                          const uint32_t* lut, bf16x8_t& o0, bf16x8_t& o1) {
    uint32_t w[8];
    if (!f.ok) {
#pragma unroll
        for (int p = 0; p < 8; ++p) w[p] = 0;
    } else if (SRC == SRC_BF16) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            w[i] = f.d0[i];
            w[4 + i] = f.d1[i];
        }
    } else if (SRC == SRC_EXP) {
#pragma unroll
        for (int p = 0; p < 8; ++p)
            w[p] = (p & 1) ? join_pair<1>(f.sm[p >> 1], exp_pair<1>(f.d0[p >> 1]))
                           : join_pair<0>(f.sm[p >> 1], exp_pair<0>(f.d0[p >> 1]));
    } else {
        uint32_t e7[8];
#pragma unroll
        for (int p = 0; p < 8; ++p) e7[p] = lut[(f.d0[p >> 2] >> (8 * (p & 3))) & 0xFFu];
        if (f.verb) {
            const int64_t pos = row * a.C + k;
            const int64_t g = pos >> 6;
            const uint32_t slot = verbatim_slot(f.word, uint32_t(g & 63), a.tile_vbase[g >> 6]);
            const u32x4_t v = load16(a.vexp + uint64_t(slot) * 64 + (pos & 63));
#pragma unroll
            for (int p = 0; p < 8; ++p) e7[p] = (p & 1) ? exp_pair<1>(v[p >> 1]) : exp_pair<0>(v[p >> 1]);
        }
#pragma unroll
        for (int p = 0; p < 8; ++p)
            w[p] = (p & 1) ? join_pair<1>(f.sm[p >> 1], e7[p]) : join_pair<0>(f.sm[p >> 1], e7[p]);
    }
    o0 = __builtin_bit_cast(bf16x8_t, u32x4_t{w[0], w[1], w[2], w[3]});
    o1 = __builtin_bit_cast(bf16x8_t, u32x4_t{w[4], w[5], w[6], w[7]});
}

// NB: 16-column batch blocks per wave; WM x WN waves per workgroup.
template <int SRC, int NB, int WM, int WN>
__global__ __launch_bounds__(256) void mfma_kernel(MatArgs a) {
    constexpr int NT = WN * NB * 16;       // batch columns per workgroup
    constexpr int MT = WM * 32;            // rows per workgroup
    constexpr int XCH = NT * (kKB / 8);    // 16-byte activation chunks per step
    constexpr int XPT = (XCH + 255) / 256; // chunks per thread
    extern __shared__ uint32_t lds[];
    uint32_t* lut = lds;                                       // 256 dwords
    uint16_t* xs = reinterpret_cast<uint16_t*>(lds + 256);     // [2][NT][kXS]

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int wm = wave % WM, wn = wave / WM;
    if (SRC == SRC_PAL) lut[tid] = (palb(a, tid & 15) << 7) | (palb(a, tid >> 4) << 23);

    const int64_t C = a.C;
    const int64_t row0 = int64_t(blockIdx.x) * MT + wm * 32;
    const int64_t nbase = int64_t(blockIdx.y) * NT;            // first batch row of this workgroup
    // K range of this split
    const int64_t nkb = C / kKB;
    const int64_t per = (nkb + a.split_k - 1) / a.split_k;
    const int64_t kb0 = int64_t(blockIdx.z) * per;
    const int64_t kb1 = min(nkb, kb0 + per);

    const int64_t arow0 = row0 + (lane & 15);
    const int64_t arow1 = arow0 + 16;
    const int ksl = 16 * (lane >> 4);                           // lane's K slice inside a step

    f32x4_t acc[2][NB];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    AFrag<SRC> fa0, fa1;
    u32x4_t xr[XPT];
    auto load_x = [&](int64_t kb) {
#pragma unroll
        for (int i = 0; i < XPT; ++i) {
            const int c = tid + i * 256;
            xr[i] = u32x4_t{0u, 0u, 0u, 0u};
            if (c < XCH) {
                const int n = c / (kKB / 8), part = c % (kKB / 8);
                const int64_t b = nbase + n;
                if (b < a.B) xr[i] = load16(a.X + b * C + kb * kKB + part * 8);
            }
        }
    };
    auto store_x = [&](int buf) {
        uint16_t* dst = xs + buf * NT * kXS;
#pragma unroll
        for (int i = 0; i < XPT; ++i) {
            const int c = tid + i * 256;
            if (c < XCH) {
                const int n = c / (kKB / 8), part = c % (kKB / 8);
                *reinterpret_cast<u32x4_t*>(dst + n * kXS + part * 8) = xr[i];
            }
        }
    };

    if (kb0 < kb1) {
        load_a<SRC>(a, arow0, kb0 * kKB + ksl, fa0);
        load_a<SRC>(a, arow1, kb0 * kKB + ksl, fa1);
        load_x(kb0);
    }
    int buf = 0;
    for (int64_t kb = kb0; kb < kb1; ++kb) {
        store_x(buf);
        __syncthreads();
        bf16x8_t A0[2], A1[2];
        rebuild_a<SRC>(a, fa0, arow0, kb * kKB + ksl, lut, A0[0], A0[1]);
        rebuild_a<SRC>(a, fa1, arow1, kb * kKB + ksl, lut, A1[0], A1[1]);
        if (kb + 1 < kb1) {
            load_a<SRC>(a, arow0, (kb + 1) * kKB + ksl, fa0);
            load_a<SRC>(a, arow1, (kb + 1) * kKB + ksl, fa1);
            load_x(kb + 1);
        }
        const uint16_t* xb = xs + buf * NT * kXS + (wn * NB * 16 + (lane & 15)) * kXS + ksl;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                const bf16x8_t B = *reinterpret_cast<const bf16x8_t*>(xb + nb * 16 * kXS + 8 * s);
                acc[0][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A0[s], B, acc[0][nb], 0, 0, 0);
                acc[1][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A1[s], B, acc[1][nb], 0, 0, 0);
            }
        }
        buf ^= 1;
    }

    // D layout: lane l holds column (batch) l%16, rows 4*(l/16) .. +3
    float* out = a.split_k > 1 ? a.partial + int64_t(blockIdx.z) * a.B * a.R : a.Y;
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            const int64_t b = nbase + wn * NB * 16 + nb * 16 + (lane & 15);
            const int64_t r = row0 + rb * 16 + 4 * (lane >> 4);
            if (b >= a.B) continue;
            float* o = out + b * a.R + r;
            const f32x4_t v = acc[rb][nb];
            if (r + 3 < a.R && ((a.R & 3) == 0)) {
                *reinterpret_cast<f32x4_t*>(o) = v;
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (r + i < a.R) o[i] = v[i];
            }
        }
    }
}

__global__ __launch_bounds__(256) void splitk_reduce(const float* __restrict__ p, int splits, int64_t n,
                                                     float* __restrict__ y) {
    const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
    if (i >= n) return;
    float s = 0.f;
    for (int z = 0; z < splits; ++z) s += p[int64_t(z) * n + i];
    y[i] = s;
}

template <int SRC, int NB, int WM, int WN>
hipError_t launch_cfg(const MatArgs& a, hipStream_t s) {
    constexpr int NT = WN * NB * 16, MT = WM * 32;
    const size_t lds = 256 * 4 + size_t(2) * NT * kXS * 2;
    static bool attr_set = false;   // opt in to more than 64 KiB of dynamic LDS once
    if (!attr_set && lds > 65536) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&mfma_kernel<SRC, NB, WM, WN>),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    dim3 grid(unsigned((a.R + MT - 1) / MT), unsigned((a.B + NT - 1) / NT), unsigned(a.split_k));
    launch_timed(mfma_kernel<SRC, NB, WM, WN>, grid, dim3(256), lds, s, a);
    return hipGetLastError();
}

template <int SRC>
hipError_t launch_src(const MatArgs& a, hipStream_t s) {
    if (a.B <= 16) return launch_cfg<SRC, 1, 4, 1>(a, s);
    if (a.B <= 32) return launch_cfg<SRC, 2, 4, 1>(a, s);
    if (a.B <= 64) return launch_cfg<SRC, 4, 4, 1>(a, s);
    if (a.B <= 128) return launch_cfg<SRC, 4, 2, 2>(a, s);
    return launch_cfg<SRC, 8, 2, 2>(a, s);
}

}  // namespace

hipError_t launch_mfma(int src, const MatArgs& a, hipStream_t s) {
    if (a.R == 0 || a.B == 0) return hipSuccess;
    hipError_t e;
    switch (src) {
        case SRC_BF16: e = launch_src<SRC_BF16>(a, s); break;
        case SRC_EXP: e = launch_src<SRC_EXP>(a, s); break;
        default: e = launch_src<SRC_PAL>(a, s); break;
    }
    if (e != hipSuccess || a.split_k <= 1) return e;
    const int64_t n = a.B * a.R;
    splitk_reduce<<<unsigned((n + 255) / 256), 256, 0, s>>>(a.partial, a.split_k, n, a.Y);
    return hipGetLastError();
}

}  // namespace uwk
