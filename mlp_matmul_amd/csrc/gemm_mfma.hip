// bf16 MFMA matmul on gfx950 for larger batches, over uncompressed weights
// or with on-chip weight reconstruction (any batch works; the launcher picks
// it above the skinny kernel's range through batch 64, and the LDS-tile
// kernel of gemm_lds.hip above that).
//
// Method: Cloudflare, "Unweight: how we compressed an LLM 22% without
// sacrificing quality", "How the reconstructive matmul works": compressed
// weights are read from HBM, rebuilt as bf16 on chip and handed straight to
// the matrix units; rebuilt weights never return to device memory.  "Why no
// single pipeline wins": at large batch the matmul runs long enough to absorb
// the reconstruction work.
//
// Mapping to CDNA4 (the page's Hopper producer/consumer TMA + WGMMA design is
// not used).  Y^T = W . X^T is a tall-skinny product (rows up to 14336, batch
// up to a few hundred), so the tiling is set by three budgets:
//   * LDS bandwidth: the activation (B) fragments come from LDS, and each one
//     feeds one v_mfma_f32_16x16x32_bf16 per 16-row block a wave owns (1 KB
//     per fragment: one row block per wave needs twice the LDS bandwidth of
//     the full MFMA rate, two row blocks exactly the LDS bandwidth);
//   * waves: a band of rows is one workgroup per batch tile, and the waves
//     of one workgroup meet at a barrier every step, so a compute unit needs
//     two waves per SIMD to overlap one wave's loads and rebuild with
//     another's MFMAs; at batch 64-256 the Llama shapes have about one
//     128-row band per compute unit, which one row block per wave (8 waves
//     to a 128-row band) fills where two row blocks (4 waves) did not;
//   * registers: the weights (A) are rebuilt straight into A-operand
//     registers from the compressed planes (no LDS round trip, no
//     redundancy: every wave owns distinct rows), double-buffered.
// A workgroup is WPG (4 or 8) waves x RBW (1 or 2) 16-row blocks by NB*16
// batch columns; a step covers 64 columns of K.  Lane l holds 16
// consecutive weights of row l%16 of each of its row blocks (columns
// 16*(l/16)..+16 of the step) and the matching activation runs as B
// fragments: the K order inside an MFMA is a free permutation as long as A
// and B agree.  All loads of step s+1 (the
// activation tile, the weight planes, the verbatim exponents) are issued
// before step s is computed, with no load behind a branch.  When each lane's
// row segment of the K-slice spans at most two tiles (slices of at most 4096
// columns: every split the Llama shapes take at large batch), the verbatim
// bitmap words and bases of those tiles are loaded into registers once, so a
// step's verbatim flag and slot are register arithmetic (1.5-5 % faster than
// the LDS tables at batch 64-256 on MI355X); otherwise the words and bases of
// every tile the workgroup's rows touch are staged in LDS once, so a step's
// verbatim flag and slot cost LDS reads, not a dependent global load.
// Split-K (blockIdx -> K slice) adds workgroups for
// short matrices; partial tiles go to a scratch array that a second kernel
// sums in a fixed order (deterministic).  Workgroups are numbered so that the
// batch tiles of one row band run back to back on one XCD and share its L2.
#include <cstdlib>

#include "device_common.h"
#include "kernels.h"

namespace uwk {

namespace {

constexpr int kKS = 64;          // K per step
constexpr int kXST = kKS + 8;    // LDS row stride of the activation tile (bf16), padded
constexpr int kMaxMT = 256;      // rows per workgroup at most

__device__ __forceinline__ uint32_t palb(const MatArgs& a, int i) { return pal_byte(a.pal, uint32_t(i)); }

// Per row block and step: the lane's 16 compressed weights.
template <int SRC>
struct AStep {
    u32x4_t d0, d1;   // BF16: 16 weights; EXP: d0 = 16 exponents; PAL: d0.xy = 16 nibbles
    u32x4_t sm;       // EXP, PAL
    u32x4_t vx;       // PAL: raw exponents when verbatim
    uint32_t verb;    // PAL
};

template <int SRC, int NB, int RBW, int WPG>
struct Step {
    static constexpr int kThreads = 64 * WPG;
    AStep<SRC> r[RBW];
    u32x4_t x[(NB * 16 * kKS / 8 + kThreads - 1) / kThreads];   // this thread's activation pieces
};

// WPG waves per workgroup, each with RBW 16-row blocks (WPG*16*RBW rows per
// workgroup).  PD steps of loads are kept in flight ahead of the step being
// computed (PD + 1 register sets).  Register budget: one or two row blocks,
// or four with four batch blocks and PD = 1, fit two waves per SIMD; deeper
// prefetch or four row blocks with eight batch blocks take the register file
// of one wave per SIMD.
template <int SRC, int NB, int PD, int RBW, int WPG, bool REGTAB = false>
__global__ __launch_bounds__(64 * WPG, (RBW <= 2 || (NB <= 4 && PD == 1)) ? 2 : 1)
void mfma_kernel(MatArgs a, int tiles_n, int split) {
    constexpr int kRBW = RBW;
    constexpr int kMT = WPG * 16 * RBW;                // rows per workgroup
    constexpr int NTHR = 64 * WPG;                     // threads per workgroup
    constexpr int NT = NB * 16;                        // batch columns per workgroup
    constexpr int XP = (NT * kKS / 8 + NTHR - 1) / NTHR;   // 16-byte activation pieces per thread
    __shared__ uint32_t lut[256];
    __shared__ __align__(16) uint16_t xs[2][NT * kXST];
    extern __shared__ __align__(16) uint32_t tabs[];   // PAL: u64 words [nt], then u32 bases [nt]

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    if (SRC == SRC_PAL && tid < 256) lut[tid] = (palb(a, tid & 15) << 7) | (palb(a, tid >> 4) << 23);

    // workgroup id -> (row band m, K slice s, batch tile n), n fastest, each
    // XCD (id % 8) taking a contiguous run of logical tiles
    const uint32_t G = gridDim.x, id = blockIdx.x;
    const uint32_t xcd = id & 7u, jx = id >> 3, q8 = G >> 3, r8 = G & 7u;
    const uint32_t L = xcd * q8 + min(xcd, r8) + jx;
    const uint32_t n_t = L % uint32_t(tiles_n);
    const uint32_t s_t = (L / uint32_t(tiles_n)) % uint32_t(split);
    const uint32_t m_t = L / (uint32_t(tiles_n) * uint32_t(split));

    const uint32_t R = uint32_t(a.R), C = uint32_t(a.C), B = uint32_t(a.B);
    const uint32_t steps = C / kKS;
    const uint32_t s_lo = steps * s_t / uint32_t(split), s_hi = steps * (s_t + 1) / uint32_t(split);
    const uint32_t n0 = n_t * NT;
    const uint32_t band0 = m_t * kMT;
    const uint32_t q = uint32_t(lane) >> 4, rl = uint32_t(lane) & 15u;

    // rows of this lane in each row block (rows past R read the last row; never stored)
    uint32_t rowc[kRBW];
#pragma unroll
    for (int rb = 0; rb < kRBW; ++rb) rowc[rb] = min(band0 + uint32_t(wave) * (16u * kRBW) + 16u * rb + rl, R - 1u);

    // verbatim tables of every tile the band touches, staged in LDS
    const uint32_t t_base = (band0 * C) >> 12;
    uint64_t* tword = reinterpret_cast<uint64_t*>(tabs);
    uint32_t nt = 0;
    if (SRC == SRC_PAL && !REGTAB) {
        const uint32_t last_row = min(band0 + kMT, R) - 1u;
        nt = ((last_row * C + C - 1u) >> 12) - t_base + 1u;
    }
    uint32_t* tbase = tabs + 2 * nt;

    const uint8_t* vb_ptr = a.vexp ? a.vexp : a.sm;
    const uint16_t* wb = static_cast<const uint16_t*>(a.w);
    const uint8_t* w8 = static_cast<const uint8_t*>(a.w);

    // issue_w: activation pieces and weight planes of step s (no dependency);
    // issue_v: the verbatim exponents (needs the LDS tables)
    auto issue_w = [&](uint32_t s, Step<SRC, NB, RBW, WPG>& st) {
        const uint32_t k0 = s * kKS;
#pragma unroll
        for (int j = 0; j < XP; ++j) {
            const uint32_t c = uint32_t(tid) + uint32_t(NTHR) * j;   // piece: batch row c/8, 8 columns (c%8)*8
            const uint32_t nb = min(c / 8u, uint32_t(NT) - 1u);
            const uint32_t b = min(n0 + nb, B - 1u);
            st.x[j] = load16(a.X + b * C + k0 + (c % 8u) * 8u);
        }
#pragma unroll
        for (int rb = 0; rb < kRBW; ++rb) {
            const uint32_t pos = rowc[rb] * C + k0 + 16u * q;
            AStep<SRC>& f = st.r[rb];
            if (SRC == SRC_BF16) {
                f.d0 = load16(wb + pos);
                f.d1 = load16(wb + pos + 8);
            } else if (SRC == SRC_EXP) {
                f.d0 = load16(w8 + pos);
                f.sm = load16(a.sm + pos);
            } else {
                const u32x2_t n = *reinterpret_cast<const u32x2_t*>(w8 + pos / 2);
                f.d0 = u32x4_t{n[0], n[1], 0u, 0u};
                f.sm = load16(a.sm + pos);
            }
        }
    };
    // REGTAB: a lane's row segment of the K-slice spans at most two tiles,
    // whose bitmap words and bases stay in registers (no LDS read per step;
    // a workgroup without steps reads its rows' first tile)
    uint32_t rt0[kRBW], rvb0[kRBW], rvb1[kRBW];
    uint64_t rw0[kRBW], rw1[kRBW];
    if (SRC == SRC_PAL && REGTAB) {
        const uint32_t sa = s_lo < s_hi ? s_lo : 0u, sb = s_lo < s_hi ? s_hi : 1u;
#pragma unroll
        for (int rb = 0; rb < kRBW; ++rb) {
            const uint32_t p0 = rowc[rb] * C + sa * kKS, p1 = rowc[rb] * C + sb * kKS - 1u;
            rt0[rb] = p0 >> 12;
            rw0[rb] = a.bitmap[rt0[rb]];
            rvb0[rb] = a.tile_vbase[rt0[rb]];
            rw1[rb] = a.bitmap[p1 >> 12];
            rvb1[rb] = a.tile_vbase[p1 >> 12];
        }
    }
    auto issue_v = [&](uint32_t s, Step<SRC, NB, RBW, WPG>& st) {
        if (SRC != SRC_PAL) return;
        const uint32_t k0 = s * kKS;
#pragma unroll
        for (int rb = 0; rb < kRBW; ++rb) {
            const uint32_t pos = rowc[rb] * C + k0 + 16u * q;
            const uint32_t g = pos >> 6, bit = g & 63u;
            uint64_t word;
            uint32_t vbase;
            if (REGTAB) {
                const bool second = (pos >> 12) != rt0[rb];
                word = second ? rw1[rb] : rw0[rb];
                vbase = second ? rvb1[rb] : rvb0[rb];
            } else {
                const uint32_t tl = (g >> 6) - t_base;
                word = tword[tl];
                vbase = tbase[tl];
            }
            AStep<SRC>& f = st.r[rb];
            f.verb = uint32_t(word >> bit) & 1u;
            const uint32_t slot = verbatim_slot(word, bit, vbase);
            // lanes outside verbatim groups all read one shared line
            f.vx = load16(vb_ptr + (f.verb ? slot * 64u + (pos & 63u) : 0u));
        }
    };
    auto stage_x = [&](uint32_t buf, const Step<SRC, NB, RBW, WPG>& st) {
#pragma unroll
        for (int j = 0; j < XP; ++j) {
            const uint32_t c = uint32_t(tid) + uint32_t(NTHR) * j;
            if (c < uint32_t(NT) * 8u)
                *reinterpret_cast<u32x4_t*>(&xs[buf][(c / 8u) * kXST + (c % 8u) * 8u]) = st.x[j];
        }
    };

    f32x4_t acc[kRBW][NB];
#pragma unroll
    for (int rb = 0; rb < kRBW; ++rb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) acc[rb][nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    auto compute = [&](uint32_t buf, const Step<SRC, NB, RBW, WPG>& st) {
        // A operands of every row block first, then per substep (8 K columns)
        // the NB activation fragments and their MFMAs: only one substep's
        // fragments are live, which leaves registers for deeper prefetch
        bf16x8_t Asub[kRBW][2];
#pragma unroll
        for (int rb = 0; rb < kRBW; ++rb) {
            const AStep<SRC>& f = st.r[rb];
            uint32_t w[8];
            if (SRC == SRC_BF16) {
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
                if (__builtin_amdgcn_ballot_w64(f.verb != 0)) {      // rare: raw exponents for verbatim lanes
#pragma unroll
                    for (int p = 0; p < 8; ++p) {
                        const uint32_t er = (p & 1) ? exp_pair<1>(f.vx[p >> 1]) : exp_pair<0>(f.vx[p >> 1]);
                        e7[p] = f.verb ? er : e7[p];
                    }
                }
#pragma unroll
                for (int p = 0; p < 8; ++p)
                    w[p] = (p & 1) ? join_pair<1>(f.sm[p >> 1], e7[p]) : join_pair<0>(f.sm[p >> 1], e7[p]);
            }
            Asub[rb][0] = __builtin_bit_cast(bf16x8_t, u32x4_t{w[0], w[1], w[2], w[3]});
            Asub[rb][1] = __builtin_bit_cast(bf16x8_t, u32x4_t{w[4], w[5], w[6], w[7]});
        }
        const uint16_t* xb = &xs[buf][rl * kXST + 16u * q];
#pragma unroll
        for (int sub = 0; sub < 2; ++sub) {
            bf16x8_t Bf[NB];
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
                Bf[nb] = *reinterpret_cast<const bf16x8_t*>(xb + nb * 16 * kXST + 8 * sub);
            // consecutive MFMAs update different accumulators (a dependent
            // pair back to back waits out the MFMA latency)
#pragma unroll
            for (int rb = 0; rb < kRBW; ++rb)
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
                    acc[rb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Asub[rb][sub], Bf[nb], acc[rb][nb], 0, 0, 0);
        }
    };

    // Start: the first step's weight loads go out first, then the tables are
    // staged (the loads before them are not waited for), then its verbatim
    // loads and the next PD-1 steps.  Steps past the slice re-issue its last
    // step, so no load is conditional.  Step t's activations go to xs[t & 1]:
    // its previous reader, step t-2, finished before every wave passed the
    // barrier of step t-1, so one barrier per step suffices.  The loop body
    // holds its PD+1 steps with no exit between them (leftover steps run
    // after the loop).
    constexpr int NS = PD + 1;
    const bool work = s_lo < s_hi;
    const uint32_t first = work ? s_lo : 0u, last = work ? s_hi - 1u : 0u;
    Step<SRC, NB, RBW, WPG> st[NS];
    issue_w(first, st[0]);
    if (SRC == SRC_PAL) {
        for (uint32_t i = uint32_t(tid); i < nt; i += uint32_t(NTHR)) {
            tword[i] = a.bitmap[t_base + i];
            tbase[i] = a.tile_vbase[t_base + i];
        }
    }
    __syncthreads();                                   // LUT and tables ready
    issue_v(first, st[0]);
#pragma unroll
    for (int j = 1; j < PD; ++j) {
        issue_w(min(first + j, last), st[j]);
        issue_v(min(first + j, last), st[j]);
    }
    if (work) {
        uint32_t s = first;
        for (; s + NS - 1 < s_hi; s += NS) {
#pragma unroll
            for (int j = 0; j < NS; ++j) {
                issue_w(min(s + j + PD, last), st[(j + PD) % NS]);
                issue_v(min(s + j + PD, last), st[(j + PD) % NS]);
                stage_x((s + j) & 1u, st[j]);
                __syncthreads();
                compute((s + j) & 1u, st[j]);
            }
        }
#pragma unroll
        for (int j = 0; j < NS - 1; ++j) {             // leftover steps: already issued
            if (s + j < s_hi) {
                stage_x((s + j) & 1u, st[j]);
                __syncthreads();
                compute((s + j) & 1u, st[j]);
            }
        }
    }

    // D layout: lane l holds batch column l%16, rows 4*(l/16) .. +3
    float* out = split > 1 ? a.partial + uint64_t(s_t) * a.B * a.R : a.Y;
    const uint32_t col = lane & 15;
#pragma unroll
    for (int rb = 0; rb < kRBW; ++rb) {
        const uint32_t r = band0 + uint32_t(wave) * (16u * kRBW) + 16u * rb + 4u * q;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            const uint32_t b = n0 + 16u * nb + col;
            if (b >= B) continue;
            float* o = out + uint64_t(b) * R + r;
            const f32x4_t v = acc[rb][nb];
            if (r + 3 < R && (R & 3u) == 0) {
                *reinterpret_cast<f32x4_t*>(o) = v;
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (r + i < R) o[i] = v[i];
            }
        }
    }
}

__global__ __launch_bounds__(256) void zero_fill(float* __restrict__ y, int64_t n) {
    const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
    if (i < n) y[i] = 0.f;
}

__global__ __launch_bounds__(256) void splitk_reduce(const float* __restrict__ p, int splits, int64_t n,
                                                     float* __restrict__ y) {
    const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
    if (i >= n) return;
    float s = 0.f;
    for (int z = 0; z < splits; ++z) s += p[int64_t(z) * n + i];
    y[i] = s;
}

// LDS bytes of the verbatim tables for a band of at most 256 rows (PAL).
size_t table_bytes(const MatArgs& a) {
    const int64_t rows = a.R < kMaxMT ? a.R : int64_t(kMaxMT);
    const int64_t nt = (rows * a.C + a.C) / 4096 + 2;
    return size_t(nt) * 12;
}

int env_int(const char* name, int dflt);

template <int SRC, int NB, int PD, int RBW, int WPG>
hipError_t launch_cfg(const MatArgs& a, hipStream_t s) {
    constexpr int NT = NB * 16, kMT = WPG * 16 * RBW;
    const int tiles_m = int((a.R + kMT - 1) / kMT), tiles_n = int((a.B + NT - 1) / NT);
    const int64_t grid = int64_t(tiles_m) * tiles_n * a.split_k;
    const int64_t slice = (a.C / kKS + a.split_k - 1) / a.split_k * kKS;
    if (SRC == SRC_PAL && slice <= 4096 && env_int("UW_MFMA_REGTAB", 1)) {   // UW_MFMA_REGTAB=0: LDS tables
        launch_timed(mfma_kernel<SRC, NB, PD, RBW, WPG, true>, dim3(unsigned(grid)), dim3(64 * WPG), 0, s, a,
                     tiles_n, int(a.split_k));
        return hipGetLastError();
    }
    const size_t lds = SRC == SRC_PAL ? table_bytes(a) : 0;
    launch_timed(mfma_kernel<SRC, NB, PD, RBW, WPG>, dim3(unsigned(grid)), dim3(64 * WPG), lds, s, a, tiles_n,
                 int(a.split_k));
    return hipGetLastError();
}

int env_int(const char* name, int dflt) {
    const char* e = getenv(name);
    return e && *e ? atoi(e) : dflt;
}

// Batch blocks per workgroup (4 up to batch 64, else 8); row blocks per
// wave (1, or 2 above batch 128 on matrices under 8192 rows); waves per
// workgroup (8 above batch 128, and above batch 64 on matrices under 8192
// rows, else 4); prefetch depth (2 for one row block and 4 waves, 3 for the
// 4-block batch tiles of the rebuilding sources with two row blocks, else
// 1).  Measured on the Llama MLP shapes at batch 64-256 on MI355X: one row
// block per wave gives a band twice the waves, so a compute unit runs two
// waves per SIMD where two row blocks left it one; the gate shape
// (14336 x 4096, palette source) at batch 64 / 128 / 256 took 31.4 / 44.9 /
// 64.6 us against 35.5 / 47.1 / 73.0 us with two row blocks per wave, and the
// bf16 source gained alike.  UW_MFMA_NB / _RBW / _WPG / _PD override for
// tuning.  Combinations that do not fit the register file are never
// instantiated.
struct Tiling {
    int nb, rbw, wpg;
};
Tiling tiling_of(const MatArgs& a) {
    const bool tall = a.R >= 8192;
    const int nb = a.B <= 64 ? 4 : 8;
    const int rbw = a.B > 128 && !tall ? 2 : 1;
    const int wpg = a.B > 128 || (a.B > 64 && !tall) ? 8 : 4;
    return {env_int("UW_MFMA_NB", nb), env_int("UW_MFMA_RBW", rbw), env_int("UW_MFMA_WPG", wpg)};
}

template <int SRC>
hipError_t launch_src(const MatArgs& a, hipStream_t s) {
    const Tiling tl = tiling_of(a);
    const int nb = tl.nb, rbw = tl.rbw, wpg = tl.wpg;
    const int pd = env_int("UW_MFMA_PD", rbw <= 1 ? (wpg <= 4 ? 2 : 1) : nb <= 4 && SRC != SRC_BF16 ? 3 : 1);
    if (rbw <= 1) {
        if (wpg <= 4) {
            if (nb <= 4) return pd <= 1 ? launch_cfg<SRC, 4, 1, 1, 4>(a, s) : launch_cfg<SRC, 4, 2, 1, 4>(a, s);
            return pd <= 1 ? launch_cfg<SRC, 8, 1, 1, 4>(a, s) : launch_cfg<SRC, 8, 2, 1, 4>(a, s);
        }
        if (nb <= 4) return pd <= 1 ? launch_cfg<SRC, 4, 1, 1, 8>(a, s) : launch_cfg<SRC, 4, 2, 1, 8>(a, s);
        return pd <= 1 ? launch_cfg<SRC, 8, 1, 1, 8>(a, s) : launch_cfg<SRC, 8, 2, 1, 8>(a, s);
    }
    if (rbw <= 2) {
        if (wpg <= 4) {
            if (nb <= 4) {
                if (pd <= 1) return launch_cfg<SRC, 4, 1, 2, 4>(a, s);
                if (pd == 2) return launch_cfg<SRC, 4, 2, 2, 4>(a, s);
                return launch_cfg<SRC, 4, 3, 2, 4>(a, s);
            }
            if (pd <= 1) return launch_cfg<SRC, 8, 1, 2, 4>(a, s);
            return launch_cfg<SRC, 8, 2, 2, 4>(a, s);
        }
        if (nb <= 4) {
            if (pd <= 1) return launch_cfg<SRC, 4, 1, 2, 8>(a, s);
            if (pd == 2) return launch_cfg<SRC, 4, 2, 2, 8>(a, s);
            return launch_cfg<SRC, 4, 3, 2, 8>(a, s);
        }
        if (pd <= 1) return launch_cfg<SRC, 8, 1, 2, 8>(a, s);
        return launch_cfg<SRC, 8, 2, 2, 8>(a, s);
    }
    if (nb <= 4) {
        if (pd <= 1) return launch_cfg<SRC, 4, 1, 4, 4>(a, s);
        if (pd == 2) return launch_cfg<SRC, 4, 2, 4, 4>(a, s);
        return launch_cfg<SRC, 4, 3, 4, 4>(a, s);
    }
    if (SRC == SRC_BF16 && pd > 1) return launch_cfg<SRC, 8, (SRC == SRC_BF16 ? 3 : 1), 4, 4>(a, s);
    return launch_cfg<SRC, 8, 1, 4, 4>(a, s);
}

}  // namespace

// K-slices that give the launch about one workgroup per CU: the smallest
// power of two (at most 8, each slice at least 4 steps) for which tiles x
// slices reaches three quarters of the CUs (measured on the Llama MLP
// shapes at batch 32-256, this is the split the autotuner picks).
int mfma_default_split(int src, const MatArgs& a, int cus) {
    if (a.R <= 0 || a.B <= 0 || a.C <= 0) return 1;
    if (lds_gemm_preferred(src, a)) return lds_gemm_default_split(src, a, cus);
    const Tiling tl = tiling_of(a);
    const int64_t mt = 16 * int64_t(tl.rbw <= 1 ? 1 : tl.rbw <= 2 ? 2 : 4) * (tl.wpg <= 4 ? 4 : 8);
    const int64_t nt = 16 * int64_t(tl.nb <= 4 ? 4 : 8);
    const int64_t tiles = ((a.R + mt - 1) / mt) * ((a.B + nt - 1) / nt);
    const int64_t steps = a.C / kKS;
    int split = 1;
    while (split < 8 && tiles * split * 4 < int64_t(cus) * 3 && steps / (2 * split) >= 4) split *= 2;
    return split;
}

// The kernel keeps a lane's row segment of one step in one 64-column group
// and stages the verbatim tables of a 256-row band in LDS (at most 48 KiB).
bool mfma_supported(const MatArgs& a) {
    return a.C % kKS == 0 && (a.C == 0 || table_bytes(a) <= 48 * 1024);
}

hipError_t launch_mfma(int src, const MatArgs& a, hipStream_t s) {
    if (a.R == 0 || a.B == 0) return hipSuccess;
    if (a.C == 0) {                                    // empty sums
        const int64_t n = a.B * a.R;
        zero_fill<<<unsigned((n + 255) / 256), 256, 0, s>>>(a.Y, n);
        return hipGetLastError();
    }
    if (!mfma_supported(a)) return hipErrorNotSupported;
    hipError_t e;
    if (lds_gemm_preferred(src, a)) e = launch_lds_gemm(src, a, s);
    else switch (src) {
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
