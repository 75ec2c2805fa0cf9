// Skinny matmul (batch 1..32) on palette-source weights with every streamed
// operand moved by the LDS DMA path, and the gate/up pair of an MLP block
// with the SiLU product in its epilogue.
//
// Method: Cloudflare, "Unweight: how we compressed an LLM 22% without
// sacrificing quality", "How the reconstructive matmul works": the 4-bit
// palette indices and sign/mantissa bytes go from HBM to on-chip storage,
// are rebuilt to bf16 there and fed to the matrix units; rebuilt weights
// never reach device memory.  "The GPU memory bottleneck": at small batch the
// product is bound by the weight stream, so what counts is how many bytes are
// in flight and how few instructions each byte costs on its way in.
//
// Mapping to CDNA4.  A wavefront owns 16 weight rows (NRB row blocks of them:
// two blocks of one matrix, or in the gate/up pair the same 16 rows of both
// matrices) and one K-slice, in steps of 128 columns.  Each step's operands
// travel with global_load_lds_dwordx4: the hardware writes lane i's 16 bytes
// to slot i of a 1 KB LDS block, so the data never occupies VGPRs on the way
// in and a wave keeps D steps in flight at the cost of LDS only (a ring of D
// slots, one LDS array per slot so the compiler can tell the slots apart).
// Per row block and step: the 4-bit indices (16 rows x 64 bytes, one load)
// and the sign/mantissa bytes (16 x 128 bytes, two loads); once per step the
// activation tile (4*XQ batch rows x 256 bytes, XQ loads; batch 17-32 takes
// two 16-column batch tiles, so each rebuilt weight feeds eight MFMAs a step
// instead of four).  The lane that
// loads a 16-byte chunk is picked so that the chunk lands at an XOR-swizzled
// slot of its row, which makes the read-back in the MFMA operand layout (16
// lanes on 16 rows, one chunk column) hit distinct banks.  Verbatim
// exponents (rare) go to registers with the step's loads, 32 bytes a lane
// (lanes outside verbatim groups all read one shared line).  The step loop
// is software pipelined with explicit s_waitcnt vmcnt: before step s is
// rebuilt exactly the loads of steps s+1..s+D-1 may still be pending.
//   MFMA: v_mfma_f32_16x16x32_bf16, lane l on row l%16 and the 32 columns
// 32*(l/16).. of the step (the K order inside an MFMA is a free permutation
// when A and B agree), four MFMAs a step and row block.  Batch rows past the
// 4*XQ loaded ones read a loaded row's fragment; their outputs are not
// stored.
#include <cstdlib>

#include "device_common.h"
#include "kernels.h"

namespace uwk {

namespace {

constexpr int kDStep = 128;        // columns per step
constexpr int kDMaxSlice = 4096;   // a wave's K-slice spans at most two tiles
constexpr int kNibBytes = 1024;    // one row block's 4-bit indices of a step
constexpr int kSmBytes = 2048;     // one row block's sign/mantissa bytes of a step
// two 16-column batch tiles per wave at most: with four (batch 33-64) the
// Llama gate/up pair measured 80-87 us against 71-77 us for two tiled MFMA
// launches and the SiLU product on MI355X
constexpr int kDMaxBatch = 32;

typedef __attribute__((address_space(3))) void* lds_void_ptr;

// Moves 16 bytes per lane from global memory to LDS: lane i's bytes land at
// dst + 16*i (dst is uniform across the wave).
__device__ __forceinline__ void dma16(const void* src, void* dst) {
    __builtin_amdgcn_global_load_lds(src, (lds_void_ptr)dst, 16, 0, 0);
}

// s_waitcnt with only vmcnt constrained (vmcnt in bits 3:0 and 15:14,
// expcnt and lgkmcnt at their maxima).
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

__device__ __forceinline__ u32x4_t lds16(const uint8_t* p) { return *reinterpret_cast<const u32x4_t*>(p); }

// Registers a step keeps from issue to rebuild (verbatim exponents).
template <int NRB>
struct VRegs {
    u32x4_t vx[NRB][2];
    uint32_t verb[NRB];
};

// NRB row blocks per wave (DUAL: block 0 of gate `a`, block 1 of `up`, same
// rows); XQ quads of activation rows; KW waves split K; D steps in flight.
template <int NRB, bool DUAL, int XQ, int KW, int D>
__global__ __launch_bounds__(64 * KW) void skinny_dma_kernel(MatArgs a, MatArgs up, uint16_t* H) {
    static_assert(!DUAL || NRB == 2, "gate/up pair: one block of each matrix");
    static_assert(D >= 2 && D <= 4 && ((XQ >= 1 && XQ <= 4) || XQ == 8), "ring depth, activation quads");
    constexpr int NB = XQ > 4 ? 2 : 1;                   // 16-column batch tiles
    constexpr int kXOff = NRB * (kNibBytes + kSmBytes);
    constexpr int kSlot = kXOff + XQ * 1024;             // LDS bytes of one step of one wave
    constexpr int kPer = NRB * 5 + XQ;                   // vector-memory instructions a step
    static_assert((D - 1) * kPer < 64, "vmcnt range");
    __shared__ uint32_t lut[DUAL ? 512 : 256];
    __shared__ __align__(16) uint8_t ring0[KW * kSlot];
    __shared__ __align__(16) uint8_t ring1[KW * kSlot];
    __shared__ __align__(16) uint8_t ring2[D > 2 ? KW * kSlot : 16];
    __shared__ __align__(16) uint8_t ring3[D > 3 ? KW * kSlot : 16];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const uint32_t lane = uint32_t(tid) & 63u;
    const uint32_t R = uint32_t(a.R), C = uint32_t(a.C), B = uint32_t(a.B);
    constexpr uint32_t kRowsPerWg = DUAL ? 16u : 16u * NRB;
    const uint32_t row0 = blockIdx.x * kRowsPerWg;
    const uint32_t steps = C / kDStep;
    const uint32_t s_lo = steps * uint32_t(wave) / KW, s_hi = steps * uint32_t(wave + 1) / KW;
    const uint32_t q = lane >> 4, rl = lane & 15u;

    auto mat = [&](int r) -> const MatArgs& { return (DUAL && r) ? up : a; };
    // first row of row block r (the gate/up pair: both blocks on the same rows)
    auto block_row = [&](int r) { return row0 + (DUAL ? 0u : 16u * uint32_t(r)); };
    auto clamp_row = [&](uint32_t row) { return row < R ? row : R - 1u; };

    // verbatim tables of the (at most two) tiles each row segment touches,
    // loaded first and on every path (a wave without steps reads its row's
    // first tile), so their wait overlaps the table fill and the barrier and
    // does not drain the first steps' loads
    uint32_t rowc[NRB], t0[NRB], vb0[NRB], vb1[NRB];
    uint64_t word0[NRB], word1[NRB];
    {
        const uint32_t sa = s_lo < s_hi ? s_lo : 0u, sb = s_lo < s_hi ? s_hi : 1u;
#pragma unroll
        for (int r = 0; r < NRB; ++r) {
            const MatArgs& m = mat(r);
            rowc[r] = clamp_row(block_row(r) + rl);
            const uint32_t p0 = rowc[r] * C + sa * kDStep, p1 = rowc[r] * C + sb * kDStep - 1u;
            t0[r] = p0 >> 12;
            word0[r] = m.bitmap[t0[r]];
            vb0[r] = m.tile_vbase[t0[r]];
            word1[r] = m.bitmap[p1 >> 12];
            vb1[r] = m.tile_vbase[p1 >> 12];
        }
    }
    for (int i = tid; i < 256; i += 64 * KW) {
        lut[i] = (pal_byte(a.pal, uint32_t(i) & 15u) << 7) | (pal_byte(a.pal, uint32_t(i) >> 4) << 23);
        if (DUAL) lut[256 + i] = (pal_byte(up.pal, uint32_t(i) & 15u) << 7) | (pal_byte(up.pal, uint32_t(i) >> 4) << 23);
    }
    // per-lane sources of the step's DMA loads (the step adds s*64 / s*128
    // bytes).  4-bit plane: lane l brings chunk c of row l/4, stored at slot
    // 4*row + (c ^ ((row >> 1) & 3)); sign/mantissa: load i, t = 64i + l,
    // chunk c of row t/8 at slot 8*row + (c ^ (row & 7)); activations: load
    // j, t = 64j + l, chunk c of batch row t/16 at slot 16*row + (c ^ (row & 7)).
    const uint8_t* nib_src[NRB];
    const uint8_t* sm_src[NRB][2];
#pragma unroll
    for (int r = 0; r < NRB; ++r) {
        const MatArgs& m = mat(r);
        {
            const uint32_t rho = lane >> 2, c = (lane & 3u) ^ ((rho >> 1) & 3u);
            nib_src[r] = static_cast<const uint8_t*>(m.w) + uint64_t(clamp_row(block_row(r) + rho)) * (C / 2) + c * 16u;
        }
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const uint32_t t = uint32_t(i) * 64u + lane, rho = t >> 3, c = (t & 7u) ^ (rho & 7u);
            sm_src[r][i] = m.sm + uint64_t(clamp_row(block_row(r) + rho)) * C + c * 16u;
        }
    }
    const uint8_t* x_src[XQ];
#pragma unroll
    for (int j = 0; j < XQ; ++j) {
        const uint32_t t = uint32_t(j) * 64u + lane, b = t >> 4, c = (t & 15u) ^ (b & 7u);
        const uint32_t bc = b < B ? b : B - 1u;
        x_src[j] = reinterpret_cast<const uint8_t*>(a.X + uint64_t(bc) * C) + c * 16u;
    }


    auto slot_base = [&](int j) -> uint8_t* {
        uint8_t* const arr = j == 0 ? ring0 : (j == 1 ? ring1 : (j == 2 ? ring2 : ring3));
        return arr + wave * kSlot;
    };

    auto issue = [&](uint32_t s, int j, VRegs<NRB>& v) {
        uint8_t* const base = slot_base(j);
#pragma unroll
        for (int r = 0; r < NRB; ++r) {
            const MatArgs& m = mat(r);
            dma16(nib_src[r] + s * 64u, base + r * kNibBytes);
            dma16(sm_src[r][0] + s * 128u, base + NRB * kNibBytes + r * kSmBytes);
            dma16(sm_src[r][1] + s * 128u, base + NRB * kNibBytes + r * kSmBytes + 1024);
            const uint32_t pos = rowc[r] * C + s * kDStep + 32u * q;
            const bool second = (pos >> 12) != t0[r];
            const uint64_t word = second ? word1[r] : word0[r];
            const uint32_t bit = (pos >> 6) & 63u;
            v.verb[r] = uint32_t(word >> bit) & 1u;
            const uint32_t slot = verbatim_slot(word, bit, second ? vb1[r] : vb0[r]);
            const uint8_t* vb_ptr = m.vexp ? m.vexp : m.sm;
            const uint32_t voff = v.verb[r] ? slot * 64u + (pos & 63u) : 0u;
            v.vx[r][0] = load16(vb_ptr + voff);
            v.vx[r][1] = load16(vb_ptr + voff + 16);
        }
#pragma unroll
        for (int jx = 0; jx < XQ; ++jx) dma16(x_src[jx] + s * 256u, base + kXOff + jx * 1024);
        // the step's loads stay together: the waits count them in issue order
        __builtin_amdgcn_sched_barrier(0);
    };

    f32x4_t acc[NRB][NB];
#pragma unroll
    for (int r = 0; r < NRB; ++r)
#pragma unroll
        for (int n = 0; n < NB; ++n) acc[r][n] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    auto compute = [&](int j, const VRegs<NRB>& v) {
        const uint8_t* const base = slot_base(j);
        // every LDS read of the step first (B fragments: batch row 16n + rl,
        // or a loaded row when fewer are loaded; the lane's 8-column runs 32q
        // + 8sub), then the table lookups of all row blocks, so the wave waits
        // on LDS twice a step
        u32x4_t xf[4][NB], nb[NRB], sm[NRB][2];
#pragma unroll
        for (int n = 0; n < NB; ++n) {
            const uint32_t xb = (16u * uint32_t(n) + rl) & uint32_t(4 * XQ - 1);
#pragma unroll
            for (int sub = 0; sub < 4; ++sub)
                xf[sub][n] = lds16(base + kXOff + (xb * 16u + ((4u * q + uint32_t(sub)) ^ (xb & 7u))) * 16u);
        }
#pragma unroll
        for (int r = 0; r < NRB; ++r) {
            nb[r] = lds16(base + r * kNibBytes + (rl * 4u + (q ^ ((rl >> 1) & 3u))) * 16u);
            const uint8_t* const smb = base + NRB * kNibBytes + r * kSmBytes;
#pragma unroll
            for (int h = 0; h < 2; ++h) sm[r][h] = lds16(smb + (rl * 8u + ((2u * q + uint32_t(h)) ^ (rl & 7u))) * 16u);
        }
        uint32_t e7[NRB][16];
#pragma unroll
        for (int r = 0; r < NRB; ++r) {
            const char* const lutm = reinterpret_cast<const char*>(lut + (DUAL ? 256 * r : 0));
#pragma unroll
            for (int p = 0; p < 16; ++p) {
                const uint32_t nbyte = (nb[r][p >> 2] >> (8 * (p & 3))) & 0xFFu;
                e7[r][p] = *reinterpret_cast<const uint32_t*>(lutm + (nbyte << 2));
            }
        }
        // a lane's 32 weights of a row block lie in one group: a verbatim
        // lane takes all of them from its raw exponents, under its own exec
        // mask (two instructions a pair, and none when no lane of the wave
        // is verbatim in that block)
#pragma unroll
        for (int r = 0; r < NRB; ++r) {
            if (v.verb[r]) {
#pragma unroll
                for (int p = 0; p < 16; ++p) {
                    const uint32_t d = v.vx[r][p >> 3][(p & 7) >> 1];
                    e7[r][p] = (p & 1) ? exp_pair<1>(d) : exp_pair<0>(d);
                }
            }
        }
#pragma unroll
        for (int r = 0; r < NRB; ++r) {
            uint32_t w[16];
#pragma unroll
            for (int p = 0; p < 16; ++p) {
                const uint32_t smw = sm[r][p >> 3][(p & 7) >> 1];
                w[p] = (p & 1) ? join_pair<1>(smw, e7[r][p]) : join_pair<0>(smw, e7[r][p]);
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
        // every read of this slot has returned before it is refilled
        __builtin_amdgcn_sched_barrier(0);
    };

    __syncthreads();                                     // LUT ready
    // D steps in flight; steps past the slice re-issue its last step, so every
    // step issues the same loads and the waits are compile-time constants.  The
    // loop body holds D steps (each slot has its own array and register set);
    // the 0..D-1 steps left over follow it.
    if (s_lo < s_hi) {
        const uint32_t last = s_hi - 1u;
        VRegs<NRB> v[D];
#pragma unroll
        for (int j = 0; j < D; ++j) issue(min(s_lo + uint32_t(j), last), j, v[j]);
        uint32_t s = s_lo;
        for (; s + D <= s_hi; s += D) {
#pragma unroll
            for (int j = 0; j < D; ++j) {
                wait_vm<(D - 1) * kPer>();
                compute(j, v[j]);
                issue(min(s + uint32_t(j + D), last), j, v[j]);
            }
        }
#pragma unroll
        for (int j = 0; j < D - 1; ++j) {
            if (s + uint32_t(j) < s_hi) {
                wait_vm<(D - 1) * kPer>();
                compute(j, v[j]);
                issue(last, j, v[j]);
            }
        }
        wait_vm<0>();                                    // no DMA may land after the LDS is reused
    }

    // D layout: lane l holds batch column l%16 of its tile, rows 4*(l/16)..+3
    // of a block
    f32x4_t res[NRB][NB];
    if (KW == 1) {
#pragma unroll
        for (int r = 0; r < NRB; ++r)
#pragma unroll
            for (int n = 0; n < NB; ++n) res[r][n] = acc[r][n];
    } else {
        // sum the K-slices in wave order, through the first ring slot
        __syncthreads();
        f32x4_t* const part = reinterpret_cast<f32x4_t*>(ring0);   // [KW][NRB][NB][64]
#pragma unroll
        for (int r = 0; r < NRB; ++r)
#pragma unroll
            for (int n = 0; n < NB; ++n) part[((wave * NRB + r) * NB + n) * 64 + int(lane)] = acc[r][n];
        __syncthreads();
        if (wave != 0) return;
#pragma unroll
        for (int r = 0; r < NRB; ++r)
#pragma unroll
            for (int n = 0; n < NB; ++n) {
                res[r][n] = part[(r * NB + n) * 64 + int(lane)];
#pragma unroll
                for (int w_ = 1; w_ < KW; ++w_) res[r][n] += part[((w_ * NRB + r) * NB + n) * 64 + int(lane)];
            }
    }
#pragma unroll
    for (int n = 0; n < NB; ++n) {
        const uint32_t b = 16u * uint32_t(n) + (lane & 15u);
        if (b >= B) continue;
        if (DUAL) {
            const uint32_t rr = row0 + 4u * q;
            const int64_t o = int64_t(b) * a.R + rr;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                if (rr + uint32_t(i) < R) {
                    if (a.Y) a.Y[o + i] = res[0][n][i];
                    if (up.Y) up.Y[o + i] = res[1][n][i];
                    H[o + i] = uint16_t(f32_to_bf16_rne(silu_mul1(res[0][n][i], res[1][n][i])));
                }
            }
        } else {
#pragma unroll
            for (int r = 0; r < NRB; ++r) {
                const uint32_t rr = block_row(r) + 4u * q;
                float* const o = a.Y + int64_t(b) * a.R + rr;
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (rr + uint32_t(i) < R) o[i] = res[r][n][i];
            }
        }
    }
}

int env_int(const char* name, int dflt) {
    const char* e = getenv(name);
    return e && *e ? atoi(e) : dflt;
}

struct DShape {
    int kw, d;
};

// K-split: the smallest (1, 2, 4, 8) that gives at least three waves per
// compute unit and keeps each slice within kDMaxSlice columns, counted in
// 16-row blocks: the K-split, and so the order of every output's sums,
// depends on the matrix shape only, so the gate/up pair is bitwise equal to
// single launches of this kernel.  Ring depth,
// as measured on MI355X on the Llama shapes: two steps for the pair (gate/up
// at batch 6-16: 36.6-38.9 us against 37.5-39.8 with three); for single
// matrices three steps up to batch 8 (the 14336x4096 gate at batch 5: 19.9
// against 23.2 us with four) and four above (batch 16: 24.9 against 25.8);
// never more than an even share of 150 KB of LDS among the waves a compute
// unit holds, nor than one workgroup's share allows (UW_DMA_KW / UW_DMA_D
// override).
DShape dma_shape(const MatArgs& a, int rows_per_wg, int slot_bytes, bool dual) {
    const int64_t cus = a.cus > 0 ? a.cus : 256;
    const int64_t steps = a.C / kDStep;
    const int64_t wgs = (a.R + rows_per_wg - 1) / rows_per_wg;
    const int64_t blocks = (a.R + 15) / 16;
    int kw = env_int("UW_DMA_KW", 0);
    if (kw <= 0) {
        kw = 1;
        while (kw < 8 && blocks * kw < 3 * cus) kw *= 2;
    }
    kw = kw <= 1 ? 1 : (kw <= 2 ? 2 : (kw <= 4 ? 4 : 8));
    while (kw < 8 && (steps + kw - 1) / kw * kDStep > kDMaxSlice) kw *= 2;
    int d = env_int("UW_DMA_D", 0);
    if (d <= 0) {
        const int64_t waves_per_cu = (wgs * kw + cus - 1) / cus;
        const int64_t budget = 150 * 1024 / (waves_per_cu > 0 ? waves_per_cu : 1);
        const int fit = int(budget / slot_bytes);
        const int want = dual ? 2 : (a.B <= 8 ? 3 : 4);
        d = want < fit ? want : fit;
    }
    d = d < 2 ? 2 : (d > 4 ? 4 : d);
    return {kw, d};
}

constexpr int kRingLds = 150 * 1024;   // LDS the ring of a workgroup may take

// Ring depths whose LDS fits a workgroup, and whose pending loads fit the
// vmcnt counter, are instantiated; a deeper request takes the deepest that
// fits, and a shape where not even two steps fit is not supported.
template <int NRB, bool DUAL, int XQ, int KW>
hipError_t launch_d(const MatArgs& a, const MatArgs& up, uint16_t* h, int d, hipStream_t s) {
    constexpr int rows = DUAL ? 16 : 16 * NRB;
    constexpr int slot = NRB * (kNibBytes + kSmBytes) + XQ * 1024;
    constexpr int per = NRB * 5 + XQ;                    // loads a step: D-1 steps pending fit vmcnt (63)
    constexpr int dlds = kRingLds / (KW * slot), dvm = 1 + 63 / per;
    constexpr int dmax = dlds < dvm ? (dlds < 4 ? dlds : 4) : (dvm < 4 ? dvm : 4);
    if constexpr (dmax < 2) {
        return hipErrorNotSupported;
    } else {
        const dim3 grid(unsigned((a.R + rows - 1) / rows)), block(64 * KW);
        d = d < dmax ? d : dmax;
        if (d <= 2) {
            launch_timed(skinny_dma_kernel<NRB, DUAL, XQ, KW, 2>, grid, block, 0, s, a, up, h);
        } else if constexpr (dmax >= 3) {
            if (d == 3) launch_timed(skinny_dma_kernel<NRB, DUAL, XQ, KW, 3>, grid, block, 0, s, a, up, h);
            if constexpr (dmax >= 4)
                if (d >= 4) launch_timed(skinny_dma_kernel<NRB, DUAL, XQ, KW, 4>, grid, block, 0, s, a, up, h);
        }
        return hipGetLastError();
    }
}

template <int NRB, bool DUAL, int XQ>
hipError_t launch_xq(const MatArgs& a, const MatArgs& up, uint16_t* h, hipStream_t s) {
    constexpr int rows = DUAL ? 16 : 16 * NRB;
    constexpr int slot = NRB * (kNibBytes + kSmBytes) + XQ * 1024;
    const DShape sh = dma_shape(a, rows, slot, DUAL);
    switch (sh.kw) {
        case 1: return launch_d<NRB, DUAL, XQ, 1>(a, up, h, sh.d, s);
        case 2: return launch_d<NRB, DUAL, XQ, 2>(a, up, h, sh.d, s);
        case 4: return launch_d<NRB, DUAL, XQ, 4>(a, up, h, sh.d, s);
        default: return launch_d<NRB, DUAL, XQ, 8>(a, up, h, sh.d, s);
    }
}

template <int NRB, bool DUAL>
hipError_t launch_nrb(const MatArgs& a, const MatArgs& up, uint16_t* h, hipStream_t s) {
    if (a.B <= 4) return launch_xq<NRB, DUAL, 1>(a, up, h, s);
    if (a.B <= 8) return launch_xq<NRB, DUAL, 2>(a, up, h, s);
    if (a.B <= 16) return launch_xq<NRB, DUAL, 4>(a, up, h, s);
    return launch_xq<NRB, DUAL, 8>(a, up, h, s);
}

}  // namespace

// The gate/up pair takes this kernel where it measured faster than the two
// register-staged skinny launches (or that kernel's own pair) on MI355X:
// batch 3-32 on matrices tall enough for one wave per 16-row block and at
// least three waves per compute unit (K unsplit; the Llama gate/up pair at
// batch 4: 36.0 against 37.8 us, batch 16: 39.1 against 46.3, batch 32: 46.6
// against 54.3 for the separate launches and the SiLU product).  Single
// matrices keep the register-staged kernel, which is faster for them (the
// 14336x4096 gate at batch 16: 23.6 against 25.1 us, batch 32: 25.9 against
// 29.3); UW_SKINNY_DMA=1 forces this kernel for both, UW_SKINNY_DMA=0 for
// neither.
bool skinny_dma_pair_preferred(const MatArgs& a) {
    const int mode = env_int("UW_SKINNY_DMA", -1);
    if (mode == 0 || !skinny_dma_supported(a)) return false;
    if (mode > 0) return true;
    const int64_t cus = a.cus > 0 ? a.cus : 256;
    return a.B >= 3 && (a.R + 15) / 16 >= 3 * cus;
}

bool skinny_dma_forced() { return env_int("UW_SKINNY_DMA", -1) > 0; }

// Whole 128-column steps, batch 1..32, every K-slice (split 8 ways at most)
// within 4096 columns.
bool skinny_dma_supported(const MatArgs& a) {
    const int64_t steps = a.C / kDStep;
    return a.B >= 1 && a.B <= kDMaxBatch && a.C > 0 && a.C % kDStep == 0 &&
           (steps + 7) / 8 * kDStep <= kDMaxSlice && a.R > 0;
}

hipError_t launch_skinny_dma(const MatArgs& a, hipStream_t s) {
    if (a.R == 0 || a.B == 0) return hipSuccess;
    if (!skinny_dma_supported(a)) return hipErrorNotSupported;
    const int nrb = env_int("UW_DMA_NRB", 1);
    return nrb >= 2 ? launch_nrb<2, false>(a, MatArgs{}, nullptr, s) : launch_nrb<1, false>(a, MatArgs{}, nullptr, s);
}

hipError_t launch_skinny_dma_gateup(const MatArgs& g, const MatArgs& u, uint16_t* h, hipStream_t s) {
    if (g.R == 0 || g.B == 0) return hipSuccess;
    if (!(skinny_dma_supported(g) && g.R == u.R && g.C == u.C && g.B == u.B)) return hipErrorNotSupported;
    return launch_nrb<2, true>(g, u, h, s);
}

}  // namespace uwk
