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
// Mapping to CDNA4.  A wavefront owns NRW consecutive output rows and walks
// their columns in slabs of 1024 weights; an *item* is one slab of all NRW
// rows.  In a slab each lane holds 16 weights of every row, laid out so that
// each load instruction of the wave reads one contiguous block (16 contiguous
// bytes per lane for the byte planes; for bf16, two 8-weight halves 512
// weights apart).  Items are software pipelined over two register sets: all
// loads of item t+1 are issued before item t is rebuilt and multiplied, and
// the loop has no data-dependent branch around a load, so the in-order vmcnt
// counter never makes a wave drain its prefetch.  The activations of a slab
// are read once (from LDS when B*C*2 <= 32 KiB, else from L2) and reused for
// all NRW rows.  Products go through v_dot2_f32_bf16 (two bf16 MACs, fp32
// sum); each row's 64 per-lane sums are reduced across the wave at the end.
//   palette source: the wave reads the verbatim bitmap words and verbatim
//     bases of all tiles its rows touch once (one per lane).  When an item is
//     issued each lane picks its group's word with a lane read, derives the
//     verbatim flag and slot, and issues the 16-byte load of its verbatim
//     exponents with the item's other loads (lanes outside verbatim groups all
//     read one shared line: no extra HBM bytes).  The rebuild maps a byte of
//     two 4-bit indices through a 256-entry LDS table to both exponents
//     already in bf16 position and merges them with the sign/mantissa bytes
//     (one v_perm and one v_and_or per pair); verbatim lanes take their raw
//     exponents instead, behind a wave-uniform branch that is skipped when no
//     lane of the slab is verbatim.  The check is per 16 weights, never per
//     element.
//   exponent source: v_perm spreads two exponent bytes into place.
#include <cstdio>
#include <cstdlib>
#include <type_traits>

#include "device_common.h"
#include "kernels.h"

namespace uwk {

namespace {

constexpr int kSlab = 1024;            // weights per row per item: 64 lanes x 16
constexpr int kXLdsMax = 32 * 1024;    // activation bytes staged in LDS at most

__device__ __forceinline__ uint32_t palb(const MatArgs& a, int i) { return pal_byte(a.pal, uint32_t(i)); }

// Element offsets (within a slab) of a lane's two 8-weight halves.
template <int SRC>
__device__ __forceinline__ uint32_t half_off(int lane, int h) {
    return SRC == SRC_BF16 ? uint32_t(h * 512 + lane * 8) : uint32_t(lane * 16 + h * 8);
}

template <int SRC, int MB>
struct Chunk {
    u32x4_t d0, d1;   // BF16: the two weight halves; EXP: d0 = 16 exponents; PAL: d0.xy = 16 nibbles
    u32x4_t sm;       // EXP, PAL: sign/mantissa bytes
    u32x4_t vx;       // PAL: verbatim exponents (meaningful when verb)
    uint32_t verb;    // PAL: 1 when the lane's 64-element group is verbatim
    u32x4_t xa[MB], xb[MB];   // activations read from L2 (row 0's chunk only)
};

// DUAL (palette source, one row per wave): the gate/up pair of a SwiGLU MLP.
// The wave's two row groups are row r of the gate matrix (a) and row r of
// the up matrix (up), over the same staged activations; the second group's
// epilogue writes h[b][r] = bf16(SiLU(g) * u), and g and u themselves when
// a.Y / up.Y are not null.
template <int SRC, int MB, int NRW, bool EXACT, bool XLDS, bool DUAL, int DEPTH, int XPC = 0>
__global__ __launch_bounds__(256) void gemv_kernel(MatArgs a, MatArgs up, uint16_t* H) {
    __shared__ uint32_t lut[DUAL ? 512 : 256];                   // nibble pair -> exponents in place
    extern __shared__ uint32_t lds[];
    uint16_t* xs = reinterpret_cast<uint16_t*>(lds);             // [B][C] when XLDS
    const int tid = threadIdx.x;
    const int64_t C = a.C;
    const uint32_t Cu = uint32_t(C);
    const int B = int(a.B);
    if (SRC == SRC_PAL) lut[tid] = (palb(a, tid & 15) << 7) | (palb(a, tid >> 4) << 23);
    if (DUAL) lut[256 + tid] = (palb(up, tid & 15) << 7) | (palb(up, tid >> 4) << 23);

    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int NG = DUAL ? 1 : a.row_groups;                      // row groups per wave
    const int64_t r0 = (int64_t(blockIdx.x) * 4 + wave) * NRW * NG;
    const bool live = r0 < a.R;                                  // wave has rows (uniform)
    const int wrows = live ? int(min(int64_t(NRW) * NG, a.R - r0)) : 0;
    const int ngroups = DUAL ? (live ? 2 : 0) : (wrows + NRW - 1) / NRW;
    const int iters = int((C + kSlab - 1) / kSlab);
    const int total = ngroups * iters;                           // items: (group, slab)
    // a wave past the matrix issues its loads from row 0 (so every wave runs
    // the same load sequence) and leaves before computing
    const int64_t rl0 = live ? r0 : 0;

    // the verbatim tables of every tile the wave's rows touch, one per lane
    const int64_t t_first = (rl0 * C) >> 12;
    uint64_t my_word = 0, my_word1 = 0;                          // my_word1, my_vbase1: DUAL's up matrix
    uint32_t my_vbase = 0, my_vbase1 = 0;
    // a lane's group inside a 1024-weight slab, and the mask of the groups below it
    const uint32_t lane_grp = uint32_t(lane) >> 2;
    const uint32_t lane_below = (1u << lane_grp) - 1u;
    // lanes outside verbatim groups all read the first line of this array
    const uint8_t* vb_ptr = a.vexp ? a.vexp : a.sm;
    const uint16_t* wb = static_cast<const uint16_t*>(a.w);
    const uint8_t* w8 = static_cast<const uint8_t*>(a.w);
    const uint8_t* vb_ptr1 = DUAL ? (up.vexp ? up.vexp : up.sm) : nullptr;
    // per-group planes (DUAL: group 1 reads the up matrix; the selects are uniform)
    auto w8_of = [&](int g) { return DUAL && g ? static_cast<const uint8_t*>(up.w) : w8; };
    auto sm_of = [&](int g) { return DUAL && g ? up.sm : a.sm; };

    float acc[NRW][MB];
#pragma unroll
    for (int r = 0; r < NRW; ++r)
#pragma unroll
        for (int b = 0; b < MB; ++b) acc[r][b] = 0.f;
    float gate_sum[MB];                                          // DUAL: the gate rows' results
#pragma unroll
    for (int b = 0; b < MB; ++b) gate_sum[b] = 0.f;

    // rows past the matrix (beyond wrows) re-read the wave's first row; their
    // sums are never stored.  issue_w: the weight planes (no dependency);
    // issue_v: the verbatim exponents, whose address needs the wave's tables.
    // an item is (row group g, slab s); items run g-major
    struct Item {
        int g, s;
    };
    auto row_of = [&](Item it, int r) -> uint32_t {
        const int rr = DUAL ? r : it.g * NRW + r;                // row inside the wave's range
        return uint32_t(rl0) + uint32_t(rr < wrows ? rr : 0);
    };
    auto issue_w = [&](Item it, Chunk<SRC, MB>* ch) {
        const uint32_t k0 = uint32_t(it.s) * kSlab;
#pragma unroll
        for (int r = 0; r < NRW; ++r) {
            const uint32_t row = row_of(it, r);
            Chunk<SRC, MB>& c = ch[r];
            uint32_t k = k0 + half_off<SRC>(lane, 0);
            if (!EXACT && k >= Cu) k = 0;
            const uint32_t pos = row * Cu + k;
            if (SRC == SRC_BF16) {
                uint32_t k1 = k0 + half_off<SRC>(lane, 1);
                if (!EXACT && k1 >= Cu) k1 = 0;
                c.d0 = load_stream16(wb + pos);
                c.d1 = load_stream16(wb + row * Cu + k1);
            } else if (SRC == SRC_EXP) {
                c.d0 = load_stream16(w8 + pos);
                c.sm = load_stream16(a.sm + pos);
            } else {
                const u32x2_t n = load_stream8(w8_of(it.g) + pos / 2);
                c.d0 = u32x4_t{n[0], n[1], 0u, 0u};
                c.sm = load_stream16(sm_of(it.g) + pos);
            }
        }
    };
    auto issue_v = [&](Item it, Chunk<SRC, MB>* ch) {
        if (SRC != SRC_PAL) return;
        const uint32_t k0 = uint32_t(it.s) * kSlab;
        const bool g1 = DUAL && it.g;                            // the up matrix's tables
        const uint64_t mw = g1 ? my_word1 : my_word;
        const uint32_t mv = g1 ? my_vbase1 : my_vbase;
        const uint8_t* vbp = g1 ? vb_ptr1 : vb_ptr;
#pragma unroll
        for (int r = 0; r < NRW; ++r) {
            const uint32_t row = row_of(it, r);
            Chunk<SRC, MB>& c = ch[r];
            uint32_t k = k0 + half_off<SRC>(lane, 0);
            if (!EXACT && k >= Cu) k = 0;
            const uint32_t pos = row * Cu + k;
            uint32_t voff = 0;
            if (EXACT) {
                // the slab lies in one tile: its word and base are uniform
                // (lane reads), its 16 groups are bits gb..gb+15 of the word
                const uint32_t sp = row * Cu + k0;
                const int tl = int((sp >> 12) - uint32_t(t_first));
                const uint64_t word =
                    (uint64_t(uint32_t(__builtin_amdgcn_readlane(int(mw >> 32), tl))) << 32) |
                    uint32_t(__builtin_amdgcn_readlane(int(uint32_t(mw)), tl));
                const uint32_t gb = (sp >> 6) & 63u;
                const uint32_t m16 = uint32_t(word >> gb) & 0xFFFFu;
                c.verb = (m16 >> lane_grp) & 1u;
                if (m16) {                                           // rare: a verbatim group in this slab
                    const uint32_t vbase = uint32_t(__builtin_amdgcn_readlane(int(mv), tl));
                    const uint64_t below = gb ? (word & ((~0ull) >> (64 - gb))) : 0ull;
                    const uint32_t slab_slot = vbase + uint32_t(__popcll(below));
                    const uint32_t slot = slab_slot + uint32_t(__popc(m16 & lane_below));
                    voff = c.verb ? slot * 64u + (pos & 63u) : 0u;
                }
            } else {
                const int tl = int((pos >> 12) - uint32_t(t_first));
                const uint64_t word = (uint64_t(uint32_t(__shfl(int(mw >> 32), tl))) << 32) |
                                      uint32_t(__shfl(int(uint32_t(mw)), tl));
                const uint32_t vbase = uint32_t(__shfl(int(mv), tl));
                const uint32_t bit = (pos >> 6) & 63u;
                c.verb = uint32_t(word >> bit) & 1u;
                if (__builtin_amdgcn_ballot_w64(c.verb != 0)) {
                    const uint32_t slot = verbatim_slot(word, bit, vbase);
                    voff = c.verb ? slot * 64u + (pos & 63u) : 0u;
                }
            }
            c.vx = load16(vbp + voff);
        }
    };
    // activations from L2 (when not staged in LDS) go out with the item, ahead
    // of its weights; batch rows past B re-read row B-1 so no load is
    // conditional
    auto issue_x = [&](Item it, Chunk<SRC, MB>* ch) {
        if (XLDS) return;
        const uint32_t k0 = uint32_t(it.s) * kSlab;
        uint32_t ka = k0 + half_off<SRC>(lane, 0), kb = k0 + half_off<SRC>(lane, 1);
        if (!EXACT) {
            if (ka >= Cu) ka = 0;
            if (kb >= Cu) kb = 0;
        }
#pragma unroll
        for (int b = 0; b < MB; ++b) {
            const uint32_t bb = uint32_t(b < B ? b : B - 1);
            ch[0].xa[b] = load16(a.X + bb * Cu + ka);
            ch[0].xb[b] = load16(a.X + bb * Cu + kb);
        }
    };
    auto issue = [&](Item it, Chunk<SRC, MB>* ch) {
        issue_x(it, ch);
        issue_w(it, ch);
        issue_v(it, ch);
    };

    auto next = [&](Item it) { return it.s + 1 == iters ? Item{it.g + 1, 0} : Item{it.g, it.s + 1}; };
    Chunk<SRC, MB> sets[DEPTH + 1][NRW];
    const Item it0{0, 0};
    // XPC > 0 (XLDS): the activation rows, at most XPC pieces of 16 bytes a
    // thread, and the verbatim tables of every tile the wave's rows touch
    // (one per lane) are loaded before item 0's weight loads; the waits
    // before the pieces are stored and before item 0's verbatim addresses
    // then cover only them, so the staging runs beside the start of the
    // weight stream.  (Without staging: weights, tables, verbatim.)  Every
    // thread loads all XPC pieces (past the end: the last one again, not
    // stored), so no load sits behind a branch.  (Issuing item 1 here as
    // well, ahead of the staging, measured slower.)
    constexpr int kXP = XLDS ? XPC : 0;
    const int64_t n16 = int64_t(B) * C / 8;
    u32x4_t xv[kXP > 0 ? kXP : 1];
    auto stage_load = [&]() {
#pragma unroll
        for (int u = 0; u < kXP; ++u) xv[u] = load16(a.X + min(int64_t(tid) + 256 * u, n16 - 1) * 8);
    };
    auto stage_store = [&]() {
        // a use of every piece keeps each load out of its store's branch
#pragma unroll
        for (int u = 0; u < kXP; ++u) asm volatile("" ::"v"(xv[u]));
#pragma unroll
        for (int u = 0; u < kXP; ++u)
            if (int64_t(tid) + 256 * u < n16) reinterpret_cast<u32x4_t*>(xs)[tid + 256 * u] = xv[u];
    };
    auto load_tables = [&]() {
        if (SRC == SRC_PAL) {
            const int64_t t_end = max(((rl0 + wrows) * C + 4095) >> 12, t_first + 1);
            const int64_t tl = min(t_first + lane, t_end - 1);
            my_word = a.bitmap[tl];
            my_vbase = a.tile_vbase[tl];
            if (DUAL) {
                my_word1 = up.bitmap[tl];
                my_vbase1 = up.tile_vbase[tl];
            }
        }
    };
    if (live && kXP > 0) {
        // staging, tables, then the weights: the waits of the stores and of
        // the verbatim addresses cover the loads issued before the weights
        stage_load();
        load_tables();
        issue_x(it0, sets[0]);
        issue_w(it0, sets[0]);
        stage_store();
        issue_v(it0, sets[0]);
    } else if (live) {
        issue_x(it0, sets[0]);
        issue_w(it0, sets[0]);
        load_tables();
        issue_v(it0, sets[0]);
    } else if (kXP > 0) {
        stage_load();
        stage_store();
    }
    if (XLDS && kXP == 0) {
        // four 16-byte pieces per thread go out before one wait (a load,
        // wait, store loop pays an L2 round trip per piece: seven of them
        // for a 14336-column row); pieces past the end re-read the last one,
        // so no load is conditional, and are not stored
        for (int64_t i0 = tid; i0 < n16; i0 += 256 * 4) {
            u32x4_t v[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) v[u] = load16(a.X + min(i0 + 256 * u, n16 - 1) * 8);
            // a use of all four here keeps each load out of its store's branch
            asm volatile("" ::"v"(v[0]), "v"(v[1]), "v"(v[2]), "v"(v[3]));
#pragma unroll
            for (int u = 0; u < 4; ++u)
                if (i0 + 256 * u < n16) reinterpret_cast<u32x4_t*>(xs)[i0 + 256 * u] = v[u];
        }
    }
    __syncthreads();
    if (!live) return;

    auto compute = [&](Item it, const Chunk<SRC, MB>* cur) {
        const uint32_t lut_off = DUAL && it.g ? 1024u : 0u;      // DUAL: the up matrix's table
        const uint32_t k0 = uint32_t(it.s) * kSlab;
        const uint32_t ka = k0 + half_off<SRC>(lane, 0), kb = k0 + half_off<SRC>(lane, 1);
        const bool oka = EXACT || ka < Cu, okb = EXACT || kb < Cu;
        // activations of this slab, shared by all rows
        u32x4_t xa[MB], xb[MB];
#pragma unroll
        for (int b = 0; b < MB; ++b) {
            if (b < B) {
                const uint32_t kka = oka ? ka : 0, kkb = okb ? kb : 0;
                if (XLDS) {
                    xa[b] = *reinterpret_cast<const u32x4_t*>(xs + b * Cu + kka);
                    xb[b] = *reinterpret_cast<const u32x4_t*>(xs + b * Cu + kkb);
                } else {
                    xa[b] = cur[0].xa[b];
                    xb[b] = cur[0].xb[b];
                }
            }
        }
#pragma unroll
        for (int r = 0; r < NRW; ++r) {
            const Chunk<SRC, MB>& c = cur[r];
            uint32_t w[8];
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
                for (int p = 0; p < 8; ++p) {
                    const uint32_t off = ((c.d0[p >> 2] >> (8 * (p & 3))) & 0xFFu) << 2;
                    e7[p] = *reinterpret_cast<const uint32_t*>(reinterpret_cast<const char*>(lut) + lut_off + off);
                }
                if (__builtin_amdgcn_ballot_w64(c.verb != 0)) {    // rare: raw exponents for verbatim lanes
#pragma unroll
                    for (int p = 0; p < 8; ++p) {
                        const uint32_t e_raw = (p & 1) ? exp_pair<1>(c.vx[p >> 1]) : exp_pair<0>(c.vx[p >> 1]);
                        e7[p] = c.verb ? e_raw : e7[p];
                    }
                }
#pragma unroll
                for (int p = 0; p < 8; ++p)
                    w[p] = (p & 1) ? join_pair<1>(c.sm[p >> 1], e7[p]) : join_pair<0>(c.sm[p >> 1], e7[p]);
            }
            if (!EXACT) {
                if (!oka) w[0] = w[1] = w[2] = w[3] = 0u;
                if (!okb) w[4] = w[5] = w[6] = w[7] = 0u;
            }
#pragma unroll
            for (int b = 0; b < MB; ++b) {
                if (b < B) {
                    float s = acc[r][b];
                    s = dot2_bf16(w[0], xa[b][0], s);
                    s = dot2_bf16(w[1], xa[b][1], s);
                    s = dot2_bf16(w[2], xa[b][2], s);
                    s = dot2_bf16(w[3], xa[b][3], s);
                    s = dot2_bf16(w[4], xb[b][0], s);
                    s = dot2_bf16(w[5], xb[b][1], s);
                    s = dot2_bf16(w[6], xb[b][2], s);
                    s = dot2_bf16(w[7], xb[b][3], s);
                    acc[r][b] = s;
                }
            }
        }
    };

    // a group's rows are complete after its last slab: reduce and store
    auto finish = [&](Item it) {
        if (it.s != iters - 1) return;
        const int g = it.g;
        if (DUAL) {
#pragma unroll
            for (int b = 0; b < MB; ++b) {
                if (b < B) {
                    const float v = wave_sum(acc[0][b]);
                    const int64_t o = int64_t(b) * a.R + r0;
                    if (g == 0) {
                        gate_sum[b] = v;
                        if (lane == 0 && a.Y) a.Y[o] = v;
                    } else if (lane == 0) {
                        if (up.Y) up.Y[o] = v;
                        H[o] = uint16_t(f32_to_bf16_rne(silu_mul1(gate_sum[b], v)));
                    }
                }
                acc[0][b] = 0.f;
            }
            return;
        }
#pragma unroll
        for (int r = 0; r < NRW; ++r) {
#pragma unroll
            for (int b = 0; b < MB; ++b) {
                const int rr = g * NRW + r;
                if (b < B && rr < wrows) {
                    const float v = wave_sum(acc[r][b]);
                    if (lane == 0) a.Y[int64_t(b) * a.R + r0 + rr] = v;
                }
                acc[r][b] = 0.f;
            }
        }
    };

    // a ring of DEPTH+1 register sets: the loads of item t+DEPTH are issued
    // before item t is computed (DEPTH 2 keeps two items in flight, for long
    // rows).  Items past the end read the wave's first row again (cache hits),
    // so no load is conditional; the body holds all DEPTH+1 steps with no exit
    // between them (leftover items are computed after the loop): a mid-body
    // exit lets the compiler fold identical steps into one with register
    // copies, which must wait for every load in flight.
    constexpr int NS = DEPTH + 1;
    Item ring[NS];
    ring[0] = it0;
#pragma unroll
    for (int j = 1; j < DEPTH; ++j) {
        ring[j] = next(ring[j - 1]);
        issue(ring[j], sets[j]);
    }
    int t = 0;
    for (; t + NS - 1 < total; t += NS) {
#pragma unroll
        for (int j = 0; j < NS; ++j) {
            const int jn = (j + DEPTH) % NS;
            ring[jn] = next(ring[(j + DEPTH - 1) % NS]);
            issue(ring[jn], sets[jn]);
            compute(ring[j], sets[j]);
            finish(ring[j]);
        }
    }
#pragma unroll
    for (int j = 0; j < NS - 1; ++j) {
        if (t + j < total) {
            compute(ring[j], sets[j]);
            finish(ring[j]);
        }
    }
}

__global__ void zero_fill(float* y, int64_t n) {
    const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
    if (i < n) y[i] = 0.f;
}

// Tuning overrides read once: UW_GEMV_NRW (rows per group), UW_GEMV_NG (row
// groups per wave), UW_GEMV_XGLOBAL=1/0 (activations from L2 / from LDS).
int env_int(const char* name, int dflt) {
    const char* e = getenv(name);
    return e ? atoi(e) : dflt;
}

// 16-byte activation pieces a thread of a 256-thread workgroup stages: 2, 4
// or 8 (at most kXLdsMax bytes)
int stage_pieces(const MatArgs& a) {
    const int64_t np = (a.B * a.C / 8 + 255) / 256;
    return np <= 2 ? 2 : (np <= 4 ? 4 : 8);
}

template <int SRC, int MB, int NRW, bool XLDS>
void launch_cfg(const MatArgs& a0, hipStream_t s) {
    // row groups per wave: long-lived waves amortise the per-wave start (tables,
    // activation staging); the wave's tiles must fit one per lane (<= 60)
    static const int ng_env = env_int("UW_GEMV_NG", 0);
    MatArgs a = a0;
    // measured on MI355X at batch 1: short rows (4096) of a tall matrix
    // (14336 rows) run best as one row per group and two groups per wave;
    // long rows (14336), and matrices under 8192 rows (attention
    // projections: more waves to fill the chip), as one row, one group
    int ng = ng_env > 0 ? ng_env : (NRW == 1 && a.C < 8192 && a.R >= 8192 ? 2 : 1);
    while (ng > 1 && int64_t(ng) * NRW * a.C > 60 * 4096) --ng;
    a.row_groups = ng;
    const int64_t waves = (a.R + int64_t(NRW) * ng - 1) / (int64_t(NRW) * ng);
    const unsigned grid = unsigned((waves + 3) / 4);
    const size_t lds = XLDS ? size_t(a.B * a.C * 2) : 0;
    // two items in flight per wave at batch 1-2 (measured on MI355X: the
    // batch-1 fused gate/up launch 32.9 -> 31.4 us); UW_GEMV_DEPTH=1 for one
    static const int depth_env = env_int("UW_GEMV_DEPTH", 0);
    const int depth = MB <= 2 ? (depth_env > 0 ? depth_env : 2) : 1;
    uint16_t* const no_h = nullptr;
    if (depth >= 2 && MB <= 2) {
        constexpr int D = MB <= 2 ? 2 : 1;
        const int xp = XLDS ? stage_pieces(a) : 0;
        auto go = [&](auto E, auto P) {
            launch_timed(gemv_kernel<SRC, MB, NRW, decltype(E)::value, XLDS, false, D, decltype(P)::value>, dim3(grid),
                         dim3(256), lds, s, a, MatArgs{}, no_h);
        };
        using T = std::true_type;
        using F = std::false_type;
        using P0 = std::integral_constant<int, 0>;
        using P2 = std::integral_constant<int, 2>;
        using P4 = std::integral_constant<int, 4>;
        using P8 = std::integral_constant<int, 8>;
        const bool ex = a.C % kSlab == 0;
        if (!XLDS) {
            if (ex) go(T{}, P0{}); else go(F{}, P0{});
        } else if (xp <= 2) {
            if (ex) go(T{}, P2{}); else go(F{}, P2{});
        } else if (xp <= 4) {
            if (ex) go(T{}, P4{}); else go(F{}, P4{});
        } else {
            if (ex) go(T{}, P8{}); else go(F{}, P8{});
        }
        return;
    }
    if (a.C % kSlab == 0)
        launch_timed(gemv_kernel<SRC, MB, NRW, true, XLDS, false, 1>, dim3(grid), dim3(256), lds, s, a, MatArgs{}, no_h);
    else
        launch_timed(gemv_kernel<SRC, MB, NRW, false, XLDS, false, 1>, dim3(grid), dim3(256), lds, s, a, MatArgs{}, no_h);
}

template <int SRC, int MB, int NRW>
void launch_x(const MatArgs& a, hipStream_t s) {
    // measured on MI355X at batch 1: the bf16 kernel runs faster reading its
    // one activation row from L2 (20.8 against 21.5 us on 14336x4096), the
    // rebuilding kernels faster from LDS (16.7 against 18.8 us, palette)
    // except on matrices of few rows, whose workgroups (about one per CU)
    // cannot hide the staging (1024x4096: 4.8-4.9 against 5.2-5.6 us; at
    // 4096x4096 LDS stays ahead, 7.3 against 7.4 us)
    static const int xg_env = env_int("UW_GEMV_XGLOBAL", -1);
    const bool xglobal = xg_env >= 0 ? xg_env == 1 : (a.B == 1 && (SRC == SRC_BF16 || a.R < 4096));
    if (a.B * a.C * 2 <= kXLdsMax && !xglobal) launch_cfg<SRC, MB, NRW, true>(a, s);
    else launch_cfg<SRC, MB, NRW, false>(a, s);
}

// Rows per group: one (measured best on both Llama shapes at batch 1; two
// reuse each activation fragment twice and are kept for tuning); the
// verbatim tables of a wave's rows must fit one per lane: NRW*C <= 60 tiles
// of 4096.
template <int SRC, int MB>
void launch_mb(const MatArgs& a, hipStream_t s) {
    static const int nrw_env = env_int("UW_GEMV_NRW", 0);
    int nrw = nrw_env ? nrw_env : 1;
    while (nrw > 1 && nrw * a.C > 60 * 4096) nrw >>= 1;
    switch (nrw) {
        case 2: launch_x<SRC, MB, 2>(a, s); break;
        default: launch_x<SRC, MB, 1>(a, s); break;
    }
}

template <int SRC>
hipError_t launch_src(const MatArgs& a, hipStream_t s) {
    if (a.B <= 1) launch_mb<SRC, 1>(a, s);
    else if (a.B <= 2) launch_mb<SRC, 2>(a, s);
    else if (a.B <= 4) launch_mb<SRC, 4>(a, s);
    else if (a.B <= 8) launch_mb<SRC, 8>(a, s);
    else launch_mb<SRC, 16>(a, s);
    return hipGetLastError();
}

// Gate/up pair: one row of each matrix per wave, activations staged in LDS.
template <int MB>
void launch_gateup_mb(const MatArgs& g, const MatArgs& u, uint16_t* h, hipStream_t s) {
    MatArgs a = g;
    a.row_groups = 1;
    const unsigned grid = unsigned((a.R + 3) / 4);
    const size_t lds = size_t(a.B * a.C * 2);
    static const int depth_env = env_int("UW_GEMV_DEPTH", 0);
    if ((depth_env == 0 || depth_env >= 2) && MB <= 2) {
        constexpr int D = MB <= 2 ? 2 : 1;
        const int xp = stage_pieces(a);
        auto go = [&](auto E, auto P) {
            launch_timed(gemv_kernel<SRC_PAL, MB, 1, decltype(E)::value, true, true, D, decltype(P)::value>, dim3(grid),
                         dim3(256), lds, s, a, u, h);
        };
        using T = std::true_type;
        using F = std::false_type;
        using P2 = std::integral_constant<int, 2>;
        using P4 = std::integral_constant<int, 4>;
        using P8 = std::integral_constant<int, 8>;
        const bool ex = a.C % kSlab == 0;
        if (xp <= 2) {
            if (ex) go(T{}, P2{}); else go(F{}, P2{});
        } else if (xp <= 4) {
            if (ex) go(T{}, P4{}); else go(F{}, P4{});
        } else {
            if (ex) go(T{}, P8{}); else go(F{}, P8{});
        }
        return;
    }
    if (a.C % kSlab == 0)
        launch_timed(gemv_kernel<SRC_PAL, MB, 1, true, true, true, 1>, dim3(grid), dim3(256), lds, s, a, u, h);
    else
        launch_timed(gemv_kernel<SRC_PAL, MB, 1, false, true, true, 1>, dim3(grid), dim3(256), lds, s, a, u, h);
}

}  // namespace

bool gemv_gateup_supported(const MatArgs& g, const MatArgs& u) {
    return g.R == u.R && g.C == u.C && g.B == u.B && g.B >= 1 && g.B <= 4 && g.C > 0 &&
           g.B * g.C * 2 <= kXLdsMax && g.C <= 60 * 4096;
}

hipError_t launch_gemv_gateup(const MatArgs& g, const MatArgs& u, uint16_t* h, hipStream_t s) {
    if (g.R == 0) return hipSuccess;
    if (!gemv_gateup_supported(g, u)) return hipErrorNotSupported;
    if (g.B <= 1) launch_gateup_mb<1>(g, u, h, s);
    else if (g.B <= 2) launch_gateup_mb<2>(g, u, h, s);
    else launch_gateup_mb<4>(g, u, h, s);
    return hipGetLastError();
}

hipError_t launch_gemv(int src, const MatArgs& a, hipStream_t s) {
    if (a.R == 0 || a.B == 0) return hipSuccess;
    if (a.C == 0) {
        const int64_t n = a.B * a.R;
        zero_fill<<<unsigned((n + 255) / 256), 256, 0, s>>>(a.Y, n);
        return hipGetLastError();
    }
    if (src == SRC_PAL && a.C > 60 * 4096) return hipErrorNotSupported;
    switch (src) {
        case SRC_BF16: return launch_src<SRC_BF16>(a, s);
        case SRC_EXP: return launch_src<SRC_EXP>(a, s);
        default: return launch_src<SRC_PAL>(a, s);
    }
}

}  // namespace uwk
