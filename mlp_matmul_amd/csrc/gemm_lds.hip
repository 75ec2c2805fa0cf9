// bf16 MFMA matmul on gfx950 for batch 64 and up, over uncompressed weights
// or with on-chip weight reconstruction, in which every weight is rebuilt
// once per workgroup into a shared LDS tile; and the fused gate/up pair of an
// MLP block with the SiLU product, above batch 32.
//
// Method: Cloudflare, "Unweight: how we compressed an LLM 22% without
// sacrificing quality", "How the reconstructive matmul works": compressed
// weights are read from HBM, rebuilt as bf16 on chip and handed to the matrix
// units; rebuilt weights never return to device memory.  "Why no single
// pipeline wins": at large batch the matmul runs long enough to absorb the
// reconstruction, so what matters is how close the product runs to the
// matrix units' rate.
//
// Mapping to CDNA4.  Y^T = W . X^T with W tall (rows up to 14336) and the
// batch 64-256.  A workgroup of eight waves (two per SIMD) owns MT = 128 rows
// x NT = 64, 128 or 256 batch columns x one K-slice, in steps of 64 columns
// (one 64-weight group of each row, so a row's verbatim flag is one bit per
// step).
//   * Per step, each lane rebuilds 16 consecutive weights of one row and
//     writes them as bf16 into an LDS tile in MFMA-fragment form: fragment
//     (16-row block, 32-column half) is 1 KB, 64 slots of 8 columns.
//   * Global loads are row-ordered: four consecutive lanes read 64 contiguous
//     bytes of one row (weights and activations alike).  CDNA4's vector L1
//     charges one access per distinct row segment a group of four lanes
//     touches, so loading straight in the fragment layout (16 rows per 16
//     lanes) cost four times the L1 accesses and stalled the address unit.
//   * The fragment slots are swizzled: chunk q of row r sits at slot
//     16q + (r ^ m), m built from the chunk's position, so the row-ordered
//     LDS writes and the fragment reads (one 256-byte run per 16 lanes) are
//     both free of bank conflicts.
//   * Each wave computes a (MT/WGM) x (NT/WGN) block of the output with
//     v_mfma_f32_16x16x32_bf16, register-blocked FM x FN: per 32-column half
//     it reads FM + FN fragments for FM*FN MFMAs.
//   * The loads of step s+P are issued before step s is computed, into P
//     register sets; the LDS tiles are double-buffered with one barrier per
//     step, after which the next step's fragments are read.
//   * Verbatim tables (bitmap word and verbatim-group base of every tile the
//     band's rows touch) are staged in LDS once, so a step's verbatim slot is
//     an LDS read, not a dependent global load.
// Each weight is rebuilt once per workgroup (the register-rebuilding tiled
// kernel rebuilds it once per wave that uses it), and a 128-row band streams
// the activations once per 128 rows.
// The gate/up pair runs 64-row bands of both matrices: waves 0-3 rebuild the
// gate rows and waves 4-7 the up rows, every wave accumulates its output
// block of both from the one activation tile, and the epilogue writes
// h = bf16(SiLU(g) * u), K unsplit (224 workgroups for the Llama gate/up
// shape with 64, 128 or 256 batch columns).
// Split-K adds workgroups for short matrices; partial tiles go to a scratch
// array that a second kernel sums in a fixed order (deterministic).
// Workgroups are numbered so that each XCD's run of workgroups shares one
// K-slice of the activations in its L2.
#include <cstdlib>

#include "device_common.h"
#include "kernels.h"

namespace uwk {

namespace {

constexpr int kLS = 64;            // K columns per step
constexpr int kLMaxTiles = 640;    // verbatim tables of a band staged in LDS at most

__device__ __forceinline__ uint32_t lpalb(const MatArgs& a, int i) { return pal_byte(a.pal, uint32_t(i)); }

// One lane's 16 compressed weights of a step.
struct LItem {
    u32x4_t d0, d1;   // BF16: 16 weights; EXP: d0 = 16 exponents
    u32x2_t nib;      // PAL: 16 nibbles
    u32x4_t sm;       // EXP, PAL: sign/mantissa bytes
    u32x4_t vx;       // PAL: raw exponents when verbatim
    uint32_t verb;    // PAL
};

template <int MT, int NT, int NW, int NMAT>
struct LStage {
    LItem w[NMAT * MT / (16 * NW)];
    u32x4_t x[NT / (8 * NW)];
};

// MT rows x NT batch columns per workgroup of NW waves, laid out WGM x (NW /
// WGM) over the tile; P steps of loads in flight.  DUAL: the gate/up pair of
// an MLP block (`a` gate, `up` up, same shape, palette sources, no K split):
// each step rebuilds the band's rows of both matrices (with 64-row bands,
// waves 0-3 rebuild gate and 4-7 up), both use the one activation tile, each
// wave accumulates its output block of both, and the epilogue writes
// H = bf16(SiLU(g) * u) (and g, u into a.Y, up.Y when those are not NULL).
template <int SRC, int MT, int NT, int NW, int WGM, int P, bool DUAL = false>
__global__ __launch_bounds__(64 * NW, 1)
void lds_gemm_kernel(MatArgs a, MatArgs up, uint16_t* H, int tiles_n, int split, int order) {
    static_assert(!DUAL || SRC == SRC_PAL, "the gate/up pair takes palette sources");
    constexpr int NMAT = DUAL ? 2 : 1;
    constexpr int WGN = NW / WGM;
    constexpr int NS = P;                              // register sets of loads
    constexpr int FM = MT / 16 / WGM, FN = NT / 16 / WGN;
    // rebuild items: a lane's item it is block wave + NW*it of the NMAT*RB
    // 16-row blocks (matrix block/RB, row block block%RB)
    constexpr int RB = MT / 16;
    constexpr int IPT = NMAT * RB / NW, XP = NT / (8 * NW);
    static_assert(IPT >= 1 && NMAT * RB % NW == 0 && (NW == RB || NW == 2 * RB) && XP >= 1 && FM >= 1 && FN >= 1,
                  "tile too small for the waves");
    constexpr int WBUF = MT * kLS, XBUF = NT * kLS;     // bf16 elements per buffer
    __shared__ __align__(16) uint16_t wl[NMAT][2 * WBUF];
    __shared__ __align__(16) uint16_t xl[2 * XBUF];
    __shared__ uint32_t lut[NMAT][256];
    __shared__ uint64_t tword[NMAT][SRC == SRC_PAL ? kLMaxTiles : 1];
    __shared__ uint32_t tbase[NMAT][SRC == SRC_PAL ? kLMaxTiles : 1];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    auto mat = [&](int m) -> const MatArgs& { return (DUAL && m) ? up : a; };
    if (SRC == SRC_PAL && tid < 256) {
        lut[0][tid] = (lpalb(a, tid & 15) << 7) | (lpalb(a, tid >> 4) << 23);
        if (DUAL) lut[NMAT - 1][tid] = (lpalb(up, tid & 15) << 7) | (lpalb(up, tid >> 4) << 23);
    }

    // workgroup id -> (row band m, K slice s, batch tile n), each XCD (id %
    // 8) taking a contiguous run of logical tiles; n fastest, then m, then s
    // (an XCD's run shares its K-slice of the activations in its L2), or
    // with order 0 n, then s, then m (a run shares its row bands' weights)
    const uint32_t G = gridDim.x, id = blockIdx.x;
    const uint32_t xcd = id & 7u, jx = id >> 3, q8 = G >> 3, r8 = G & 7u;
    const uint32_t L = xcd * q8 + min(xcd, r8) + jx;
    const uint32_t n_t = L % uint32_t(tiles_n);
    const uint32_t tiles_m = (uint32_t(a.R) + MT - 1) / MT;
    uint32_t s_t, m_t;
    if (order) {
        m_t = (L / uint32_t(tiles_n)) % tiles_m;
        s_t = L / (uint32_t(tiles_n) * tiles_m);
    } else {
        s_t = (L / uint32_t(tiles_n)) % uint32_t(split);
        m_t = L / (uint32_t(tiles_n) * uint32_t(split));
    }

    const uint32_t R = uint32_t(a.R), C = uint32_t(a.C), B = uint32_t(a.B);
    const uint32_t steps = C / kLS;
    const uint32_t s_lo = steps * s_t / uint32_t(split), s_hi = steps * (s_t + 1) / uint32_t(split);
    const uint32_t n0 = n_t * NT;
    const uint32_t band0 = m_t * MT;

    // The lane's items: row block wave + NW*it, row lane/4, columns
    // 16*(lane%4)..+15 of the step, so four consecutive lanes read 64
    // contiguous bytes of one row (rows past R read the last row; never
    // stored).  Fragment slots are swizzled: chunk q (8 columns) of row r of a
    // fragment sits at slot 16q + (r ^ m), m from the chunk's position, which
    // keeps these row-order writes and the fragment-order reads free of bank
    // conflicts.
    // matrix and row block of item it (NW == RB: matrix it, block wave;
    // NW == 2 RB, one item: matrix wave/RB, block wave%RB)
    auto item_mat = [&](int it) -> int { return NW == RB ? it : (wave + NW * it) / RB; };
    auto item_rb = [&](int it) -> uint32_t { return NW == RB ? uint32_t(wave) : uint32_t((wave + NW * it) % RB); };
    uint32_t rowc[IPT];
#pragma unroll
    for (int it = 0; it < IPT; ++it) rowc[it] = min(band0 + 16u * item_rb(it) + uint32_t(lane >> 2), R - 1u);
    const uint32_t lc = uint32_t(lane & 3), lr = uint32_t(lane >> 2);
    const uint32_t koff = 16u * lc;
    // W: the item's chunks 2(lc%2), 2(lc%2)+1 of half lc/2 (bf16 elements,
    // inside its row block's pair of fragments)
    const uint32_t wm_sw = 4u * (lc & 1u) + 10u * (lc >> 1);
    const uint32_t wslot = ((lc >> 1) * 64u + (lr ^ wm_sw) + 32u * (lc & 1u)) * 8u;
    // X: chunk lc of row lr of a fragment
    const uint32_t xslot = ((lr ^ (4u * (lc & 1u) + 10u * (lc >> 1))) + 16u * lc) * 8u;

    // verbatim tables of every tile the band's rows touch
    const uint32_t t_base = (band0 * C) >> 12;
    uint32_t nt = 0;
    if (SRC == SRC_PAL) {
        const uint32_t last_row = min(band0 + MT, R) - 1u;
        nt = ((last_row * C + C - 1u) >> 12) - t_base + 1u;
    }


    // issue_w: activation pieces and weight planes of step s (no dependency);
    // issue_v: the verbatim exponents (needs the LDS tables)
    auto issue_w = [&](uint32_t s, LStage<MT, NT, NW, NMAT>& st) {
        const uint32_t k0 = s * kLS;
#pragma unroll
        for (int j = 0; j < XP; ++j) {
            // fragment wave + NW*j of the tile (batch block f/2, half f%2):
            // chunk lane%4 of batch row lane/4
            const uint32_t f = uint32_t(wave + NW * j);
            const uint32_t b = min(n0 + 16u * (f >> 1) + lr, B - 1u);
            st.x[j] = load16(a.X + b * C + k0 + 32u * (f & 1u) + 8u * lc);
        }
#pragma unroll
        for (int it = 0; it < IPT; ++it) {
            const int m = item_mat(it);
            const uint32_t pos = rowc[it] * C + k0 + koff;
            LItem& f = st.w[it];
            const uint16_t* wb = static_cast<const uint16_t*>(mat(m).w);
            const uint8_t* w8 = static_cast<const uint8_t*>(mat(m).w);
            if (SRC == SRC_BF16) {
                f.d0 = load16(wb + pos);
                f.d1 = load16(wb + pos + 8);
            } else if (SRC == SRC_EXP) {
                f.d0 = load16(w8 + pos);
                f.sm = load16(mat(m).sm + pos);
            } else {
                f.nib = *reinterpret_cast<const u32x2_t*>(w8 + pos / 2);
                f.sm = load16(mat(m).sm + pos);
            }
        }
    };
    auto issue_v = [&](uint32_t s, LStage<MT, NT, NW, NMAT>& st) {
        if (SRC != SRC_PAL) return;
        const uint32_t k0 = s * kLS;
#pragma unroll
        for (int it = 0; it < IPT; ++it) {
            const int m = item_mat(it);
            const uint32_t pos = rowc[it] * C + k0 + koff;
            const uint32_t g = pos >> 6, bit = g & 63u;
            const uint32_t tl = (g >> 6) - t_base;
            const uint64_t word = tword[m][tl];
            LItem& f = st.w[it];
            f.verb = uint32_t(word >> bit) & 1u;
            const uint32_t slot = verbatim_slot(word, bit, tbase[m][tl]);
            const uint8_t* vb_ptr = mat(m).vexp ? mat(m).vexp : mat(m).sm;
            // lanes outside verbatim groups all read one shared line
            f.vx = load16(vb_ptr + (f.verb ? slot * 64u + (pos & 63u) : 0u));
        }
    };
    // commit: rebuild the step's weights into W buffer `buf` and store its
    // activation pieces into X buffer `buf`
    auto commit = [&](const LStage<MT, NT, NW, NMAT>& st, uint32_t buf) {
        uint16_t* xd = xl + buf * XBUF + xslot;
#pragma unroll
        for (int j = 0; j < XP; ++j) store16(xd + uint32_t(wave + NW * j) * 512u, st.x[j]);
#pragma unroll
        for (int it = 0; it < IPT; ++it) {
            const int m = item_mat(it);
            const LItem& f = st.w[it];
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
                for (int p = 0; p < 8; ++p) e7[p] = lut[m][(f.nib[p >> 2] >> (8 * (p & 3))) & 0xFFu];
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
            uint16_t* wd = wl[m] + buf * WBUF + item_rb(it) * (2u * 64u * 8u) + wslot;
            store16(wd, u32x4_t{w[0], w[1], w[2], w[3]});
            store16(wd + 16 * 8, u32x4_t{w[4], w[5], w[6], w[7]});
        }
    };

    const uint32_t wm = uint32_t(wave) / WGN, wn = uint32_t(wave) % WGN;
    f32x4_t acc[NMAT][FM][FN];
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
#pragma unroll
            for (int fn = 0; fn < FN; ++fn) acc[m][fm][fn] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // fragment reads: lane l takes chunk l/16 of row l%16 (swizzled slot)
    const uint32_t rq = uint32_t(lane >> 4), rr = uint32_t(lane & 15);
    const uint32_t wread0 = ((rr ^ (4u * ((rq >> 1) & 1u))) + 16u * rq) * 8u;
    const uint32_t wread1 = ((rr ^ (4u * ((rq >> 1) & 1u) + 10u)) + 16u * rq) * 8u + 512u;
    const uint32_t xread = ((rr ^ (4u * (rq & 1u) + 10u * (rq >> 1))) + 16u * rq) * 8u;
    // a step's fragments: read from LDS right after the barrier that makes
    // them visible, while the previous step's MFMAs still run
    struct Frags {
        bf16x8_t A[NMAT][2][FM], B[2][FN];
    };
    auto read_frags = [&](uint32_t buf, Frags& fr) {
        const uint16_t* xsrc = xl + buf * XBUF + xread;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
#pragma unroll
            for (int m = 0; m < NMAT; ++m)
#pragma unroll
            for (int fm = 0; fm < FM; ++fm)
                fr.A[m][h][fm] = *reinterpret_cast<const bf16x8_t*>(wl[m] + buf * WBUF + (wm * FM + fm) * 1024u +
                                                                    (h ? wread1 : wread0));
#pragma unroll
            for (int fn = 0; fn < FN; ++fn)
                fr.B[h][fn] = *reinterpret_cast<const bf16x8_t*>(xsrc + ((wn * FN + fn) * 2u + h) * 512u);
        }
    };
    auto mma = [&](const Frags& fr) {
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int m = 0; m < NMAT; ++m)
#pragma unroll
            for (int fm = 0; fm < FM; ++fm)
#pragma unroll
                for (int fn = 0; fn < FN; ++fn)
                    acc[m][fm][fn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fr.A[m][h][fm], fr.B[h][fn],
                                                                             acc[m][fm][fn], 0, 0, 0);
    };

    // Start: the first P steps' weight and activation loads go out first, then
    // the tables are staged (those loads are not waited for), then their
    // verbatim loads.  Steps past the slice re-issue its last step, so no load
    // is conditional.  Step u of the slice is staged in buffers u & 1.  In
    // the pass of step u: the loads of step u+P go out, step u's MFMAs run
    // on fragments already in registers, step u+1 is rebuilt into the other
    // buffers, a barrier, then step u+1's fragments are read.  The buffers
    // step u+1 is committed to were last read for step u-1, before the
    // barrier of the pass of step u-1.
    const uint32_t n = s_hi > s_lo ? s_hi - s_lo : 0u;
    const uint32_t first = n ? s_lo : 0u, last = n ? s_hi - 1u : 0u;
    LStage<MT, NT, NW, NMAT> st[NS];
#pragma unroll
    for (int j = 0; j < P; ++j) issue_w(min(first + j, last), st[j]);
    if (SRC == SRC_PAL) {
        for (uint32_t i = uint32_t(tid); i < nt; i += 64u * NW)
#pragma unroll
            for (int m = 0; m < NMAT; ++m) {
                tword[m][i] = mat(m).bitmap[t_base + i];
                tbase[m][i] = mat(m).tile_vbase[t_base + i];
            }
    }
    __syncthreads();                                   // LUT and tables ready
#pragma unroll
    for (int j = 0; j < P; ++j) issue_v(min(first + j, last), st[j]);
    Frags fr;
    if (n) commit(st[0], 0u);
    __syncthreads();
    if (n) read_frags(0u, fr);

    // main loop: NS steps per pass, every one followed by a commit (u + 1 <
    // n); step u's loads sit in set u % NS
    uint32_t u0 = 0;
    for (; u0 + NS < n; u0 += NS) {
#pragma unroll
        for (int j = 0; j < NS; ++j) {
            const uint32_t u = u0 + j;
            issue_w(min(first + u + P, last), st[(j + P) % NS]);
            issue_v(min(first + u + P, last), st[(j + P) % NS]);
            mma(fr);
            commit(st[(j + 1) % NS], (u + 1) & 1u);
            __syncthreads();
            read_frags((u + 1) & 1u, fr);
        }
    }
    // the last steps
#pragma unroll
    for (int j = 0; j < NS; ++j) {
        const uint32_t u = u0 + j;
        if (u < n) {
            if (u + P < n) {
                issue_w(first + u + P, st[(j + P) % NS]);
                issue_v(first + u + P, st[(j + P) % NS]);
            }
            mma(fr);
            if (u + 1 < n) {
                commit(st[(j + 1) % NS], (u + 1) & 1u);
                __syncthreads();
                read_frags((u + 1) & 1u, fr);
            }
        }
    }

    // D layout: lane l holds batch column l%16, rows 4*(l/16) .. +3
    const uint32_t col = lane & 15, q = uint32_t(lane) >> 4;
    if constexpr (DUAL) {
        // h = bf16(SiLU(g) * u), as uw_silu_mul_bf16 computes it; g and u too
        // when asked for
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) {
            const uint32_t r = band0 + (wm * FM + fm) * 16u + 4u * q;
#pragma unroll
            for (int fn = 0; fn < FN; ++fn) {
                const uint32_t b = n0 + (wn * FN + fn) * 16u + col;
                if (b >= B) continue;
                const f32x4_t gv = acc[0][fm][fn], uv = acc[1][fm][fn];
                uint32_t hb[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) hb[i] = f32_to_bf16_rne(silu_mul1(gv[i], uv[i]));
                const uint64_t o = uint64_t(b) * R + r;
                if (r + 3 < R && (R & 3u) == 0) {
                    *reinterpret_cast<u32x2_t*>(H + o) = u32x2_t{hb[0] | (hb[1] << 16), hb[2] | (hb[3] << 16)};
                    if (a.Y) *reinterpret_cast<f32x4_t*>(a.Y + o) = gv;
                    if (up.Y) *reinterpret_cast<f32x4_t*>(up.Y + o) = uv;
                } else {
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        if (r + i < R) {
                            H[o + i] = uint16_t(hb[i]);
                            if (a.Y) a.Y[o + i] = gv[i];
                            if (up.Y) up.Y[o + i] = uv[i];
                        }
                }
            }
        }
        return;
    }
    float* out = split > 1 ? a.partial + uint64_t(s_t) * a.B * a.R : a.Y;
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
        const uint32_t r = band0 + (wm * FM + fm) * 16u + 4u * q;
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
            const uint32_t b = n0 + (wn * FN + fn) * 16u + col;
            if (b >= B) continue;
            float* o = out + uint64_t(b) * R + r;
            const f32x4_t v = acc[0][fm][fn];
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

int lenv_int(const char* name, int dflt) {
    const char* e = getenv(name);
    return e && *e ? atoi(e) : dflt;
}

// Tile configurations: rows x batch columns per workgroup, waves, wave rows.
// Measured on the Llama MLP shapes on MI355X (gate 14336 x 4096, down 4096 x
// 14336), palette source, against the register-rebuilding tiled kernel:
// 128 x 64 at batch 64 (gate 29.5 against 33.1 us, down 27.7 against 32.7),
// 128 x 128 at batch 128 (38.0 against 45.8, 36.1 against 42.0), 128 x 256
// at batch 256 (56.0 against 68.2, 52.1 against 66.2).  Four-wave tiles of
// 64 rows (64 x 64 to 64 x 256) measured slower than all of these: each
// 64-row band streams the activations once more.
struct LCfg {
    int mt, nt, nw, wgm;
};
constexpr LCfg kLCfgs[] = {
    {128, 64, 8, 2},    // 0: 64 x 16 wave tiles
    {128, 128, 8, 2},   // 1: 64 x 32
    {128, 256, 8, 2},   // 2: 64 x 64
};
constexpr int kNLCfg = int(sizeof(kLCfgs) / sizeof(kLCfgs[0]));

// The configuration for a shape: by batch; above batch 128 the bf16 source
// and tall matrices (at least 8192 rows: enough 128 x 128 tiles to fill the
// chip without splitting K) keep 128 x 128 (gate at batch 256, bf16: 42.4
// against 48.1 us for 128 x 256), short matrices with the rebuilding sources
// take 128 x 256 (UW_LDS_CFG overrides).
int lds_cfg(int src, const MatArgs& a) {
    const int c = a.B <= 64 ? 0 : a.B <= 128 || src == SRC_BF16 || a.R >= 8192 ? 1 : 2;
    const int e = lenv_int("UW_LDS_CFG", c);
    return e < 0 || e >= kNLCfg ? c : e;
}

// Tiles of the band's verbatim tables (PAL): at most kLMaxTiles.
int64_t lds_tiles(int src, const MatArgs& a) { return (int64_t(kLCfgs[lds_cfg(src, a)].mt) * a.C + a.C) / 4096 + 2; }

template <int SRC, int MT, int NT, int NW, int WGM, int P>
void lds_launch_cfg(const MatArgs& a, hipStream_t s) {
    const int tiles_m = int((a.R + MT - 1) / MT), tiles_n = int((a.B + NT - 1) / NT);
    const int64_t grid = int64_t(tiles_m) * tiles_n * a.split_k;
    launch_timed(lds_gemm_kernel<SRC, MT, NT, NW, WGM, P>, dim3(unsigned(grid)), dim3(64 * NW), 0, s, a, a,
                 static_cast<uint16_t*>(nullptr), tiles_n, int(a.split_k), lenv_int("UW_LDS_ORDER", 1));
}

template <int SRC, int CI>
void lds_launch_ci(const MatArgs& a, hipStream_t s) {
    constexpr LCfg c = kLCfgs[CI];
    const int p = lenv_int("UW_LDS_P", 2);
    if (p <= 2) lds_launch_cfg<SRC, c.mt, c.nt, c.nw, c.wgm, 2>(a, s);
    else if (p == 3 || c.nt > 128) lds_launch_cfg<SRC, c.mt, c.nt, c.nw, c.wgm, 3>(a, s);
    else if (p <= 4) lds_launch_cfg<SRC, c.mt, c.nt, c.nw, c.wgm, (c.nt > 128 ? 3 : 4)>(a, s);
    else lds_launch_cfg<SRC, c.mt, c.nt, c.nw, c.wgm, (c.nt > 128 ? 3 : 6)>(a, s);
}

template <int SRC>
void lds_launch_src(const MatArgs& a, hipStream_t s) {
    switch (lds_cfg(SRC, a)) {
        case 0: lds_launch_ci<SRC, 0>(a, s); break;
        case 1: lds_launch_ci<SRC, 1>(a, s); break;
        default: lds_launch_ci<SRC, 2>(a, s); break;
    }
}

}  // namespace

bool lds_gemm_supported(int src, const MatArgs& a) {
    return a.C > 0 && a.C % kLS == 0 && (src != SRC_PAL || lds_tiles(src, a) <= kLMaxTiles);
}

// Whether the tiled MFMA family runs this kernel for a shape: above batch 64.
// At batch 64 the weight stream bounds the product and the register-staged
// tiled kernel's shorter step does better: the 32-layer Llama MLP stack took
// 3.54 ms here against 3.35 ms there (palette source), gate alone 24.9
// against 22.5 us (bf16).  UW_MFMA_LDS=0 turns it off, =1 takes it at every
// batch.
bool lds_gemm_preferred(int src, const MatArgs& a) {
    if (!lds_gemm_supported(src, a)) return false;
    const int e = lenv_int("UW_MFMA_LDS", -1);
    if (e == 0) return false;
    if (e == 1) return true;
    return a.B > 64;
}

// K-slices that give the launch about one workgroup per CU: the smallest
// power of two (at most 8, each slice at least 4 steps) for which tiles x
// slices reaches three quarters of the CUs.
int lds_gemm_default_split(int src, const MatArgs& a, int cus) {
    if (a.R <= 0 || a.B <= 0 || a.C <= 0) return 1;
    const LCfg c = kLCfgs[lds_cfg(src, a)];
    const int64_t tiles = ((a.R + c.mt - 1) / c.mt) * ((a.B + c.nt - 1) / c.nt);
    const int64_t steps = a.C / kLS;
    int split = 1;
    while (split < 8 && tiles * split * 4 < int64_t(cus) * 3 && steps / (2 * split) >= 4) split *= 2;
    return split;
}

// The gate/up pair on this kernel: palette sources of one shape whose band
// tables fit, above batch 32 (UW_GATEUP_LDS=0 turns it off,
// UW_GATEUP_LDS_MIN moves the threshold).  Bands of 64 rows, waves 0-3
// rebuilding gate and 4-7 up, 64 batch columns through batch 64, 128 through
// 128, 256 above (224 workgroups for the Llama gate/up shape through batch
// 256), K unsplit.  Measured on the Llama MLP stack (8 layers, MI355X)
// against two launches and the SiLU kernel: batch 48 0.758 against
// 0.86-0.90 ms, 64 0.813 against 0.93, 128 0.974 against 1.13-1.15, 256
// 1.398 against 1.67.  Bands of 128 rows (each weight rebuilt once per 64 or
// 128 batch columns) took 1.219 ms at batch 128 and 1.52-1.54 ms at 256.
bool lds_gateup_supported(const MatArgs& g, const MatArgs& u) {
    return g.R == u.R && g.C == u.C && g.B == u.B && g.B > lenv_int("UW_GATEUP_LDS_MIN", 32) &&
           lds_gemm_supported(SRC_PAL, g) && g.R * g.C < (int64_t(1) << 31) && g.B * g.C < (int64_t(1) << 31) &&
           g.B * g.R < (int64_t(1) << 31) && lenv_int("UW_GATEUP_LDS", 1) != 0;
}

template <int NT>
void lds_launch_pair(const MatArgs& g, const MatArgs& u, uint16_t* h, hipStream_t s) {
    const int tiles_m = int((g.R + 63) / 64), tiles_n = int((g.B + NT - 1) / NT);
    launch_timed(lds_gemm_kernel<SRC_PAL, 64, NT, 8, 2, 2, true>, dim3(unsigned(tiles_m * tiles_n)), dim3(512), 0, s,
                 g, u, h, tiles_n, 1, 1);
}

hipError_t launch_lds_gateup(const MatArgs& g, const MatArgs& u, uint16_t* h, hipStream_t s) {
    if (g.B <= 64) lds_launch_pair<64>(g, u, h, s);
    else if (g.B <= 128) lds_launch_pair<128>(g, u, h, s);
    else lds_launch_pair<256>(g, u, h, s);
    return hipGetLastError();
}

hipError_t launch_lds_gemm(int src, const MatArgs& a, hipStream_t s) {
    switch (src) {
        case SRC_BF16: lds_launch_src<SRC_BF16>(a, s); break;
        case SRC_EXP: lds_launch_src<SRC_EXP>(a, s); break;
        default: lds_launch_src<SRC_PAL>(a, s); break;
    }
    return hipGetLastError();
}

}  // namespace uwk
