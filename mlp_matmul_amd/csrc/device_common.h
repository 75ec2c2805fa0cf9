// Device helpers shared by the gfx950 kernels of libunweight.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace uwk {

constexpr int kWave = 64;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t bswap32(uint32_t v) {
    // byte reverse: selector picks bytes 3,2,1,0 of v
    return __builtin_amdgcn_perm(0u, v, 0x00010203u);
}

// Two bf16 weights (elements 2q and 2q+1 of a 4-element group) as one dword,
// low half = even element.  `sm4` holds 4 sign/mantissa bytes, `e7pair` the
// two exponents already shifted into bf16 position: e_even << 7 | e_odd << 23.
// sign -> bit 15, mantissa -> bits 6..0 of each half.
template <int Q>
__device__ __forceinline__ uint32_t join_pair(uint32_t sm4, uint32_t e7pair) {
    constexpr uint32_t sel = Q == 0 ? 0x01010000u : 0x03030202u;  // [a, a, b, b]
    uint32_t smp = __builtin_amdgcn_perm(0u, sm4, sel);
    return (smp & 0x807F807Fu) | e7pair;
}

// e_even << 7 | e_odd << 23 from exponent bytes 2Q, 2Q+1 of `e4`.
template <int Q>
__device__ __forceinline__ uint32_t exp_pair(uint32_t e4) {
    constexpr uint32_t sel = Q == 0 ? 0x010C000Cu : 0x030C020Cu;  // [0, a, 0, b]
    return __builtin_amdgcn_perm(0u, e4, sel) >> 1;
}

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                           __builtin_bit_cast(bf16x2_t, b), c, false);
}

// Sum over the 64 lanes of a wave; the total lands in every lane.  Butterfly
// within rows of 16 lanes through DPP row rotations, then across rows with
// lane permutes (2 of the 6 steps go through the LDS crossbar).
__device__ __forceinline__ float dpp_ror(float v, int n) {
    const int iv = __builtin_bit_cast(int, v);
    int r;
    switch (n) {
        case 1: r = __builtin_amdgcn_update_dpp(0, iv, 0x121, 0xF, 0xF, false); break;   // row_ror:1
        case 2: r = __builtin_amdgcn_update_dpp(0, iv, 0x122, 0xF, 0xF, false); break;   // row_ror:2
        case 4: r = __builtin_amdgcn_update_dpp(0, iv, 0x124, 0xF, 0xF, false); break;   // row_ror:4
        default: r = __builtin_amdgcn_update_dpp(0, iv, 0x128, 0xF, 0xF, false); break;  // row_ror:8
    }
    return __builtin_bit_cast(float, r);
}

__device__ __forceinline__ float wave_sum(float v) {
    v += dpp_ror(v, 8);
    v += dpp_ror(v, 4);
    v += dpp_ror(v, 2);
    v += dpp_ror(v, 1);        // every lane of a 16-lane row holds the row sum
    v += __shfl_xor(v, 16, kWave);
    v += __shfl_xor(v, 32, kWave);
    return v;
}

__device__ __forceinline__ uint32_t lane_id() { return __lane_id(); }

// Load 16 bytes with a streaming (non-temporal) hint: the data is read once.
__device__ __forceinline__ u32x4_t load_stream16(const void* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
}
__device__ __forceinline__ u32x2_t load_stream8(const void* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(p));
}
__device__ __forceinline__ u32x4_t load16(const void* p) {
    return *reinterpret_cast<const u32x4_t*>(p);
}
__device__ __forceinline__ void store16(void* p, u32x4_t v) {
    *reinterpret_cast<u32x4_t*>(p) = v;
}

// Index of a verbatim group among all verbatim groups: the count before its
// tile plus the flagged groups before it inside the tile's bitmap word.
// fp32 -> bf16 bits, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
    const uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (u >> 16) | 0x40u;
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// SiLU(g) * u in fp32 (HIP's expf): the SwiGLU step between gate/up and down.
__device__ __forceinline__ float silu_mul1(float g, float u) { return g / (1.0f + expf(-g)) * u; }

// Palette byte i (0..15) of the four packed palette words, selected without
// indexing: the words stay in scalar registers and no memory is read.
__device__ __forceinline__ uint32_t pal_byte(const uint32_t (&pal)[4], uint32_t i) {
    // readfirstlane keeps the four words opaque uniform values, so the selects
    // are not folded back into a load from a lane-dependent address
    const uint32_t p0 = __builtin_amdgcn_readfirstlane(pal[0]), p1 = __builtin_amdgcn_readfirstlane(pal[1]);
    const uint32_t p2 = __builtin_amdgcn_readfirstlane(pal[2]), p3 = __builtin_amdgcn_readfirstlane(pal[3]);
    const uint32_t lo = (i & 4u) ? p1 : p0;
    const uint32_t hi = (i & 4u) ? p3 : p2;
    return (((i & 8u) ? hi : lo) >> (8u * (i & 3u))) & 0xFFu;
}

__device__ __forceinline__ uint32_t verbatim_slot(uint64_t word, uint32_t bit, uint32_t vbase) {
    uint64_t below = bit ? (word & ((~0ull) >> (64 - bit))) : 0ull;
    return vbase + uint32_t(__popcll(below));
}

}  // namespace uwk
