// Kernel argument blocks and launchers (host-callable) of libunweight.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace uwk {

// MODE_GEMV: Huffman decode inside a batch-1 matmul (no decoded output;
// per-tile partial sums of the rows the tile covers, cols >= 4096)
enum DecodeMode { MODE_FULL = 0, MODE_EXP = 1, MODE_PAL = 2, MODE_GEMV = 3 };
enum WeightSource { SRC_BF16 = 0, SRC_EXP = 1, SRC_PAL = 2 };

struct DecodeArgs {
    const uint8_t* sm;
    const uint8_t* stream;
    const uint8_t* glen;        // padded coded bits of each group / 4
    const uint32_t* tile_off;
    const uint32_t* tile_vbase;
    const uint8_t* vexp;
    const uint64_t* bitmap;
    const uint8_t* dlut;
    const uint32_t* mlut;
    uint64_t stream_bytes;
    uint32_t max_tile_bytes;
    int64_t G, T;
    int32_t lmax;
    int32_t buf_words;   // LDS dwords per wave for one staged tile stream
    uint32_t pal[4];     // palette bytes, index s in byte s%4 of pal[s/4]
    void* out;           // FULL/EXP/PAL: decoded plane; GEMV: partial sums float[2T]
    const uint16_t* x;   // GEMV: bf16 activation [C]
    int64_t C;           // GEMV: columns of the matrix; 4096: a tile is one row and out is y itself
};

// Weights of one matmul and where they come from.
struct MatArgs {
    const void* w;              // SRC_BF16: bf16 W; SRC_EXP: exponent plane; SRC_PAL: nibbles
    const uint8_t* sm;          // sign/mantissa plane (SRC_EXP, SRC_PAL)
    const uint8_t* vexp;        // SRC_PAL: verbatim exponents
    const uint64_t* bitmap;     // SRC_PAL: verbatim bitmap
    const uint32_t* tile_vbase; // SRC_PAL: verbatim groups before each tile
    const uint16_t* X;          // [B, C] bf16
    float* Y;                   // [B, R] fp32
    float* partial;             // split-K partial sums [split, B, R] (MFMA)
    int64_t R, C, B;
    int32_t split_k;
    int32_t row_groups;         // GEMV: groups of NRW rows one wave walks in turn
    int32_t cus;                // compute units of the device (launch shapes that fill it); 0: 256
    uint32_t pal[4];
};

hipError_t launch_decode(int mode, const DecodeArgs& a, hipStream_t s);
// Huffman decode inside a batch-1 matmul: a.out = partial sums float[2T],
// a.x the activation, a.C >= 4096; then y[r] summed per row in tile order.
hipError_t launch_decode_gemv(const DecodeArgs& a, int64_t rows, float* y, hipStream_t s);
hipError_t launch_gemv(int src, const MatArgs& a, hipStream_t s);
// Fused gate/up GEMV with the SiLU product (palette sources, batch 1..4).
bool gemv_gateup_supported(const MatArgs& gate, const MatArgs& up);
hipError_t launch_gemv_gateup(const MatArgs& gate, const MatArgs& up, uint16_t* h, hipStream_t s);
hipError_t launch_mfma(int src, const MatArgs& a, hipStream_t s);
bool mfma_supported(const MatArgs& a);
// Split-K that fills the chip for the tiled MFMA family on `cus` compute units.
int mfma_default_split(int src, const MatArgs& a, int cus);
// The tiled MFMA kernel that rebuilds each weight once per workgroup into a
// shared LDS tile (batch 64 and up by default; partial sums as launch_mfma).
bool lds_gemm_supported(int src, const MatArgs& a);
bool lds_gemm_preferred(int src, const MatArgs& a);
int lds_gemm_default_split(int src, const MatArgs& a, int cus);
hipError_t launch_lds_gemm(int src, const MatArgs& a, hipStream_t s);
// The fused gate/up pair with the SiLU product on that kernel (palette
// sources, batch above 64); g.Y / u.Y receive g and u when not NULL.
bool lds_gateup_supported(const MatArgs& g, const MatArgs& u);
hipError_t launch_lds_gateup(const MatArgs& g, const MatArgs& u, uint16_t* h, hipStream_t s);
hipError_t launch_mfma_gemv(int src, const MatArgs& a, hipStream_t s);
bool mfma_gemv_supported(const MatArgs& a);
// Fused gate/up on the skinny MFMA kernel with the SiLU product (palette
// sources, batch 1..16).
bool mfma_gemv_gateup_supported(const MatArgs& gate, const MatArgs& up);
hipError_t launch_mfma_gemv_gateup(const MatArgs& gate, const MatArgs& up, uint16_t* h, hipStream_t s);
// Skinny MFMA kernel with LDS-DMA operand streaming (palette sources, batch
// 1..32), single matrices and the gate/up pair.
bool skinny_dma_supported(const MatArgs& a);
// Whether the gate/up pair of this shape and batch takes this kernel (the
// library's choice, or forced by UW_SKINNY_DMA).
bool skinny_dma_pair_preferred(const MatArgs& a);
// Whether single matrices are forced onto this kernel (UW_SKINNY_DMA=1).
bool skinny_dma_forced();
hipError_t launch_skinny_dma(const MatArgs& a, hipStream_t s);
hipError_t launch_skinny_dma_gateup(const MatArgs& gate, const MatArgs& up, uint16_t* h, hipStream_t s);
hipError_t launch_silu_mul(const float* g, const float* u, int64_t n, uint16_t* h, hipStream_t s);

// LDS bytes the decoder needs for a code of longest length lmax.
size_t decode_lds_bytes(int lmax, uint32_t max_tile_bytes, int* buf_words);

// Kernel timer: while enabled, each matmul kernel launch takes the next
// (start, stop) event pair, recorded by the launch itself around the kernel.
bool timer_next(hipEvent_t* start, hipEvent_t* stop);

template <class K, class... Args>
void launch_timed(K kernel, dim3 grid, dim3 block, size_t lds, hipStream_t s, Args... args) {
    hipEvent_t e0, e1;
    if (timer_next(&e0, &e1))
        hipExtLaunchKernelGGL(kernel, grid, block, uint32_t(lds), s, e0, e1, 0, args...);
    else
        hipLaunchKernelGGL(kernel, grid, block, lds, s, args...);
}

}  // namespace uwk
