// h = bf16(SiLU(g) * u): the step between the gate/up and down projections of
// a SwiGLU MLP (gate, up and down are the three matrices the Unweight page
// compresses, "How to compress model weights effectively").  fp32 math with
// HIP's expf; bf16 by round-to-nearest-even, NaN kept quiet.
#include "device_common.h"
#include "kernels.h"

namespace uwk {

namespace {

__global__ __launch_bounds__(256) void silu_mul_kernel(const float* __restrict__ g, const float* __restrict__ u,
                                                       int64_t n, uint16_t* __restrict__ h) {
    const int64_t i4 = (int64_t(blockIdx.x) * 256 + threadIdx.x) * 4;
    if (i4 + 4 <= n) {
        const f32x4_t gv = *reinterpret_cast<const f32x4_t*>(g + i4);
        const f32x4_t uv = *reinterpret_cast<const f32x4_t*>(u + i4);
        const uint32_t b0 = f32_to_bf16_rne(silu_mul1(gv[0], uv[0]));
        const uint32_t b1 = f32_to_bf16_rne(silu_mul1(gv[1], uv[1]));
        const uint32_t b2 = f32_to_bf16_rne(silu_mul1(gv[2], uv[2]));
        const uint32_t b3 = f32_to_bf16_rne(silu_mul1(gv[3], uv[3]));
        *reinterpret_cast<u32x2_t*>(h + i4) = u32x2_t{b0 | (b1 << 16), b2 | (b3 << 16)};
    } else {
        for (int64_t i = i4; i < n; ++i) h[i] = uint16_t(f32_to_bf16_rne(silu_mul1(g[i], u[i])));
    }
}

}  // namespace

hipError_t launch_silu_mul(const float* g, const float* u, int64_t n, uint16_t* h, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    const int64_t threads = (n + 3) / 4;
    silu_mul_kernel<<<unsigned((threads + 255) / 256), 256, 0, s>>>(g, u, n, h);
    return hipGetLastError();
}

}  // namespace uwk
