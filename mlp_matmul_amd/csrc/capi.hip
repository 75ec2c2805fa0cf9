// C ABI entry points of libunweight: argument checks, scratch layout,
// pipeline composition and kernel dispatch.  See unweight.h for the contract.
//
// Pipelines follow Cloudflare, "Unweight: how we compressed an LLM 22% without
// sacrificing quality", section "Four ways to use compressed weights":
//   full      Huffman decode -> bf16 in scratch -> plain bf16 matmul
//   exp       exponent-only decode -> u8 in scratch -> reconstructive matmul
//   pal       palette transcode -> nibbles in scratch -> reconstructive matmul
//   direct    reconstructive matmul on nibbles made once at load time
#include <algorithm>
#include <atomic>
#include <map>
#include <mutex>
#include <cstdlib>
#include <cstring>
#include <string>

#include "kernels.h"
#include "uw_internal.h"

namespace {

int hip_fail(hipError_t e, const char* what) {
    return uw::fail(UW_EHIP, std::string(what) + ": " + hipGetErrorString(e));
}

hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

uint64_t align256(uint64_t x) { return (x + 255) & ~uint64_t(255); }

void pack_palette(const uint8_t pal[16], uint32_t out[4]) {
    for (int i = 0; i < 4; ++i)
        out[i] = uint32_t(pal[4 * i]) | (uint32_t(pal[4 * i + 1]) << 8) | (uint32_t(pal[4 * i + 2]) << 16) |
                 (uint32_t(pal[4 * i + 3]) << 24);
}

int check_dmat(const uw_dmat* d, const char* who) {
    if (!d) return uw::fail(UW_EINVAL, std::string(who) + ": NULL descriptor");
    if (d->rows < 0 || d->cols < 0 || d->cols % uw::kGroup)
        return uw::fail(UW_EINVAL, std::string(who) + ": bad shape");
    if (d->groups != d->rows * d->cols / uw::kGroup || d->tiles != (d->groups + uw::kTile - 1) / uw::kTile)
        return uw::fail(UW_EINVAL, std::string(who) + ": inconsistent descriptor sizes");
    if (d->lmax < 0 || d->lmax > uw::kMaxCodeLen || d->palette_size < 0 || d->palette_size > 16)
        return uw::fail(UW_EINVAL, std::string(who) + ": bad code/palette size");
    return UW_OK;
}

int check_decoder_inputs(const uw_dmat* d, const char* who, bool need_sm) {
    int rc = check_dmat(d, who);
    if (rc) return rc;
    if (d->groups == 0) return UW_OK;
    if (!d->glen || !d->tile_off || !d->tile_vbase || !d->bitmap || !d->dlut || !d->mlut ||
        (d->stream_bytes && !d->stream) || (d->verbatim_groups && !d->vexp) || (need_sm && !d->sm))
        return uw::fail(UW_EINVAL, std::string(who) + ": a required device section is NULL");
    if (!aligned16(d->stream) || !aligned16(d->dlut) || !aligned16(d->mlut) || !aligned16(d->vexp) || !aligned16(d->sm))
        return uw::fail(UW_EINVAL, std::string(who) + ": device sections must be 16-byte aligned");
    // a tile holds at most 64 x 64 codewords of lmax bits
    if ((d->stream_bytes && d->max_tile_bytes == 0) ||
        d->max_tile_bytes > uint64_t(512) * uint64_t(d->lmax > 0 ? d->lmax : 1) + 1)
        return uw::fail(UW_EINVAL, std::string(who) + ": max_tile_bytes out of range for lmax");
    return UW_OK;
}

uwk::DecodeArgs decode_args(const uw_dmat* d, void* out) {
    uwk::DecodeArgs a{};
    a.sm = d->sm;
    a.stream = d->stream;
    a.glen = d->glen;
    a.tile_off = d->tile_off;
    a.tile_vbase = d->tile_vbase;
    a.vexp = d->vexp;
    a.bitmap = d->bitmap;
    a.dlut = d->dlut;
    a.mlut = d->mlut;
    a.stream_bytes = d->stream_bytes;
    a.max_tile_bytes = uint32_t(d->max_tile_bytes);
    a.G = d->groups;
    a.T = d->tiles;
    a.lmax = d->lmax;
    pack_palette(d->palette, a.pal);
    a.out = out;
    return a;
}

int run_decode(const uw_dmat* d, void* out, int mode, void* stream, const char* who) {
    uw::clear_error();
    int rc = check_decoder_inputs(d, who, mode == uwk::MODE_FULL);
    if (rc) return rc;
    if (d->groups && (!out || !aligned16(out)))
        return uw::fail(UW_EINVAL, std::string(who) + ": output must be a 16-byte aligned device pointer");
    hipError_t e = uwk::launch_decode(mode, decode_args(d, out), as_stream(stream));
    return e == hipSuccess ? UW_OK : hip_fail(e, who);
}

// Compute units of the current device (256 if it cannot be queried).
int device_cus() {
    static std::atomic<int> known[64];                 // per device, 0 until queried
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess) {
        (void)hipGetLastError();
        return 256;
    }
    if (dev >= 0 && dev < 64 && (cus = known[dev].load(std::memory_order_relaxed)) > 0) return cus;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) {
        (void)hipGetLastError();
        return 256;
    }
    if (dev >= 0 && dev < 64) known[dev].store(cus, std::memory_order_relaxed);
    return cus;
}

}  // namespace

namespace uw {
int current_device() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) {
        (void)hipGetLastError();
        return -1;
    }
    return dev;
}

std::string device_key(int ordinal) {
    if (ordinal < 0) return "none";
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, ordinal) != hipSuccess) {
        (void)hipGetLastError();
        return "none";
    }
    std::string arch(prop.gcnArchName);
    for (char& c : arch)
        if (c == ' ' || c == '\t' || c == '\n') c = '_';
    return arch + "/" + std::to_string(prop.multiProcessorCount) + "cu";
}
}  // namespace uw

namespace {

// The kernel family UW_KERNEL_AUTO picks for a shape.  Measured on MI355X
// (Llama MLP shapes): the GEMV wins at batch 1 (below batch 4 for bf16
// weights), the skinny MFMA kernel from there through 32 (the autotuner's
// choice at batch 32 on both shapes), the tiled kernel above.
int auto_kernel(int src, const uwk::MatArgs& a) {
    const int64_t gemv_below = src == uwk::SRC_BF16 ? 4 : 2;
    return a.B < gemv_below ? UW_KERNEL_GEMV
                            : (a.B <= 32 && uwk::mfma_gemv_supported(a) ? UW_KERNEL_SKINNY : UW_KERNEL_MFMA);
}

// split_k 0: the library's choice, K-slices for the tiled MFMA kernel that
// fill the chip (1 for the other kernels).
int resolve_split(int src, const uwk::MatArgs& a, int kernel, int split_k) {
    if (split_k != 0) return split_k;
    return kernel == UW_KERNEL_MFMA ? uwk::mfma_default_split(src, a, device_cus()) : 1;
}

// Common checks and dispatch of one matmul.
int run_matmul(int src, const uwk::MatArgs& a0, int kernel, int split_k, void* scratch, uint64_t scratch_bytes,
               void* stream, const char* who) {
    uwk::MatArgs a = a0;
    if (a.R < 0 || a.C < 0 || a.C % uw::kGroup || a.B < 0)
        return uw::fail(UW_EINVAL, std::string(who) + ": bad shape (cols must be a multiple of 64)");
    if (a.B > (int64_t(1) << 24) || a.R * a.C >= (int64_t(1) << 31) || a.B * a.C >= (int64_t(1) << 31) ||
        a.B * a.R >= (int64_t(1) << 31))
        return uw::fail(UW_EUNSUPPORTED, std::string(who) + ": size beyond the supported range");
    if (a.R == 0 || a.B == 0) return UW_OK;
    if (!a.X || !a.Y || !aligned16(a.X) || !aligned16(a.Y) || (a.R * a.C && (!a.w || !aligned16(a.w))))
        return uw::fail(UW_EINVAL, std::string(who) + ": NULL or misaligned device pointer");
    if (src != uwk::SRC_BF16 && a.R * a.C && (!a.sm || !aligned16(a.sm)))
        return uw::fail(UW_EINVAL, std::string(who) + ": sign/mantissa plane missing");
    if (src == uwk::SRC_PAL && a.R * a.C && (!a.bitmap || !a.tile_vbase))
        return uw::fail(UW_EINVAL, std::string(who) + ": verbatim tables missing");
    if (kernel == UW_KERNEL_AUTO) kernel = auto_kernel(src, a);
    if (kernel == UW_KERNEL_GEMV && a.B > 16)
        return uw::fail(UW_EINVAL, std::string(who) + ": the GEMV kernel takes batch <= 16");
    if (kernel == UW_KERNEL_SKINNY && !uwk::mfma_gemv_supported(a))
        return uw::fail(UW_EUNSUPPORTED, std::string(who) + ": the skinny MFMA kernel needs cols % 128 == 0 and cols <= 32768");
    if (kernel < UW_KERNEL_GEMV || kernel > UW_KERNEL_SKINNY)
        return uw::fail(UW_EINVAL, std::string(who) + ": unknown kernel");
    if (split_k < 0 || split_k > 64) return uw::fail(UW_EINVAL, std::string(who) + ": split_k must be 0..64");
    if (split_k == 0) {
        // the library's choice, as large as the scratch the caller gave allows
        split_k = resolve_split(src, a, kernel, 0);
        while (split_k > 1 && (!scratch || !aligned16(scratch) ||
                               scratch_bytes < uint64_t(split_k) * uint64_t(a.B) * uint64_t(a.R) * 4))
            split_k >>= 1;
    }
    a.cus = device_cus();
    if (kernel == UW_KERNEL_MFMA && !uwk::mfma_supported(a))
        return uw::fail(UW_EUNSUPPORTED, std::string(who) + ": the tiled MFMA kernel takes cols <= 65536");
    hipError_t e;
    if (kernel == UW_KERNEL_GEMV) {
        e = uwk::launch_gemv(src, a, as_stream(stream));
    } else if (kernel == UW_KERNEL_SKINNY) {
        e = uwk::launch_mfma_gemv(src, a, as_stream(stream));
    } else {
        a.split_k = split_k;
        if (split_k > 1) {
            const uint64_t need = uint64_t(split_k) * a.B * a.R * 4;
            if (!scratch || scratch_bytes < need || !aligned16(scratch))
                return uw::fail(UW_EINVAL, std::string(who) + ": split_k > 1 needs split_k*batch*rows*4 bytes of scratch");
            a.partial = static_cast<float*>(scratch);
        }
        e = uwk::launch_mfma(src, a, as_stream(stream));
    }
    return e == hipSuccess ? UW_OK : hip_fail(e, who);
}

uwk::MatArgs compressed_args(const uw_dmat* d, const void* w, const uint16_t* X, int64_t batch, float* Y) {
    uwk::MatArgs a{};
    a.w = w;
    a.sm = d->sm;
    a.vexp = d->vexp;
    a.bitmap = d->bitmap;
    a.tile_vbase = d->tile_vbase;
    a.X = X;
    a.Y = Y;
    a.R = d->rows;
    a.C = d->cols;
    a.B = batch;
    a.split_k = 1;
    pack_palette(d->palette, a.pal);
    return a;
}

// per-tile partial sums of the Huffman-decode GEMV: two floats per tile
uint64_t huff_partial_bytes(int64_t rows, int64_t cols) {
    const uint64_t n = uint64_t(rows) * uint64_t(cols);
    return 8 * ((n + 4095) / 4096);
}

uint64_t decoded_bytes(int pipeline, int64_t rows, int64_t cols) {
    const uint64_t n = uint64_t(rows) * uint64_t(cols);
    switch (pipeline) {
        case UW_PIPE_FULL: return 2 * n;
        case UW_PIPE_EXP: return n;
        case UW_PIPE_PAL: return n / 2;
        default: return 0;
    }
}

// UW_PIPE_HUFF: the decoder's GEMV mode (batch 1, cols >= 4096).
int huff_gemv(const uw_dmat* d, const uint16_t* X, int64_t batch, float* Y, void* scratch, uint64_t scratch_bytes,
              void* stream) {
    const char* who = "uw_matmul(UW_PIPE_HUFF)";
    if (batch < 0) return uw::fail(UW_EINVAL, std::string(who) + ": negative batch");
    if (d->rows == 0 || batch == 0) return UW_OK;
    if (batch != 1 || d->cols < 4096 || d->cols >= (int64_t(1) << 31))
        return uw::fail(UW_EUNSUPPORTED, std::string(who) + ": needs batch 1 and 4096 <= cols < 2^31");
    int rc = check_decoder_inputs(d, who, true);
    if (rc) return rc;
    if (!X || !Y || !aligned16(X) || !aligned16(Y))
        return uw::fail(UW_EINVAL, std::string(who) + ": NULL or misaligned X or Y");
    if (!scratch || !aligned16(scratch) || scratch_bytes < huff_partial_bytes(d->rows, d->cols))
        return uw::fail(UW_EINVAL, std::string(who) + ": scratch smaller than uw_scratch_bytes()");
    uwk::DecodeArgs a = decode_args(d, scratch);
    a.x = X;
    a.C = d->cols;
    hipError_t e = uwk::launch_decode_gemv(a, d->rows, Y, as_stream(stream));
    return e == hipSuccess ? UW_OK : hip_fail(e, who);
}

}  // namespace

// ------------------------------------------------------- one MLP block
// Scratch of uw_mlp_layer: a decoded plane per matrix (so the next matrix's
// decode can run while the current matmul reads its own), g and u (fp32),
// h (bf16), then the split-K partials of the matmuls (shared: they run one
// after another on the layer's stream).
struct MlpLayout {
    uint64_t dec[3], g, u, h, part, part_bytes, total;
};

MlpLayout mlp_layout(int pipeline, int64_t F, int64_t H, int64_t B) {
    MlpLayout l{};
    uint64_t off = 0;
    for (int m = 0; m < 3; ++m) {
        l.dec[m] = off;
        off += align256(decoded_bytes(pipeline, F, H));
    }
    l.g = off;
    off += align256(uint64_t(B) * uint64_t(F) * 4);
    l.u = off;
    off += align256(uint64_t(B) * uint64_t(F) * 4);
    l.h = off;
    off += align256(uint64_t(B) * uint64_t(F) * 2);
    l.part = off;
    // the split-K partials the library's split choice needs for either shape
    const int64_t pg = uw_scratch_bytes(UW_PIPE_DIRECT, F, H, B, 0), pd = uw_scratch_bytes(UW_PIPE_DIRECT, H, F, B, 0);
    l.part_bytes = align256(uint64_t(std::max<int64_t>(0, std::max(pg, pd))));
    l.total = off + l.part_bytes;
    return l;
}

int decode_for(const uw_dmat* d, int pipeline, void* dec, void* s) {
    switch (pipeline) {
        case UW_PIPE_FULL: return uw_decode_full(d, static_cast<uint16_t*>(dec), s);
        case UW_PIPE_EXP: return uw_decode_exponents(d, static_cast<uint8_t*>(dec), s);
        case UW_PIPE_PAL: return uw_transcode_palette(d, static_cast<uint8_t*>(dec), s);
        default: return UW_OK;
    }
}

// One matmul of the block from its decoded plane (UW_KERNEL_AUTO, split-K
// the library's choice within the partials area).
int matmul_from(const uw_dmat* d, int pipeline, const void* dec, const uint16_t* X, int64_t B, float* Y, void* part,
                uint64_t part_bytes, void* s) {
    switch (pipeline) {
        case UW_PIPE_FULL:
            return uw_gemm_bf16(static_cast<const uint16_t*>(dec), d->rows, d->cols, X, B, Y, UW_KERNEL_AUTO, 0, part,
                                part_bytes, s);
        case UW_PIPE_EXP:
            return uw_gemm_recon_exp(d, static_cast<const uint8_t*>(dec), X, B, Y, UW_KERNEL_AUTO, 0, part, part_bytes, s);
        case UW_PIPE_PAL:
            return uw_gemm_recon_pal(d, static_cast<const uint8_t*>(dec), X, B, Y, UW_KERNEL_AUTO, 0, part, part_bytes, s);
        default:
            return uw_gemm_recon_pal(d, d->nib, X, B, Y, UW_KERNEL_AUTO, 0, part, part_bytes, s);
    }
}

// Events that order the decode stream against the layer's stream: created
// once per host thread and device, re-recorded by every call (a wait takes
// the record made before it, so reuse across calls is safe).
struct LayerEvents {
    hipEvent_t start = nullptr, dec[3] = {nullptr, nullptr, nullptr};
};

int layer_events(LayerEvents** out) {
    thread_local std::map<int, LayerEvents> per_device;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "uw_mlp_layer");
    LayerEvents& ev = per_device[dev];
    if (!ev.start) {
        hipEvent_t made[4] = {};
        for (int i = 0; i < 4; ++i) {
            e = hipEventCreateWithFlags(&made[i], hipEventDisableTiming);
            if (e != hipSuccess) {
                for (int j = 0; j < i; ++j) (void)hipEventDestroy(made[j]);
                return hip_fail(e, "uw_mlp_layer");
            }
        }
        ev.start = made[0];
        for (int m = 0; m < 3; ++m) ev.dec[m] = made[m + 1];
    }
    *out = &ev;
    return UW_OK;
}

// ------------------------------------------------ allocation-free variant
// uw_gemm_recon_pal_static keeps the tiled kernel's split-K partial sums in
// this file-scope device array instead of caller scratch.  In host code the
// name `scratch` is only a stand-in for the array: its device address, one
// copy per GPU, comes from hipGetSymbolAddress and is what every launch gets.
static __device__ __align__(256) uint8_t scratch[UW_STATIC_SCRATCH_BYTES];

namespace {
std::mutex g_static_mu;
void* g_static_ptr[64];        // per device ordinal: the address of `scratch` there

int static_scratch(void** out, const char* who) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, who);
    if (dev < 0 || dev >= 64) return uw::fail(UW_EUNSUPPORTED, std::string(who) + ": device ordinal above 63");
    std::lock_guard<std::mutex> lk(g_static_mu);
    if (!g_static_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_fail(e, who);
        if (!p) return uw::fail(UW_EHIP, std::string(who) + ": no device address for the static scratch");
        g_static_ptr[dev] = p;
    }
    *out = g_static_ptr[dev];
    return UW_OK;
}
}  // namespace

extern "C" {

int uw_dmat_init(uw_dmat* d, const uw_info* info, const void* const dev[UW_NUM_SECTIONS]) {
    uw::clear_error();
    if (!d || !info || !dev) return uw::fail(UW_EINVAL, "uw_dmat_init: NULL argument");
    std::memset(d, 0, sizeof(*d));
    d->rows = info->rows;
    d->cols = info->cols;
    d->groups = info->groups;
    d->tiles = info->tiles;
    d->verbatim_groups = info->verbatim_groups;
    d->stream_bytes = info->section_bytes[UW_SEC_STREAM];
    d->max_tile_bytes = info->max_tile_bytes;
    d->palette_size = info->palette_size;
    d->lmax = info->lmax;
    std::memcpy(d->palette, info->palette, 16);
    d->sm = static_cast<const uint8_t*>(dev[UW_SEC_SM]);
    d->stream = static_cast<const uint8_t*>(dev[UW_SEC_STREAM]);
    d->glen = static_cast<const uint8_t*>(dev[UW_SEC_GLEN]);
    d->tile_off = static_cast<const uint32_t*>(dev[UW_SEC_TILE_OFF]);
    d->tile_vbase = static_cast<const uint32_t*>(dev[UW_SEC_TILE_VBASE]);
    d->vexp = static_cast<const uint8_t*>(dev[UW_SEC_VEXP]);
    d->bitmap = static_cast<const uint64_t*>(dev[UW_SEC_BITMAP]);
    d->nib = static_cast<const uint8_t*>(dev[UW_SEC_NIB]);
    d->dlut = static_cast<const uint8_t*>(dev[UW_SEC_DLUT]);
    d->mlut = static_cast<const uint32_t*>(dev[UW_SEC_MLUT]);
    return check_dmat(d, "uw_dmat_init");
}

int uw_decode_full(const uw_dmat* d, uint16_t* out_bf16, void* stream) {
    return run_decode(d, out_bf16, uwk::MODE_FULL, stream, "uw_decode_full");
}

int uw_decode_exponents(const uw_dmat* d, uint8_t* out_e, void* stream) {
    return run_decode(d, out_e, uwk::MODE_EXP, stream, "uw_decode_exponents");
}

int uw_transcode_palette(const uw_dmat* d, uint8_t* out_nib, void* stream) {
    return run_decode(d, out_nib, uwk::MODE_PAL, stream, "uw_transcode_palette");
}

int uw_gemm_bf16(const uint16_t* W, int64_t rows, int64_t cols, const uint16_t* X, int64_t batch, float* Y,
                 int kernel, int split_k, void* scratch, uint64_t scratch_bytes, void* stream) {
    uw::clear_error();
    uwk::MatArgs a{};
    a.w = W;
    a.X = X;
    a.Y = Y;
    a.R = rows;
    a.C = cols;
    a.B = batch;
    a.split_k = 1;
    return run_matmul(uwk::SRC_BF16, a, kernel, split_k, scratch, scratch_bytes, stream, "uw_gemm_bf16");
}

int uw_gemm_recon_exp(const uw_dmat* d, const uint8_t* e, const uint16_t* X, int64_t batch, float* Y, int kernel,
                      int split_k, void* scratch, uint64_t scratch_bytes, void* stream) {
    uw::clear_error();
    int rc = check_dmat(d, "uw_gemm_recon_exp");
    if (rc) return rc;
    return run_matmul(uwk::SRC_EXP, compressed_args(d, e, X, batch, Y), kernel, split_k, scratch, scratch_bytes,
                      stream, "uw_gemm_recon_exp");
}

int uw_gemm_recon_pal(const uw_dmat* d, const uint8_t* nib, const uint16_t* X, int64_t batch, float* Y, int kernel,
                      int split_k, void* scratch, uint64_t scratch_bytes, void* stream) {
    uw::clear_error();
    int rc = check_dmat(d, "uw_gemm_recon_pal");
    if (rc) return rc;
    if (d->groups && d->verbatim_groups && !d->vexp)
        return uw::fail(UW_EINVAL, "uw_gemm_recon_pal: verbatim exponents missing");
    return run_matmul(uwk::SRC_PAL, compressed_args(d, nib, X, batch, Y), kernel, split_k, scratch, scratch_bytes,
                      stream, "uw_gemm_recon_pal");
}

int64_t uw_scratch_bytes(int pipeline, int64_t rows, int64_t cols, int64_t batch, int split_k) {
    uw::clear_error();
    if (pipeline < UW_PIPE_FULL || pipeline > UW_PIPE_HUFF || rows < 0 || cols < 0 || batch < 0 || split_k < 0)
        return uw::fail(UW_EINVAL, "uw_scratch_bytes: bad argument");
    if (pipeline == UW_PIPE_HUFF) return int64_t(align256(huff_partial_bytes(rows, cols)));
    if (split_k == 0) {
        // the largest split_k 0 resolves to, over the weight sources, with
        // the kernel UW_KERNEL_AUTO picks
        uwk::MatArgs a{};
        a.R = rows;
        a.C = cols;
        a.B = batch;
        split_k = 1;
        if (cols % uw::kGroup == 0)
            for (int src : {uwk::SRC_BF16, uwk::SRC_EXP, uwk::SRC_PAL})
                split_k = std::max(split_k, resolve_split(src, a, auto_kernel(src, a), 0));
    }
    uint64_t n = align256(decoded_bytes(pipeline, rows, cols));
    if (split_k > 1) n += align256(uint64_t(split_k) * uint64_t(batch) * uint64_t(rows) * 4);
    return int64_t(n);
}

int uw_matmul(const uw_dmat* d, int pipeline, int kernel, int split_k, const uint16_t* X, int64_t batch, float* Y,
              void* scratch, uint64_t scratch_bytes, void* stream) {
    uw::clear_error();
    int rc = check_dmat(d, "uw_matmul");
    if (rc) return rc;
    if (pipeline == UW_PIPE_AUTO) {
        int p, k, s;
        if (uw_plan_lookup(d->rows, d->cols, batch, &p, &k, &s) == UW_OK) {
            pipeline = p;
            kernel = k;
            split_k = s;
        } else {
            pipeline = d->nib ? UW_PIPE_DIRECT : UW_PIPE_PAL;
            kernel = UW_KERNEL_AUTO;
            split_k = 0;
        }
        uw::clear_error();
    }
    if (pipeline == UW_PIPE_HUFF) return huff_gemv(d, X, batch, Y, scratch, scratch_bytes, stream);
    if (pipeline < UW_PIPE_FULL || pipeline > UW_PIPE_DIRECT)
        return uw::fail(UW_EINVAL, "uw_matmul: pipeline must be UW_PIPE_AUTO or FULL/EXP/PAL/DIRECT/HUFF");
    if (pipeline == UW_PIPE_DIRECT && d->groups && !d->nib)
        return uw::fail(UW_EINVAL, "uw_matmul: direct palette needs the NIB section on the device");
    // split_k 0 shrinks to what the scratch holds: only the decoded plane is required
    const int64_t need = uw_scratch_bytes(pipeline, d->rows, d->cols, batch, split_k == 0 ? 1 : split_k);
    if (need < 0) return int(need);
    if (uint64_t(need) > scratch_bytes || (need > 0 && (!scratch || !aligned16(scratch))))
        return uw::fail(UW_EINVAL, "uw_matmul: scratch smaller than uw_scratch_bytes()");
    uint8_t* dec = static_cast<uint8_t*>(scratch);
    const uint64_t dec_bytes = align256(decoded_bytes(pipeline, d->rows, d->cols));
    void* part = dec_bytes ? dec + dec_bytes : scratch;
    const uint64_t part_bytes = scratch_bytes - dec_bytes;
    switch (pipeline) {
        case UW_PIPE_FULL:
            rc = uw_decode_full(d, reinterpret_cast<uint16_t*>(dec), stream);
            if (rc) return rc;
            return uw_gemm_bf16(reinterpret_cast<uint16_t*>(dec), d->rows, d->cols, X, batch, Y, kernel, split_k, part,
                                part_bytes, stream);
        case UW_PIPE_EXP:
            rc = uw_decode_exponents(d, dec, stream);
            if (rc) return rc;
            return uw_gemm_recon_exp(d, dec, X, batch, Y, kernel, split_k, part, part_bytes, stream);
        case UW_PIPE_PAL:
            rc = uw_transcode_palette(d, dec, stream);
            if (rc) return rc;
            return uw_gemm_recon_pal(d, dec, X, batch, Y, kernel, split_k, part, part_bytes, stream);
        default:
            return uw_gemm_recon_pal(d, d->nib, X, batch, Y, kernel, split_k, part, part_bytes, stream);
    }
}

int uw_mlp_gate_up(const uw_dmat* gate, const uw_dmat* up, const uint16_t* X, int64_t batch, uint16_t* h,
                   float* g_out, float* u_out, void* stream) {
    uw::clear_error();
    const char* who = "uw_mlp_gate_up";
    if (!gate || !up) return uw::fail(UW_EINVAL, std::string(who) + ": NULL matrix");
    if (gate->rows != up->rows || gate->cols != up->cols || gate->rows < 0 || gate->cols % uw::kGroup)
        return uw::fail(UW_EINVAL, std::string(who) + ": gate and up must have the same shape (cols % 64 == 0)");
    if (batch < 0) return uw::fail(UW_EINVAL, std::string(who) + ": negative batch");
    if (gate->rows == 0 || batch == 0) return UW_OK;
    if (!X || !h || !aligned16(X) || !aligned16(h) || (g_out && !aligned16(g_out)) || (u_out && !aligned16(u_out)))
        return uw::fail(UW_EINVAL, std::string(who) + ": NULL or misaligned device pointer");
    for (const uw_dmat* d : {gate, up}) {
        int rc = check_dmat(d, who);
        if (rc) return rc;
        if (!d->nib || !d->sm || !d->bitmap || !d->tile_vbase || !aligned16(d->nib) || !aligned16(d->sm))
            return uw::fail(UW_EINVAL, std::string(who) + ": a matrix lacks its NIB/SM/BITMAP/TILE_VBASE sections");
        if (d->verbatim_groups && !d->vexp)
            return uw::fail(UW_EINVAL, std::string(who) + ": verbatim exponents missing");
    }
    uwk::MatArgs g = compressed_args(gate, gate->nib, X, batch, g_out);
    uwk::MatArgs u = compressed_args(up, up->nib, X, batch, u_out);
    g.cus = u.cus = device_cus();
    const bool small = gate->rows * gate->cols < (int64_t(1) << 31) && batch * gate->cols < (int64_t(1) << 31);
    // batch 1-2: the GEMV pair; 3-32: a skinny MFMA pair (measured on MI355X)
    static const int gemv_max = [] {
        const char* e = getenv("UW_GATEUP_GEMV_MAX");
        return e && *e ? atoi(e) : 2;
    }();
    hipError_t e;
    if (small && batch <= gemv_max && uwk::gemv_gateup_supported(g, u))
        e = uwk::launch_gemv_gateup(g, u, h, as_stream(stream));
    else if (small && uwk::mfma_gemv_gateup_supported(g, u))
        e = uwk::launch_mfma_gemv_gateup(g, u, h, as_stream(stream));
    else if (uwk::lds_gateup_supported(g, u))
        e = uwk::launch_lds_gateup(g, u, h, as_stream(stream));
    else
        return uw::fail(UW_EUNSUPPORTED, std::string(who) +
                                             ": needs batch 1..16, cols % 128 == 0, cols <= 32768 and a K-split of at "
                                             "most 4 for the shape (batch 1-2: or batch*cols*2 <= 32768; batch 17-32: "
                                             "at least 48 rows per compute unit), or batch above 32");
    return e == hipSuccess ? UW_OK : hip_fail(e, who);
}

int64_t uw_mlp_scratch_bytes(int pipeline, int64_t rows, int64_t cols, int64_t batch) {
    uw::clear_error();
    if (pipeline < UW_PIPE_FULL || pipeline > UW_PIPE_DIRECT || rows < 0 || cols < 0 || batch < 0 ||
        cols % uw::kGroup || rows % uw::kGroup)
        return uw::fail(UW_EINVAL, "uw_mlp_scratch_bytes: bad argument (rows and cols must be multiples of 64)");
    return int64_t(mlp_layout(pipeline, rows, cols, batch).total);
}

int uw_mlp_layer(const uw_dmat* gate, const uw_dmat* up, const uw_dmat* down, int pipeline, const uint16_t* X,
                 int64_t batch, float* y, void* scratch, uint64_t scratch_bytes, void* stream, void* aux_stream) {
    uw::clear_error();
    const char* who = "uw_mlp_layer";
    if (!gate || !up || !down) return uw::fail(UW_EINVAL, std::string(who) + ": NULL matrix");
    const int64_t F = gate->rows, H = gate->cols;
    if (up->rows != F || up->cols != H || down->rows != H || down->cols != F || F % uw::kGroup || H % uw::kGroup ||
        F < 0 || H < 0)
        return uw::fail(UW_EINVAL, std::string(who) + ": gate and up must be [F, H] and down [H, F], F and H multiples of 64");
    if (pipeline < UW_PIPE_FULL || pipeline > UW_PIPE_DIRECT)
        return uw::fail(UW_EINVAL, std::string(who) + ": pipeline must be UW_PIPE_FULL, EXP, PAL or DIRECT");
    if (batch < 0) return uw::fail(UW_EINVAL, std::string(who) + ": negative batch");
    if (batch == 0 || H == 0) return UW_OK;
    if (!X || !y || !aligned16(X) || !aligned16(y))
        return uw::fail(UW_EINVAL, std::string(who) + ": NULL or misaligned X or y");
    const MlpLayout l = mlp_layout(pipeline, F, H, batch);
    if (scratch_bytes < l.total || !scratch || !aligned16(scratch))
        return uw::fail(UW_EINVAL, std::string(who) + ": scratch smaller than uw_mlp_scratch_bytes()");
    uint8_t* base = static_cast<uint8_t*>(scratch);
    float* g = reinterpret_cast<float*>(base + l.g);
    float* u = reinterpret_cast<float*>(base + l.u);
    uint16_t* h = reinterpret_cast<uint16_t*>(base + l.h);
    void* part = base + l.part;
    const uw_dmat* mats[3] = {gate, up, down};
    void* dec[3] = {base + l.dec[0], base + l.dec[1], base + l.dec[2]};
    int rc;

    if (pipeline == UW_PIPE_DIRECT) {
        // nothing to decode; gate/up fused into one launch where it applies
        bool fused = false;
        if (batch <= 16) {
            rc = uw_mlp_gate_up(gate, up, X, batch, h, nullptr, nullptr, stream);
            if (rc && rc != UW_EUNSUPPORTED) return rc;
            fused = rc == UW_OK;
        }
        if (!fused) {
            if ((rc = matmul_from(gate, pipeline, nullptr, X, batch, g, part, l.part_bytes, stream))) return rc;
            if ((rc = matmul_from(up, pipeline, nullptr, X, batch, u, part, l.part_bytes, stream))) return rc;
            if ((rc = uw_silu_mul_bf16(g, u, batch * F, h, stream))) return rc;
        }
        return matmul_from(down, pipeline, nullptr, h, batch, y, part, l.part_bytes, stream);
    }

    if (!aux_stream) {
        // one stream: each matrix decoded right before its matmul
        for (int m = 0; m < 3; ++m) {
            if ((rc = decode_for(mats[m], pipeline, dec[m], stream))) return rc;
            const uint16_t* xin = m < 2 ? X : h;
            float* yout = m == 0 ? g : (m == 1 ? u : y);
            if ((rc = matmul_from(mats[m], pipeline, dec[m], xin, batch, yout, part, l.part_bytes, stream))) return rc;
            if (m == 1 && (rc = uw_silu_mul_bf16(g, u, batch * F, h, stream))) return rc;
        }
        return UW_OK;
    }

    // two streams: the three decodes run back to back on aux_stream (after
    // everything already on stream, which may still read this scratch), each
    // matmul on stream waits only for its own matrix's decode, so the decode
    // of up and down overlaps the gate and up matmuls
    LayerEvents* ev = nullptr;
    if ((rc = layer_events(&ev))) return rc;
    hipStream_t s = as_stream(stream), a = as_stream(aux_stream);
    hipError_t e = hipEventRecord(ev->start, s);
    if (e == hipSuccess) e = hipStreamWaitEvent(a, ev->start, 0);
    if (e != hipSuccess) return hip_fail(e, who);
    for (int m = 0; m < 3; ++m) {
        if ((rc = decode_for(mats[m], pipeline, dec[m], aux_stream))) return rc;
        if ((e = hipEventRecord(ev->dec[m], a)) != hipSuccess) return hip_fail(e, who);
    }
    for (int m = 0; m < 3; ++m) {
        if ((e = hipStreamWaitEvent(s, ev->dec[m], 0)) != hipSuccess) return hip_fail(e, who);
        const uint16_t* xin = m < 2 ? X : h;
        float* yout = m == 0 ? g : (m == 1 ? u : y);
        if ((rc = matmul_from(mats[m], pipeline, dec[m], xin, batch, yout, part, l.part_bytes, stream))) return rc;
        if (m == 1 && (rc = uw_silu_mul_bf16(g, u, batch * F, h, stream))) return rc;
    }
    return UW_OK;
}

int uw_gemm_recon_pal_static(const uw_dmat* d, const uint8_t* nib, const uint16_t* X, int64_t batch, float* Y,
                             int kernel, int split_k, void* stream) {
    uw::clear_error();
    const char* who = "uw_gemm_recon_pal_static";
    int rc = check_dmat(d, who);
    if (rc) return rc;
    if (d->groups && d->verbatim_groups && !d->vexp)
        return uw::fail(UW_EINVAL, std::string(who) + ": verbatim exponents missing");
    if (batch < 0 || split_k < 0 || split_k > 64) return uw::fail(UW_EINVAL, std::string(who) + ": bad batch or split_k");
    const uint64_t need = uint64_t(split_k > 1 ? split_k : 0) * uint64_t(batch) * uint64_t(d->rows) * 4;
    if (need > UW_STATIC_SCRATCH_BYTES)
        return uw::fail(UW_EINVAL, std::string(who) + ": split_k * batch * rows * 4 = " + std::to_string(need) +
                                       " bytes of partial sums exceed the static scratch of " +
                                       std::to_string(uint64_t(UW_STATIC_SCRATCH_BYTES)) + " bytes");
    void* p = nullptr;
    if ((rc = static_scratch(&p, who))) return rc;
    return run_matmul(uwk::SRC_PAL, compressed_args(d, nib, X, batch, Y), kernel, split_k, p, UW_STATIC_SCRATCH_BYTES,
                      stream, who);
}

int uw_silu_mul_bf16(const float* g, const float* u, int64_t n, uint16_t* h, void* stream) {
    uw::clear_error();
    if (n < 0) return uw::fail(UW_EINVAL, "uw_silu_mul_bf16: negative n");
    if (n == 0) return UW_OK;
    if (!g || !u || !h || !aligned16(g) || !aligned16(u) || !aligned16(h))
        return uw::fail(UW_EINVAL, "uw_silu_mul_bf16: NULL or misaligned pointer");
    hipError_t e = uwk::launch_silu_mul(g, u, n, h, as_stream(stream));
    return e == hipSuccess ? UW_OK : hip_fail(e, "uw_silu_mul_bf16");
}

}  // extern "C"
