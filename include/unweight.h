/*
 * unweight.h -- C ABI of the MI355X (gfx950) compressed-MLP matmul library.
 *
 * The method: Cloudflare, "Unweight: how we compressed an LLM 22% without
 * sacrificing quality".
 *   - "How to compress model weights effectively": a bf16 weight's sign and
 *     mantissa are kept raw; its exponent byte is Huffman coded against the
 *     matrix's 16 most frequent exponents (the palette); a 64-element row that
 *     holds any other exponent is kept verbatim.
 *   - "Four ways to use compressed weights": full Huffman decode to bf16 then a
 *     plain matmul; exponent-only decode; runtime transcode to 4-bit palette
 *     indices; direct palette (indices made once at load time).  The last three
 *     feed a reconstructive matmul.
 *   - "How the reconstructive matmul works": the fused kernel reads compressed
 *     data, rebuilds bf16 on chip and multiplies; rebuilt weights never return
 *     to device memory.
 *   - "Why no single pipeline wins": the best pipeline depends on batch size
 *     and matrix shape and is picked per matrix x batch by measuring.
 *
 * Conventions
 *   - Every function returns int: UW_OK (0) or a negative UW_E* code, except
 *     where stated.  uw_last_error() returns a thread-local message for the
 *     last failure on the calling thread.  No C++ exception crosses the ABI.
 *   - A weight matrix W is [rows, cols] row-major bf16 bit patterns
 *     (uint16_t), the layout of torch.nn.Linear.weight (out x in).  cols must
 *     be a multiple of 64.  Activations X are [batch, cols] bf16 row-major;
 *     outputs Y are [batch, rows] fp32 row-major: Y = X . W^T, accumulated in
 *     fp32.
 *   - Host pointers are marked (host); every other pointer is a device
 *     pointer owned by the caller.  The library never allocates device
 *     memory; the caller allocates outputs and any scratch
 *     (uw_scratch_bytes).  Device buffers must be 16-byte aligned.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Device calls
 *     are asynchronous and stream ordered; errors found before launch are
 *     returned, launch failures surface as UW_EHIP.
 *   - Host blobs (uw_blob) are owned by the library and freed with
 *     uw_blob_free.
 *   - The pages define the operations, not an API.  Calls that cite a passage
 *     implement it; the rest are this library's own design decisions, marked
 *     "(API)": error text, versioning, blob access and serialization, the
 *     validator, scratch sizing, the device-matrix descriptor, the SiLU
 *     helper, the kernel timer and the plan-file format.
 */
#ifndef UNWEIGHT_H
#define UNWEIGHT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ------------------------------------------------------------ error codes */
#define UW_OK            0
#define UW_EINVAL       -1   /* bad argument (shape, pointer, mode) */
#define UW_ENOMEM       -2   /* host allocation failed */
#define UW_EFORMAT      -3   /* blob fails validation */
#define UW_EHIP         -4   /* HIP runtime error */
#define UW_EUNSUPPORTED -5   /* valid request the library does not handle */

/* (API) Thread-local text of the last error on this thread ("" if none). */
const char* uw_last_error(void);

/* (API) Library version, (major << 16) | minor. */
int uw_version(void);

/* (API) sizeof(uw_info), sizeof(uw_dmat), sizeof(uw_opts) as compiled, so a binding
 * can check its mirror of these structs (any pointer may be NULL). */
int uw_abi_struct_sizes(uint64_t* info, uint64_t* dmat, uint64_t* opts);

/* ------------------------------------------------------------- the format */
/* Sections of a compressed matrix.  N = rows*cols, G = N/64 groups of 64
 * consecutive elements of a row, T = ceil(G/64) tiles of 64 groups, V
 * verbatim groups.
 *   SM         uint8[N]    sign/mantissa byte, (sign << 7) | mantissa
 *   STREAM     uint8[S]    Huffman codes of the palette index of every element
 *                          of every non-verbatim group, MSB-first, each
 *                          group followed by zero bits up to a multiple of 4
 *                          bits; tile t starts at byte TILE_OFF[t]
 *   GLEN       uint8[G]    padded bits of each group / 4 (0 for verbatim
 *                          groups; at most 64*15/4 = 240): a group starts
 *                          4 * (sum of GLEN before it in its tile) bits after
 *                          its tile's first byte
 *   TILE_OFF   uint32[T+1] stream byte offset of each tile; [T] = S
 *   TILE_VBASE uint32[T+1] verbatim groups before each tile; [T] = V
 *   VEXP       uint8[64*V] raw exponent bytes of the verbatim groups, in order
 *   BITMAP     uint64[T]   bit (g % 64) of word g/64 set iff group g verbatim
 *   NIB        uint8[N/2]  direct-palette form: palette index of element i in
 *                          byte i/2, low nibble for even i; 0 in verbatim groups
 *   DLUT       uint8[2^L]  decode table (derived, not serialized): entry v =
 *                          (symbol << 4) | length of the codeword that prefixes
 *                          the L-bit string v, L = longest code length
 *   MLUT       uint32[4096] multi-symbol decode table (derived, not
 *                          serialized): entry v describes the codewords that
 *                          lie wholly inside the 12-bit string v, taken one
 *                          after another as DLUT decodes them, at most 4:
 *                          bits 0-7 their total length, bits 8-15 four times
 *                          their count, bits 16+4k the symbol of the k-th.
 *                          Count 0 means the first codeword is longer than
 *                          12 bits (decode it with DLUT). */
enum {
    UW_SEC_SM = 0,
    UW_SEC_STREAM,
    UW_SEC_GLEN,
    UW_SEC_TILE_OFF,
    UW_SEC_TILE_VBASE,
    UW_SEC_VEXP,
    UW_SEC_BITMAP,
    UW_SEC_NIB,
    UW_SEC_DLUT,
    UW_SEC_MLUT,
    UW_NUM_SECTIONS
};

typedef struct uw_blob uw_blob;

typedef struct {
    int emit_palette;   /* nonzero: also build the NIB section */
    int threads;        /* host threads for compression, 0 = all cores */
} uw_opts;

typedef struct {
    int64_t rows, cols;
    int64_t groups, tiles, verbatim_groups;
    int32_t palette_size;          /* P <= 16 */
    int32_t lmax;                  /* longest code length, <= 15 */
    uint8_t palette[16];           /* exponent of palette index s (0 unused) */
    uint8_t lengths[16];           /* code length of symbol s, 0 = no code */
    uint16_t codes[16];            /* canonical codeword of symbol s */
    uint64_t hist[256];            /* exponent histogram (0 after deserialize) */
    uint64_t section_bytes[UW_NUM_SECTIONS];
    uint64_t huffman_form_bytes;   /* header + all sections but NIB and DLUT */
    uint64_t palette_form_bytes;   /* header + SM + NIB + VEXP + BITMAP + TILE_VBASE */
    int32_t has_palette;           /* NIB section present */
    uint32_t max_tile_bytes;       /* longest tile of STREAM, bytes */
} uw_info;

/* Compress W (host, [rows, cols] bf16 bits) into a new blob.
 * Page: "How to compress model weights effectively" (field split, top-16
 * palette, Huffman-coded exponent, verbatim 64-element rows) and "Four ways to
 * use compressed weights" (the 4-bit form made at load time, opts->emit_palette).
 * opts may be NULL (no NIB, all cores).  UW_EINVAL if cols % 64 != 0 or a
 * size is negative; UW_ENOMEM on host allocation failure.  On success *out
 * owns the result (free with uw_blob_free). */
int uw_compress(const uint16_t* w /*host*/, int64_t rows, int64_t cols,
                const uw_opts* opts, uw_blob** out);

/* (API) Fill *info (host) from a blob. */
int uw_blob_info(const uw_blob* blob, uw_info* info);

/* (API) Borrow a host pointer to section `sec` and its byte size (pointer valid
 * until uw_blob_free; NULL with size 0 for an empty or absent section). */
int uw_blob_section(const uw_blob* blob, int sec, const void** ptr, uint64_t* bytes);

/* (API) Serialize to a byte image: a 256-byte header (magic "UWF2", format version
 * 2) then each stored section at a 256-byte aligned offset.  With buf == NULL
 * only *need is set.  UW_EINVAL if cap < *need. */
int uw_blob_serialize(const uw_blob* blob, void* buf /*host*/, uint64_t cap, uint64_t* need);

/* (API) Parse a serialized image into a new blob and validate it (UW_EFORMAT,
 * also for version-1 images, whose group lengths were 16-bit). */
int uw_blob_deserialize(const void* buf /*host*/, uint64_t bytes, uw_blob** out);

/* Build the NIB section of a blob that lacks it (host transcode). */
int uw_blob_add_palette(uw_blob* blob);

/* (API) Free a blob (NULL is a no-op). */
void uw_blob_free(uw_blob* blob);

/* (API) Structural checks before any launch: magic sizes, C % 64, palette size,
 * code lengths (Kraft equality, <= 15), monotone tile offsets, per-tile
 * sum of GLEN against the tile's bytes, verbatim groups coded with 0 bits,
 * bitmap popcounts against TILE_VBASE and VEXP, no bitmap bits past G.
 * UW_EFORMAT with a message on the first violation. */
int uw_validate(const uw_blob* blob);

/* ------------------------------------------------ device-resident matrices */
/* A compressed matrix whose sections the caller has copied to device memory.
 * Pointers of sections a call does not read may be NULL: the Huffman
 * decoders read SM (full mode only), STREAM, GLEN, TILE_OFF, TILE_VBASE,
 * VEXP, BITMAP, DLUT, MLUT; the palette-source matmul reads SM, NIB (or a
 * transcoded copy), VEXP, BITMAP, TILE_VBASE; the exponent-source matmul
 * reads SM and a decoded exponent plane. */
typedef struct {
    int64_t rows, cols, groups, tiles, verbatim_groups;
    uint64_t stream_bytes;
    uint64_t max_tile_bytes;       /* longest tile of STREAM (sizes the decoders' LDS) */
    int32_t palette_size, lmax;
    uint8_t palette[16];
    const uint8_t* sm;
    const uint8_t* stream;
    const uint8_t* glen;
    const uint32_t* tile_off;
    const uint32_t* tile_vbase;
    const uint8_t* vexp;
    const uint64_t* bitmap;
    const uint8_t* nib;
    const uint8_t* dlut;
    const uint32_t* mlut;
} uw_dmat;

/* (API) Fill a descriptor from blob info (host) and device section pointers
 * (dev[s] for section s, NULL where absent). */
int uw_dmat_init(uw_dmat* d, const uw_info* info, const void* const dev[UW_NUM_SECTIONS]);

/* ------------------------------------------------ preprocessing (decoders) */
/* Pipeline 1 preprocessing ("Four ways to use compressed weights", full
 * Huffman decode): rebuild every bf16 weight into out_bf16 [rows, cols].
 * One wavefront per 64-group tile; lanes find their group's first bit by a
 * prefix sum of GLEN and decode up to four codewords per lookup of MLUT; the
 * tile's stream and MLUT sit in LDS, the stream buffer sized by the
 * descriptor's max_tile_bytes.  UW_EINVAL when a section the decoder reads is
 * NULL, a section or the output is not 16-byte aligned, or max_tile_bytes is
 * 0 for a nonempty stream or above 512*lmax+1 (no tile of lmax-bit codes is
 * longer).  A STREAM whose tiles exceed max_tile_bytes decodes wrongly but
 * is never read or written out of bounds. */
int uw_decode_full(const uw_dmat* d, uint16_t* out_bf16, void* stream);

/* Pipeline 2 preprocessing (exponent-only decode): the exponent byte of every
 * weight, verbatim groups included, into out_e [rows, cols] uint8.  Same
 * decoder, layout rules and errors as uw_decode_full (SM is not read). */
int uw_decode_exponents(const uw_dmat* d, uint8_t* out_e, void* stream);

/* Pipeline 3 preprocessing (palette transcode), also the load-time producer of
 * pipeline 4's form: 4-bit palette indices into out_nib [rows*cols/2], byte
 * layout of the NIB section (0 in verbatim groups).  Same decoder, layout
 * rules and errors as uw_decode_full (SM is not read). */
int uw_transcode_palette(const uw_dmat* d, uint8_t* out_nib, void* stream);

/* ---------------------------------------------------------------- matmuls */
/* Kernel family selector for the matmuls (the autotuner's search space). */
enum {
    UW_KERNEL_AUTO = 0,    /* GEMV at batch 1 (below 4 for bf16 weights), SKINNY up to 32 (when supported), MFMA above */
    UW_KERNEL_GEMV = 1,    /* wavefront-reduction GEMV (v_dot2 bf16), batch <= 16 */
    UW_KERNEL_MFMA = 2,    /* tiled bf16 MFMA, any batch; cols <= 65536.  Through batch 64 each wave
                              rebuilds its own 16-row blocks in registers; above 64 eight waves share
                              each weight, rebuilt once into an LDS tile of 128 rows x 64/128/256
                              batch columns */
    UW_KERNEL_SKINNY = 3   /* bf16 MFMA, 16 rows x one K-slice per wave, batch tiles of <= 64;
                              needs cols % 128 == 0 and cols <= 32768 (else UW_EUNSUPPORTED) */
};

/* Uncompressed baseline and pipeline 1's consumer ("Four ways to use
 * compressed weights": the plain matmul after a full decode).
 * Y[batch, rows] = X[batch, cols] . W[rows, cols]^T, fp32 accumulate.
 * `kernel` is a UW_KERNEL_* value; split_k > 1 (MFMA only) needs
 * uw_scratch_bytes(UW_PIPE_BF16, ...) bytes of scratch, else scratch may be
 * NULL.  split_k 0 lets the library choose: for the tiled MFMA kernel the
 * smallest power of two up to 8 that gives about one workgroup per compute
 * unit, lowered to what the scratch holds; 1 for the other kernels.  The
 * reconstructive matmuls below take split_k the same way. */
int uw_gemm_bf16(const uint16_t* W, int64_t rows, int64_t cols,
                 const uint16_t* X, int64_t batch, float* Y,
                 int kernel, int split_k, void* scratch, uint64_t scratch_bytes,
                 void* stream);

/* Reconstructive matmul, exponent source (pipeline 2's consumer): weights
 * rebuilt on chip from the decoded exponent plane e [rows, cols] and d->sm.
 * ("How the reconstructive matmul works".) */
int uw_gemm_recon_exp(const uw_dmat* d, const uint8_t* e,
                      const uint16_t* X, int64_t batch, float* Y,
                      int kernel, int split_k, void* scratch, uint64_t scratch_bytes,
                      void* stream);

/* Reconstructive matmul, palette source (pipelines 3 and 4): weights rebuilt
 * on chip from 4-bit indices nib (NIB layout; d->nib for direct palette or a
 * uw_transcode_palette output), d->sm, and d->vexp for verbatim groups found
 * through d->bitmap and d->tile_vbase. */
int uw_gemm_recon_pal(const uw_dmat* d, const uint8_t* nib,
                      const uint16_t* X, int64_t batch, float* Y,
                      int kernel, int split_k, void* scratch, uint64_t scratch_bytes,
                      void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc):
 * uw_gemm_recon_pal with the tiled MFMA kernel's split-K partial sums kept in
 * a library-owned device array of UW_STATIC_SCRATCH_BYTES per GPU (reserved
 * on each device the library runs on until the process ends) instead of
 * caller scratch.  Same arguments, kernels and results as uw_gemm_recon_pal
 * with that scratch: bit-identical output for the same kernel and split_k.
 * split_k 0 takes the library's split lowered to what the array holds; an
 * explicit split_k > 1 with split_k * batch * rows * 4 above
 * UW_STATIC_SCRATCH_BYTES is UW_EINVAL.  Allocates nothing: no hipMalloc,
 * hipFree or allocating library call.  Every call on a GPU shares that GPU's
 * array, so calls that overlap on one GPU (on different streams, or from
 * several threads without ordering) race on it; calls ordered on one stream
 * are safe.  The array keeps the last call's partial sums (every launch writes
 * the partials it reads). */
#define UW_STATIC_SCRATCH_BYTES (64ull << 20)
int uw_gemm_recon_pal_static(const uw_dmat* d, const uint8_t* nib,
                             const uint16_t* X, int64_t batch, float* Y,
                             int kernel, int split_k, void* stream);

/* ------------------------------------------------------------- pipelines */
enum {
    UW_PIPE_AUTO = 0,     /* consult the plan table (uw_plan_*) */
    UW_PIPE_FULL = 1,     /* full decode -> bf16 scratch -> bf16 matmul */
    UW_PIPE_EXP = 2,      /* exponent decode -> u8 scratch -> recon matmul */
    UW_PIPE_PAL = 3,      /* palette transcode -> nibble scratch -> recon matmul */
    UW_PIPE_DIRECT = 4,   /* recon matmul on the resident NIB section */
    UW_PIPE_BF16 = 5,     /* uncompressed weights (baseline; not for uw_matmul) */
    UW_PIPE_HUFF = 6      /* Huffman decode inside a batch-1 matmul: the Huffman
                             form (the decoder's sections) read once, no decoded
                             plane; batch 1 and cols >= 4096 only (else
                             UW_EUNSUPPORTED); kernel and split_k are ignored;
                             scratch: 8 * ceil(rows*cols/4096) bytes of per-tile
                             partial sums, added per row in tile order (the
                             result is deterministic).  Goes past the page's four
                             pipelines ("Four ways to use compressed weights"):
                             its decode and matmul fused in one pass. */
};

/* (API) Scratch bytes uw_matmul needs for (pipeline, shape, batch, split_k)
 * (UW_PIPE_HUFF: the per-tile partial sums, whatever split_k);
 * split_k 0: for the split the library would choose with UW_KERNEL_AUTO on
 * the current device.  Returns the size (>= 0) or a negative error code. */
int64_t uw_scratch_bytes(int pipeline, int64_t rows, int64_t cols, int64_t batch, int split_k);

/* One matmul through a pipeline ("Four ways to use compressed weights").
 * UW_PIPE_AUTO looks up (rows, cols, batch) in the plan table and falls
 * back to UW_PIPE_DIRECT (or UW_PIPE_PAL without a NIB section) with
 * UW_KERNEL_AUTO and split_k 0.  scratch must hold uw_scratch_bytes(...)
 * bytes (with split_k 0: at least the split-1 size; a larger split is used
 * as far as the scratch allows).  UW_EINVAL on a too-small scratch. */
int uw_matmul(const uw_dmat* d, int pipeline, int kernel, int split_k,
              const uint16_t* X, int64_t batch, float* Y,
              void* scratch, uint64_t scratch_bytes, void* stream);

/* (API) h[i] = bf16_rne(SiLU(g[i]) * u[i]), SiLU(z) = z / (1 + exp(-z)), in
 * fp32; g, u fp32 [n], h bf16 bits [n].  The step between the gate/up and
 * down projections of a SwiGLU MLP (the MLP whose matrices "How to compress
 * model weights effectively" compresses; the page gives no formula for it). */
int uw_silu_mul_bf16(const float* g, const float* u, int64_t n, uint16_t* h, void* stream);

/* Fused gate/up projections of a SwiGLU MLP block on the direct-palette
 * form ("How the reconstructive matmul works": both compressed matrices are
 * rebuilt on chip inside one launch; the gate, up and down matrices are the
 * ones "How to compress model weights effectively" compresses):
 *   g = X . gate^T,  u = X . up^T  (fp32 accumulation), h[b][r] =
 *   bf16_rne(SiLU(g) * u) with the same SiLU arithmetic as uw_silu_mul_bf16.
 * Batch 1-2 runs the GEMV pair: g and u equal uw_gemm_recon_pal with
 * UW_KERNEL_GEMV bit for bit.  Batch 3-32 on matrices of at least 48 rows
 * per compute unit (12288 on MI355X) runs the pair on the skinny kernel that
 * streams its operands into LDS by DMA, which sums each output's K in one
 * wave (K unsplit up to 4096 columns): g and u are the same products as
 * uw_gemm_recon_pal with UW_KERNEL_SKINNY, summed in another order (equal
 * within the matmul's fp32 rounding, not bit for bit).  Other shapes at
 * batch 3-16 run the register-staged skinny pair: g and u equal
 * uw_gemm_recon_pal with UW_KERNEL_SKINNY bit for bit (same K-split).
 * Above batch 32 (other shapes and batches where the skinny pairs do not
 * apply) the pair runs on the tiled MFMA kernel that rebuilds each weight
 * once per workgroup into an LDS tile (64-row bands x 64, 128 or 256 batch
 * columns, K unsplit; both matrices share each activation tile): g and u
 * equal uw_gemm_recon_pal with UW_KERNEL_MFMA at split_k 1 above batch 64 bit
 * for bit (same K order), and that kernel forced (UW_MFMA_LDS=1) at 33-64.  In every case h is bit-identical
 * to uw_silu_mul_bf16 on the g, u the call computes.
 * gate, up: same shape [rows, cols], both with a NIB section; X bf16 bits
 * [batch, cols]; h bf16 bits [batch, rows]; g_out, u_out fp32 [batch, rows]
 * or NULL (not written).  Device pointers, 16-byte aligned, caller-owned.
 * UW_EINVAL on NULL/misaligned pointers, mismatched shapes, an inconsistent
 * descriptor, or verbatim groups without their VEXP section;
 * UW_EUNSUPPORTED unless cols % 128 == 0, cols <= 32768 and either
 * 1 <= batch <= 32 on a matrix of at least 48 rows per compute unit, or
 * 1 <= batch <= 16 and the library splits K at most 4 ways for this shape on
 * the current device (about one wave per SIMD: at least ~4096 rows on
 * MI355X), or, at batch 1-2, batch*cols*2 <= 32768 and cols <= 245760, or
 * batch above 32 with cols % 64 == 0 (and cols <= 20416, the verbatim
 * tables of a 128-row band in LDS). */
int uw_mlp_gate_up(const uw_dmat* gate, const uw_dmat* up, const uint16_t* X, int64_t batch,
                   uint16_t* h, float* g_out, float* u_out, void* stream);

/* (API) Scratch bytes of uw_mlp_layer for gate and up of shape [rows, cols] and
 * down of shape [cols, rows] (rows, cols multiples of 64): one decoded plane
 * per matrix, g and u (fp32), h (bf16), split-K partials.  Returns the size
 * or a negative error code. */
int64_t uw_mlp_scratch_bytes(int pipeline, int64_t rows, int64_t cols, int64_t batch);

/* One SwiGLU MLP block through one pipeline ("Four ways to use compressed
 * weights"), y = down . bf16(SiLU(X . gate^T) * (X . up^T)):
 * gate, up [F, H], down [H, F]; X bf16 bits [batch, H]; y fp32 [batch, F].
 * Each matmul runs with UW_KERNEL_AUTO and the library's split-K choice;
 * UW_PIPE_DIRECT fuses gate/up into one launch (uw_mlp_gate_up) where it
 * applies, with the same results except at batch 2, where the fused launch
 * is the GEMV pair (faster there on MI355X) while UW_KERNEL_AUTO alone would
 * take the skinny MFMA kernel (the two agree to rounding).
 * With aux_stream NULL every step runs on `stream`.  With an aux_stream (a
 * second stream of the caller's) and a decoding pipeline (FULL, EXP, PAL),
 * the three decodes run there, ordered after the work already on `stream`,
 * and each matmul waits only for its own matrix's decode, so decoding the
 * next matrix overlaps the current matmul (the page's "Why no single
 * pipeline wins": preprocessing adds to latency unless it overlaps).  All
 * results are ordered on `stream` when the call returns; y is bit-identical
 * to the one-stream order.  scratch: uw_mlp_scratch_bytes() bytes, device,
 * 16-byte aligned, caller-owned; calls that share a scratch must be ordered
 * on one `stream`.  Errors: UW_EINVAL (shapes, pipeline, NULL/misaligned
 * pointers, small scratch), UW_EHIP. */
int uw_mlp_layer(const uw_dmat* gate, const uw_dmat* up, const uw_dmat* down, int pipeline,
                 const uint16_t* X, int64_t batch, float* y,
                 void* scratch, uint64_t scratch_bytes, void* stream, void* aux_stream);

/* ----------------------------------------------------------- kernel timer */
/* (API) Per-launch durations of the matmul kernels (GEMV and MFMA), for measuring
 * them on their own stream.  While enabled, each matmul kernel launch takes
 * the next of `capacity` HIP event pairs, which the launch records at the
 * kernel's own start and end (hipExtLaunchKernel); launches beyond capacity
 * are not timed.  uw_kernel_timer_read waits for the recorded launches and
 * writes their durations in ms, in launch order (*count = launches recorded).
 * Process-global; enable from one thread at a time. */
int uw_kernel_timer_enable(int capacity);
int uw_kernel_timer_disable(void);
int uw_kernel_timer_reset(void);
int uw_kernel_timer_read(float* ms /*host*/, int max, int* count /*host*/);

/* --------------------------------------------------------------- autotune */
/* Plan table: (device, rows, cols, batch) -> (pipeline, kernel, split_k),
 * filled by a measuring autotuner ("Why no single pipeline wins": the best
 * pipeline is picked per matrix and batch by measuring).  The device is the
 * calling thread's current HIP device (set, lookup and count act on its
 * entries; clear empties the table for every device).  Process-global,
 * thread-safe.  pipeline: UW_PIPE_FULL..UW_PIPE_DIRECT or UW_PIPE_HUFF;
 * split_k 1..64.  lookup returns UW_EINVAL when the key is absent. */
int uw_plan_set(int64_t rows, int64_t cols, int64_t batch, int pipeline, int kernel, int split_k);
int uw_plan_lookup(int64_t rows, int64_t cols, int64_t batch, int* pipeline, int* kernel, int* split_k);
int uw_plan_clear(void);
int uw_plan_count(void);
/* Text file: a first line "uwplan-v2 <device>", <device> being
 * "<gcnArchName>/<compute units>cu" of the current device ("none" without
 * one), then one "rows cols batch pipeline kernel split_k" line per entry of
 * that device.  load rejects a file tuned on another device (UW_EUNSUPPORTED)
 * and a malformed one (UW_EFORMAT), leaving the table unchanged; UW_EINVAL
 * when the file cannot be opened or written. */
int uw_plan_save(const char* path /*host*/);
int uw_plan_load(const char* path /*host*/);

#ifdef __cplusplus
}
#endif

#endif /* UNWEIGHT_H */
