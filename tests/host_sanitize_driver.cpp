// Host-library exercise for the sanitizer build (AddressSanitizer +
// UndefinedBehaviorSanitizer, g++, CPU only): every host entry point of
// include/unweight.h on ordinary, ragged and degenerate matrices, serialized
// images with corrupted or truncated bytes, and the plan table.  Test
// infrastructure: it checks memory safety and a few structural facts of the
// format, not the codec's values (the Python oracle does that).
// Exit status 0 and "ok" on success; a sanitizer report or a message on the
// first failure otherwise.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <string>
#include <vector>

#include "unweight.h"

// The host sources take the device's identity for tuned plans from the HIP
// half of the library, which this CPU-only build does not link: here there
// is no device (what the library reports when none can be selected).
namespace uw {
int current_device() { return -1; }
std::string device_key(int) { return "none"; }
}  // namespace uw

namespace {

void need(bool ok, const std::string& what) {
    if (!ok) {
        std::fprintf(stderr, "FAIL: %s (%s)\n", what.c_str(), uw_last_error());
        std::exit(1);
    }
}

uint16_t bf16_bits(float f) {
    uint32_t u;
    std::memcpy(&u, &f, 4);
    return uint16_t((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);   // finite inputs only
}

std::vector<uint16_t> gaussian(int64_t rows, int64_t cols, float sigma, double p_out, uint64_t seed) {
    std::mt19937_64 rng(seed);
    std::normal_distribution<float> n(0.f, 1.f);
    std::uniform_real_distribution<double> u(0.0, 1.0);
    std::vector<uint16_t> w(size_t(rows * cols));
    for (auto& x : w) x = bf16_bits(u(rng) < p_out ? n(rng) * 4.f : n(rng) * sigma);
    return w;
}

std::vector<uint8_t> section(const uw_blob* b, int sec) {
    const void* p = nullptr;
    uint64_t n = 0;
    need(uw_blob_section(b, sec, &p, &n) == UW_OK, "uw_blob_section");
    const uint8_t* q = static_cast<const uint8_t*>(p);
    return n ? std::vector<uint8_t>(q, q + n) : std::vector<uint8_t>();
}

std::vector<uint8_t> serialize(const uw_blob* b) {
    uint64_t need_bytes = 0;
    need(uw_blob_serialize(b, nullptr, 0, &need_bytes) == UW_OK, "serialize size");
    std::vector<uint8_t> img(need_bytes);
    need(uw_blob_serialize(b, img.data(), img.size(), &need_bytes) == UW_OK, "serialize");
    if (need_bytes > 1)
        need(uw_blob_serialize(b, img.data(), need_bytes - 1, &need_bytes) == UW_EINVAL, "serialize into a short buffer");
    return img;
}

// One matrix through compress, validate, info, sections, serialize and
// deserialize, the host palette transcode, and a corrupted-image sweep.
void exercise(const std::vector<uint16_t>& w, int64_t rows, int64_t cols, const char* name, uint64_t seed) {
    const std::string tag = std::string(name) + " " + std::to_string(rows) + "x" + std::to_string(cols);
    uw_opts opts{1, 0};
    uw_blob* b = nullptr;
    need(uw_compress(w.data(), rows, cols, &opts, &b) == UW_OK, tag + ": compress");
    need(uw_validate(b) == UW_OK, tag + ": validate");
    uw_info info;
    need(uw_blob_info(b, &info) == UW_OK, tag + ": info");
    need(info.rows == rows && info.cols == cols && info.groups == rows * cols / 64, tag + ": info shape");
    need(info.palette_size >= 0 && info.palette_size <= 16 && info.lmax >= 0 && info.lmax <= 15, tag + ": code");

    const void* sp = nullptr;
    uint64_t sn = 0;
    need(uw_blob_section(b, UW_NUM_SECTIONS, &sp, &sn) != UW_OK && uw_blob_section(b, -1, &sp, &sn) != UW_OK,
         tag + ": section index out of range rejected");

    // the sign/mantissa plane is the input with the exponent bits masked out
    const std::vector<uint8_t> sm = section(b, UW_SEC_SM);
    need(int64_t(sm.size()) >= rows * cols, tag + ": sm size");
    for (int64_t i = 0; i < rows * cols; ++i) {
        const uint16_t x = w[size_t(i)];
        need(sm[size_t(i)] == uint8_t(((x >> 8) & 0x80u) | (x & 0x7Fu)), tag + ": sm byte");
    }

    // compressing with one thread gives the same sections
    uw_opts one{1, 1};
    uw_blob* b1 = nullptr;
    need(uw_compress(w.data(), rows, cols, &one, &b1) == UW_OK, tag + ": compress, one thread");
    for (int s = 0; s < UW_NUM_SECTIONS; ++s) need(section(b, s) == section(b1, s), tag + ": threads agree");
    uw_blob_free(b1);

    // the host palette transcode builds the NIB section compress emits
    uw_opts none{0, 0};
    uw_blob* b2 = nullptr;
    need(uw_compress(w.data(), rows, cols, &none, &b2) == UW_OK, tag + ": compress without NIB");
    need(section(b2, UW_SEC_NIB).empty(), tag + ": no NIB");
    need(uw_blob_add_palette(b2) == UW_OK, tag + ": add palette");
    need(section(b2, UW_SEC_NIB) == section(b, UW_SEC_NIB), tag + ": NIB");
    uw_blob_free(b2);

    // serialized image round trip
    const std::vector<uint8_t> img = serialize(b);
    uw_blob* b3 = nullptr;
    need(uw_blob_deserialize(img.data(), img.size(), &b3) == UW_OK, tag + ": deserialize");
    need(uw_validate(b3) == UW_OK, tag + ": validate after deserialize");
    for (int s = 0; s < UW_NUM_SECTIONS; ++s) need(section(b, s) == section(b3, s), tag + ": round trip");
    uw_blob_free(b3);

    // corrupted and truncated images: an error or a blob that validates,
    // never an out-of-bounds access
    std::mt19937_64 rng(seed);
    for (int k = 0; k < 300; ++k) {
        std::vector<uint8_t> bad = img;
        const int flips = 1 + int(rng() % 4);
        for (int f = 0; f < flips; ++f) {
            // mostly the 256-byte header and the small tables, sometimes anywhere
            const size_t lim = (rng() % 4) ? std::min<size_t>(bad.size(), 4096) : bad.size();
            bad[size_t(rng() % lim)] ^= uint8_t(1u << (rng() % 8));
        }
        if (rng() % 5 == 0) bad.resize(size_t(rng() % bad.size()));
        uw_blob* c = nullptr;
        const int rc = uw_blob_deserialize(bad.data(), bad.size(), &c);
        if (rc == UW_OK) {
            need(uw_validate(c) == UW_OK, tag + ": accepted image validates");
            uw_info ci;
            need(uw_blob_info(c, &ci) == UW_OK, tag + ": accepted image info");
            (void)serialize(c);
            uw_blob_free(c);
        } else {
            need(rc < 0 && c == nullptr, tag + ": rejected image yields no blob");
        }
    }
    uw_blob_free(b);
}

}  // namespace

int main() {
    // version and struct sizes
    {
        need(uw_version() > 0, "version");
        uint64_t si = 0, sd = 0, so = 0;
        need(uw_abi_struct_sizes(&si, &sd, &so) == UW_OK, "struct sizes");
        need(si == sizeof(uw_info) && sd == sizeof(uw_dmat) && so == sizeof(uw_opts), "struct sizes match");
        need(uw_abi_struct_sizes(nullptr, nullptr, nullptr) == UW_OK, "struct sizes, NULL pointers");
    }
    // argument errors
    {
        std::vector<uint16_t> w(64 * 3, 0x3C00);
        uw_blob* b = nullptr;
        need(uw_compress(w.data(), 3, 63, nullptr, &b) == UW_EINVAL && b == nullptr, "cols % 64 rejected");
        need(uw_compress(w.data(), -1, 64, nullptr, &b) == UW_EINVAL, "negative rows rejected");
        need(uw_compress(nullptr, 3, 64, nullptr, &b) == UW_EINVAL, "NULL weights rejected");
        need(uw_blob_deserialize(w.data(), 10, &b) != UW_OK && b == nullptr, "short image rejected");
        need(uw_validate(nullptr) != UW_OK, "NULL blob rejected");
        need(uw_blob_info(nullptr, nullptr) != UW_OK && uw_last_error()[0] != '\0', "NULL info reports an error");
        need(uw_blob_section(nullptr, UW_SEC_SM, nullptr, nullptr) != UW_OK, "NULL section rejected");
        uw_blob_free(nullptr);
    }
    // ordinary and ragged shapes
    const int64_t shapes[][2] = {{1, 64}, {3, 128}, {37, 1088}, {128, 4096}, {257, 192}, {64, 8192}};
    uint64_t seed = 1;
    for (const auto& s : shapes) {
        exercise(gaussian(s[0], s[1], 0.02f, 1e-3, seed), s[0], s[1], "gaussian", seed);
        ++seed;
    }
    // zero matrix rows
    {
        std::vector<uint16_t> none;
        uw_blob* b = nullptr;
        need(uw_compress(none.data(), 0, 128, nullptr, &b) == UW_OK && b, "zero rows");
        need(uw_validate(b) == UW_OK, "zero rows validate");
        (void)serialize(b);
        uw_blob_free(b);
    }
    // degenerate content: all zeros (one symbol), every group verbatim (more
    // than 16 exponents in each group), infinities, NaNs and subnormals
    {
        const int64_t R = 16, C = 256;
        std::vector<uint16_t> zeros(size_t(R * C), 0);
        exercise(zeros, R, C, "zeros", 101);
        std::vector<uint16_t> spread(size_t(R * C));
        for (int64_t i = 0; i < R * C; ++i) spread[size_t(i)] = uint16_t(((i % 64) * 4 + 1) << 7 | (i & 0x7F));
        exercise(spread, R, C, "all verbatim", 102);
        std::vector<uint16_t> special = gaussian(R, C, 0.02f, 0.0, 103);
        const uint16_t odd[] = {0x7F80, 0xFF80, 0x7FC0, 0xFFC1, 0x0001, 0x8001, 0x007F, 0x0000, 0x8000};
        for (size_t i = 0; i < special.size(); i += 37) special[i] = odd[(i / 37) % 9];
        exercise(special, R, C, "special", 103);
    }
    // plan table: set, look up, save, clear, load, and a file that is not a plan
    {
        need(uw_plan_clear() == UW_OK, "plan clear");
        need(uw_plan_set(14336, 4096, 1, UW_PIPE_DIRECT, UW_KERNEL_GEMV, 1) == UW_OK, "plan set");
        need(uw_plan_set(4096, 14336, 64, UW_PIPE_PAL, UW_KERNEL_MFMA, 8) == UW_OK, "plan set 2");
        need(uw_plan_count() == 2, "plan count");
        int p = 0, k = 0, s = 0;
        need(uw_plan_lookup(4096, 14336, 64, &p, &k, &s) == UW_OK && p == UW_PIPE_PAL && k == UW_KERNEL_MFMA && s == 8,
             "plan lookup");
        char path[] = "/tmp/uw_plan_XXXXXX";
        const int fd = mkstemp(path);
        need(fd >= 0, "temp file");
        std::fclose(fdopen(fd, "w"));
        need(uw_plan_save(path) == UW_OK, "plan save");
        need(uw_plan_clear() == UW_OK && uw_plan_count() == 0, "plan cleared");
        need(uw_plan_load(path) == UW_OK && uw_plan_count() == 2, "plan load");
        need(uw_plan_lookup(14336, 4096, 1, &p, &k, &s) == UW_OK && p == UW_PIPE_DIRECT, "plan after load");
        FILE* f = std::fopen(path, "w");
        need(f != nullptr, "rewrite temp file");
        std::fputs("not a plan\n\x01\x02 rows cols", f);
        std::fclose(f);
        (void)uw_plan_load(path);   // an error or an empty table; never a crash
        f = std::fopen(path, "w");
        need(f != nullptr, "rewrite temp file");
        std::fputs("uwplan-v2 none\n1 64 1 4 0 1\n1 64 2 4 0", f);   // truncated last entry
        std::fclose(f);
        need(uw_plan_clear() == UW_OK, "plan clear");
        need(uw_plan_load(path) == UW_EFORMAT && uw_plan_count() == 0, "truncated plan refused, table unchanged");
        f = std::fopen(path, "w");
        need(f != nullptr, "rewrite temp file");
        std::fputs("uwplan-v2 gfx000/1cu\n1 64 1 4 0 1\n", f);
        std::fclose(f);
        need(uw_plan_load(path) == UW_EUNSUPPORTED && uw_plan_count() == 0, "other device's plan refused");
        std::remove(path);
        need(uw_plan_clear() == UW_OK, "plan clear at end");
    }
    std::puts("ok");
    return 0;
}
