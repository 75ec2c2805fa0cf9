// Error reporting and the autotuner's plan table.
//
// The plan table holds, per device and (rows, cols, batch), the pipeline and kernel a
// measuring autotuner picked: the Unweight page ("Why no single pipeline
// wins") finds that the best of its four pipelines changes with batch size
// and with the matrix shape (gate/up against down), so the runtime picks per
// matrix and batch from measurements on the target hardware.
#include <cstdio>
#include <map>
#include <mutex>
#include <tuple>
#include <vector>

#include "uw_internal.h"

namespace {
thread_local std::string g_last_error;

struct PlanVal {
    int pipeline, kernel, split_k;
};
// Keyed by (device ordinal, rows, cols, batch): a choice measured on one
// device says nothing about another.
using PlanKey = std::tuple<int, int64_t, int64_t, int64_t>;
std::mutex g_plan_mu;
std::map<PlanKey, PlanVal> g_plan;

constexpr const char* kPlanMagic = "uwplan-v2";

// nullptr when (key, value) may enter the table, else what is wrong with it
const char* plan_entry_error(int64_t rows, int64_t cols, int64_t batch, int pipeline, int kernel, int split_k) {
    if (rows < 0 || cols < 0 || batch < 1) return "bad key";
    if (pipeline < UW_PIPE_FULL || pipeline > UW_PIPE_HUFF || pipeline == UW_PIPE_BF16)
        return "pipeline must be one of FULL/EXP/PAL/DIRECT/HUFF";
    if (kernel < UW_KERNEL_AUTO || kernel > UW_KERNEL_SKINNY || split_k < 1 || split_k > 64)
        return "bad kernel or split_k";
    return nullptr;
}
}  // namespace

namespace uw {
int fail(int code, const std::string& msg) {
    g_last_error = msg;
    return code;
}
void clear_error() { g_last_error.clear(); }
}  // namespace uw

extern "C" {

const char* uw_last_error(void) { return g_last_error.c_str(); }

int uw_abi_struct_sizes(uint64_t* info, uint64_t* dmat, uint64_t* opts) {
    if (info) *info = sizeof(uw_info);
    if (dmat) *dmat = sizeof(uw_dmat);
    if (opts) *opts = sizeof(uw_opts);
    return UW_OK;
}

int uw_plan_set(int64_t rows, int64_t cols, int64_t batch, int pipeline, int kernel, int split_k) {
    uw::clear_error();
    if (const char* why = plan_entry_error(rows, cols, batch, pipeline, kernel, split_k))
        return uw::fail(UW_EINVAL, std::string("uw_plan_set: ") + why);
    const int dev = uw::current_device();
    std::lock_guard<std::mutex> lk(g_plan_mu);
    g_plan[{dev, rows, cols, batch}] = {pipeline, kernel, split_k};
    return UW_OK;
}

int uw_plan_lookup(int64_t rows, int64_t cols, int64_t batch, int* pipeline, int* kernel, int* split_k) {
    uw::clear_error();
    if (!pipeline || !kernel || !split_k) return uw::fail(UW_EINVAL, "uw_plan_lookup: NULL argument");
    const int dev = uw::current_device();
    std::lock_guard<std::mutex> lk(g_plan_mu);
    auto it = g_plan.find({dev, rows, cols, batch});
    if (it == g_plan.end()) return uw::fail(UW_EINVAL, "uw_plan_lookup: no entry");
    *pipeline = it->second.pipeline;
    *kernel = it->second.kernel;
    *split_k = it->second.split_k;
    return UW_OK;
}

int uw_plan_clear(void) {
    std::lock_guard<std::mutex> lk(g_plan_mu);
    g_plan.clear();
    return UW_OK;
}

int uw_plan_count(void) {
    const int dev = uw::current_device();
    std::lock_guard<std::mutex> lk(g_plan_mu);
    int n = 0;
    for (auto& kv : g_plan) n += std::get<0>(kv.first) == dev;
    return n;
}

int uw_plan_save(const char* path) {
    uw::clear_error();
    if (!path) return uw::fail(UW_EINVAL, "uw_plan_save: NULL path");
    const int dev = uw::current_device();
    const std::string key = uw::device_key(dev);
    FILE* f = std::fopen(path, "w");
    if (!f) return uw::fail(UW_EINVAL, std::string("uw_plan_save: cannot open ") + path);
    std::fprintf(f, "%s %s\n", kPlanMagic, key.c_str());
    std::lock_guard<std::mutex> lk(g_plan_mu);
    for (auto& kv : g_plan)
        if (std::get<0>(kv.first) == dev)
            std::fprintf(f, "%lld %lld %lld %d %d %d\n", (long long)std::get<1>(kv.first),
                         (long long)std::get<2>(kv.first), (long long)std::get<3>(kv.first), kv.second.pipeline,
                         kv.second.kernel, kv.second.split_k);
    const bool ok = std::ferror(f) == 0;
    if (std::fclose(f) != 0 || !ok) return uw::fail(UW_EINVAL, std::string("uw_plan_save: write failed on ") + path);
    return UW_OK;
}

int uw_plan_load(const char* path) {
    uw::clear_error();
    if (!path) return uw::fail(UW_EINVAL, "uw_plan_load: NULL path");
    FILE* f = std::fopen(path, "r");
    if (!f) return uw::fail(UW_EINVAL, std::string("uw_plan_load: cannot open ") + path);
    char magic[32] = {}, saved[256] = {};
    if (std::fscanf(f, "%31s %255s", magic, saved) != 2 || std::string(magic) != kPlanMagic) {
        std::fclose(f);
        return uw::fail(UW_EFORMAT, std::string("uw_plan_load: ") + path + " does not start with '" + kPlanMagic +
                                        " <device>'");
    }
    const std::string key = uw::device_key(uw::current_device());
    if (key != saved) {
        std::fclose(f);
        return uw::fail(UW_EUNSUPPORTED, std::string("uw_plan_load: plan was tuned on ") + saved +
                                             ", the current device is " + key);
    }
    // parse everything first so that a malformed file leaves the table unchanged
    struct Row {
        long long r, c, b;
        int p, k, s;
    };
    std::vector<Row> rows;
    Row x;
    int n;
    while ((n = std::fscanf(f, "%lld %lld %lld %d %d %d", &x.r, &x.c, &x.b, &x.p, &x.k, &x.s)) == 6) rows.push_back(x);
    std::fclose(f);
    if (n != EOF) return uw::fail(UW_EFORMAT, "uw_plan_load: malformed line");
    for (const Row& e : rows)
        if (const char* why = plan_entry_error(e.r, e.c, e.b, e.p, e.k, e.s))
            return uw::fail(UW_EFORMAT, std::string("uw_plan_load: ") + why);
    const int dev = uw::current_device();
    std::lock_guard<std::mutex> lk(g_plan_mu);
    for (const Row& e : rows) g_plan[{dev, e.r, e.c, e.b}] = {e.p, e.k, e.s};
    return UW_OK;
}

}  // extern "C"
