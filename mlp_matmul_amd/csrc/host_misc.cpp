// Error reporting and the autotuner's plan table.
//
// The plan table holds, per (rows, cols, batch), the pipeline and kernel a
// measuring autotuner picked: the Unweight page ("Why no single pipeline
// wins") finds that the best of its four pipelines changes with batch size
// and with the matrix shape (gate/up against down), so the runtime picks per
// matrix and batch from measurements on the target hardware.
#include <cstdio>
#include <map>
#include <mutex>
#include <tuple>

#include "uw_internal.h"

namespace {
thread_local std::string g_last_error;

struct PlanVal {
    int pipeline, kernel, split_k;
};
std::mutex g_plan_mu;
std::map<std::tuple<int64_t, int64_t, int64_t>, PlanVal> g_plan;
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
    if (rows < 0 || cols < 0 || batch < 1) return uw::fail(UW_EINVAL, "uw_plan_set: bad key");
    if (pipeline < UW_PIPE_FULL || pipeline > UW_PIPE_DIRECT)
        return uw::fail(UW_EINVAL, "uw_plan_set: pipeline must be one of UW_PIPE_FULL..UW_PIPE_DIRECT");
    if (kernel < UW_KERNEL_AUTO || kernel > UW_KERNEL_SKINNY || split_k < 1 || split_k > 64)
        return uw::fail(UW_EINVAL, "uw_plan_set: bad kernel or split_k");
    std::lock_guard<std::mutex> lk(g_plan_mu);
    g_plan[{rows, cols, batch}] = {pipeline, kernel, split_k};
    return UW_OK;
}

int uw_plan_lookup(int64_t rows, int64_t cols, int64_t batch, int* pipeline, int* kernel, int* split_k) {
    uw::clear_error();
    if (!pipeline || !kernel || !split_k) return uw::fail(UW_EINVAL, "uw_plan_lookup: NULL argument");
    std::lock_guard<std::mutex> lk(g_plan_mu);
    auto it = g_plan.find({rows, cols, batch});
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
    std::lock_guard<std::mutex> lk(g_plan_mu);
    return int(g_plan.size());
}

int uw_plan_save(const char* path) {
    uw::clear_error();
    if (!path) return uw::fail(UW_EINVAL, "uw_plan_save: NULL path");
    FILE* f = std::fopen(path, "w");
    if (!f) return uw::fail(UW_EINVAL, std::string("uw_plan_save: cannot open ") + path);
    std::lock_guard<std::mutex> lk(g_plan_mu);
    for (auto& kv : g_plan)
        std::fprintf(f, "%lld %lld %lld %d %d %d\n", (long long)std::get<0>(kv.first),
                     (long long)std::get<1>(kv.first), (long long)std::get<2>(kv.first), kv.second.pipeline,
                     kv.second.kernel, kv.second.split_k);
    std::fclose(f);
    return UW_OK;
}

int uw_plan_load(const char* path) {
    uw::clear_error();
    if (!path) return uw::fail(UW_EINVAL, "uw_plan_load: NULL path");
    FILE* f = std::fopen(path, "r");
    if (!f) return uw::fail(UW_EINVAL, std::string("uw_plan_load: cannot open ") + path);
    long long r, c, b;
    int p, k, s, n;
    int rc = UW_OK;
    while ((n = std::fscanf(f, "%lld %lld %lld %d %d %d", &r, &c, &b, &p, &k, &s)) == 6) {
        rc = uw_plan_set(r, c, b, p, k, s);
        if (rc != UW_OK) break;
    }
    if (rc == UW_OK && n != EOF) rc = uw::fail(UW_EFORMAT, "uw_plan_load: malformed line");
    std::fclose(f);
    return rc;
}

}  // extern "C"
