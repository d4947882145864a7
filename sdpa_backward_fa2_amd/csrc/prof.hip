// Per-kernel timing (sdpa_profile_begin / sdpa_profile_end): event pairs that
// the runtime fills with each kernel's own dispatch timestamps.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>
#include <vector>

#include "../../include/sdpa_bwd.h"
#include "prof.h"

namespace sdpa {
namespace {

struct Mark {
    hipEvent_t start = nullptr, stop = nullptr;
    int kid = 0;
};

struct ProfState {
    std::atomic<bool> on{false};
    std::mutex mu;
    std::vector<Mark> pool;
    size_t used = 0;
    bool error = false;
};

ProfState& state() {
    static ProfState s;
    return s;
}

}  // namespace

bool prof_enabled() { return state().on.load(std::memory_order_relaxed); }

void prof_events(int kid, hipEvent_t* start, hipEvent_t* stop) {
    ProfState& s = state();
    std::lock_guard<std::mutex> lk(s.mu);
    *start = *stop = nullptr;
    if (s.used == s.pool.size()) {
        Mark m;
        if (hipEventCreate(&m.start) != hipSuccess || hipEventCreate(&m.stop) != hipSuccess) {
            s.error = true;
            return;
        }
        s.pool.push_back(m);
    }
    Mark& m = s.pool[s.used++];
    m.kid = kid;
    *start = m.start;
    *stop = m.stop;
}

}  // namespace sdpa

extern "C" {

int sdpa_profile_begin(void) {
    sdpa::ProfState& s = sdpa::state();
    std::lock_guard<std::mutex> lk(s.mu);
    s.used = 0;
    s.error = false;
    s.on.store(true);
    return SDPA_OK;
}

int sdpa_profile_end(int n_kernels, double* total_ms, int64_t* launches) {
    if (!total_ms || !launches) return SDPA_ERR_NULLPTR;
    if (n_kernels < 0) return SDPA_ERR_INVALID;
    sdpa::ProfState& s = sdpa::state();
    std::lock_guard<std::mutex> lk(s.mu);
    s.on.store(false);
    for (int i = 0; i < n_kernels; ++i) { total_ms[i] = 0.0; launches[i] = 0; }
    if (s.error) return SDPA_ERR_HIP;
    for (size_t i = 0; i < s.used; ++i) {
        sdpa::Mark& m = s.pool[i];
        if (hipEventSynchronize(m.stop) != hipSuccess) return SDPA_ERR_HIP;
        float ms = 0.f;
        if (hipEventElapsedTime(&ms, m.start, m.stop) != hipSuccess) return SDPA_ERR_HIP;
        if (m.kid < n_kernels) {
            total_ms[m.kid] += ms;
            launches[m.kid] += 1;
        }
    }
    s.used = 0;
    return SDPA_OK;
}

const char* sdpa_kernel_name(int kernel_id) {
    static const char* names[sdpa::KID_COUNT] = {
        "fwd_kernel", "bwd_pre_kernel", "bwd_main_kernel", "bwd_dq_convert_kernel",
        "bwd_dq8_kernel", "nsa_index_kernels", "nsa_kv_kernel", "nsa_dq_kernel",
        "bwd_fused8_kernel", "nsa_kv_reduce_kernel", "bwd_fused2_kernel"};
    if (kernel_id < 0 || kernel_id >= sdpa::KID_COUNT) return "";
    return names[kernel_id];
}

}  // extern "C"
