// Optional per-kernel timing with HIP events, for measurement tools.
//
// While enabled (sdpa_profile_begin .. sdpa_profile_end) every launch through
// PROF_LAUNCH records an event pair on the launch stream around the kernel.
// Disabled, the hooks cost one relaxed load per launch.
#pragma once

#include <hip/hip_runtime.h>

namespace sdpa {

enum KernelId {
    KID_FWD = 0,
    KID_BWD_PRE = 1,
    KID_BWD_MAIN = 2,
    KID_BWD_DQ_CONVERT = 3,
    KID_BWD_DQ_DET = 4,
    KID_NSA_INDEX = 5,
    KID_NSA_KV = 6,
    KID_NSA_DQ = 7,
    KID_BWD_FUSED = 8,
    KID_NSA_KV_REDUCE = 9,
    KID_COUNT = 10
};

bool prof_enabled();
void prof_mark(int kernel_id, hipStream_t st, bool start);

}  // namespace sdpa

#define PROF_LAUNCH(kid, st, ...)                                          \
    do {                                                                   \
        const bool prof_on_ = ::sdpa::prof_enabled();                      \
        if (prof_on_) ::sdpa::prof_mark((kid), (st), true);                \
        hipLaunchKernelGGL(__VA_ARGS__);                                   \
        if (prof_on_) ::sdpa::prof_mark((kid), (st), false);               \
    } while (0)
