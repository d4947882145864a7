// Optional per-kernel timing for measurement tools.
//
// While enabled (sdpa_profile_begin .. sdpa_profile_end) every launch through
// PROF_LAUNCH goes out through hipExtLaunchKernelGGL with a start/stop event
// pair: the runtime writes the kernel's own begin and end timestamps into the
// events from its dispatch packet, so the elapsed time is the kernel's
// execution time, without the extra stream packets (and the gaps they add)
// that events recorded around a launch bring.  Disabled, the hooks cost one
// relaxed load per launch and the launch is a plain hipLaunchKernelGGL.
#pragma once

#include <hip/hip_ext.h>
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
    KID_BWD_FUSED2 = 10,
    KID_COUNT = 11
};

bool prof_enabled();
// The event pair for the next launch of kernel_id (both null when no event
// could be created; the launch then goes out untimed and the run reports a
// HIP error at sdpa_profile_end).
void prof_events(int kernel_id, hipEvent_t* start, hipEvent_t* stop);

}  // namespace sdpa

#define PROF_LAUNCH(kid, st, kernel, grid, block, shmem, stream, ...)                       \
    do {                                                                                   \
        if (::sdpa::prof_enabled()) {                                                      \
            hipEvent_t prof_a_ = nullptr, prof_b_ = nullptr;                               \
            ::sdpa::prof_events((kid), &prof_a_, &prof_b_);                                \
            hipExtLaunchKernelGGL(kernel, grid, block, shmem, stream, prof_a_, prof_b_, 0, \
                                  __VA_ARGS__);                                            \
        } else {                                                                           \
            hipLaunchKernelGGL(kernel, grid, block, shmem, stream, __VA_ARGS__);           \
        }                                                                                  \
    } while (0)
