// NSA selected-attention backward: placeholder entry points until the gathered
// kernels land.
#include <hip/hip_runtime.h>

#include "../../include/sdpa_bwd.h"

extern "C" {

int sdpa_bwd_selected_workspace_size(int, int64_t, const int64_t*, const int64_t*, int64_t, int64_t,
                                     int64_t, int64_t, int64_t, int, size_t*) {
    return SDPA_ERR_UNSUPPORTED;
}

int sdpa_bwd_selected(int, int64_t, const int64_t*, const int64_t*, int64_t, int64_t, int64_t, double,
                      int, const int32_t*, int64_t, int64_t, int64_t, int64_t, int64_t, int,
                      const sdpa_tensor3*, const sdpa_tensor3*, const sdpa_tensor3*, const sdpa_tensor3*,
                      const sdpa_tensor3*, const sdpa_stats*, const sdpa_tensor3*, const sdpa_tensor3*,
                      const sdpa_tensor3*, void*, size_t, void*) {
    return SDPA_ERR_UNSUPPORTED;
}

int sdpa_selected_build_index(int64_t, const int64_t*, const int64_t*, int64_t, const int32_t*, int64_t,
                              int64_t, int64_t, int64_t, int64_t, int32_t*, int32_t*, void*, size_t, void*) {
    return SDPA_ERR_UNSUPPORTED;
}

}
