// SDPA backward, FlashAttention-2 style, for gfx950: the Dqk = 192 kernels of
// the dense and packed paths, Dv = 192 or 128 (the key-tile kernel and the
// atomic-free dQ pass),
// instantiated from bwd_big.h.  A translation unit of its own: these kernels
// run one wavefront per SIMD at the full 512 registers, and the build gives
// this file the default machine scheduler.
#include "bwd_big.h"

namespace sdpa {

hipError_t launch_bwd_d192(const BwdParams& p, const BwdLaunch& L, hipStream_t st) {
    if (L.Dv == 128)
        return L.dtype == 0 ? launch_bwd_big_d<F16, 192, 128>(p, L, st) : launch_bwd_big_d<BF16, 192, 128>(p, L, st);
    return L.dtype == 0 ? launch_bwd_big_d<F16, 192, 192>(p, L, st) : launch_bwd_big_d<BF16, 192, 192>(p, L, st);
}

}  // namespace sdpa
