// SDPA backward, FlashAttention-2 style, for gfx950: the D=128 kernels (and
// the D=64 key-tile kernel of the atomic dQ mode), instantiated from
// bwd_big.h in a translation unit of its own so that they take their own
// machine-scheduler strategy.
#include "bwd_big.h"

namespace sdpa {

hipError_t launch_bwd_d128(const BwdParams& p, const BwdLaunch& L, hipStream_t st) {
    return L.dtype == 0 ? launch_bwd_big_d<F16, 128, 128>(p, L, st) : launch_bwd_big_d<BF16, 128, 128>(p, L, st);
}

hipError_t launch_bwd_d64_atomic(const BwdParams& p, const BwdLaunch& L, hipStream_t st) {
    if (L.dtype == 0)
        return L.causal ? launch_bwd_atomic_t<F16, 64, true>(p, L, st) : launch_bwd_atomic_t<F16, 64, false>(p, L, st);
    return L.causal ? launch_bwd_atomic_t<BF16, 64, true>(p, L, st) : launch_bwd_atomic_t<BF16, 64, false>(p, L, st);
}

}  // namespace sdpa
