// Launch entry points of the gfx950 kernels, called by the C-ABI host code.
#pragma once

#include <hip/hip_runtime.h>

#include "common.h"

namespace sdpa {

// Kernels address the rows of one tile (at most 128) as 32-bit byte offsets
// from the tile's first row, so a row (sequence or token) stride must lie in
// [0, 2^23) elements; the host entry points reject other strides.
constexpr int64_t kMaxRowStride = (int64_t)1 << 23;
inline bool row_stride_ok(int64_t s) { return s >= 0 && s < kMaxRowStride; }

struct BwdLaunch {
    int dtype;            // 0 fp16, 1 bf16
    int D;                // head dim of Q and K: 64, 128 or 192
    int Dv;               // of V, O and dO: D, or 128 with D = 192
    bool causal;
    bool deterministic;
    int n_seq;            // batch (dense) or number of packed sequences
    int max_kv_tiles;     // ceil(max key length / 128)
    int max_kv_tiles64;   // ceil(max key length / 64)
    int max_q_tiles128;   // ceil(max query length / 128)
    int max_q_tiles64;    // ceil(max query length / 64)
    // Packed batches launch in chunks of sequences: the row-wise preprocess
    // runs with the first chunk, the dQ conversion with the last.
    static constexpr int kFirst = 1, kLast = 2;
    int phase = kFirst | kLast;
};

hipError_t launch_fwd(const FwdParams& p, int dtype, int D, int Dv, int max_lq, bool causal, hipStream_t st);
hipError_t launch_bwd(const BwdParams& p, const BwdLaunch& L, hipStream_t st);
// The D=128 backward (bwd128.hip) and the D=192 backward (bwd192.hip);
// launch_bwd hands those calls to them.
hipError_t launch_bwd_d128(const BwdParams& p, const BwdLaunch& L, hipStream_t st);
hipError_t launch_bwd_d192(const BwdParams& p, const BwdLaunch& L, hipStream_t st);
// The D=64 backward with FA2's fp32-atomic dQ accumulation (bwd128.hip's
// key-tile kernel at D=64 and the dQ conversion).
hipError_t launch_bwd_d64_atomic(const BwdParams& p, const BwdLaunch& L, hipStream_t st);
// Delta and log2-LSE per statistics row (and the dQ accumulator clear).
hipError_t launch_bwd_pre(const BwdParams& p, int dtype, int D, bool zero_dq, hipStream_t st);
// Sets the text sdpa_last_error() returns on this thread.
void set_last_error(const char* msg);

}  // namespace sdpa
