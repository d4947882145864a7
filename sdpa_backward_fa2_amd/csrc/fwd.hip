// Attention forward in training mode: O and the natural-log LSE per row.
//
// This produces the statistics the backward consumes (the cuDNN SDPA sample's
// forward graph with is_inference=False emits o and stats; forward-graph cell).
// It is a FlashAttention-style forward: each wavefront owns 32 query rows,
// keys stream through LDS 64 at a time, and a running max and sum give the
// softmax without materialising it.  Packed batches read each sequence's
// token range from the sequence table.  Scores are computed transposed
// (S^T = K Q^T) so that every lane holds one query column: row statistics are
// lane-local and need a single exchange with the other lane half.
#include "common.h"
#include "kernels.h"
#include "prof.h"

namespace sdpa {

// D: head dim of Q and K; DV: of V and O.
template <class T, int D, int DV, bool CAUSAL>
__global__ __launch_bounds__(256) void fwd_kernel(FwdParams p) {
    constexpr int BQ = 128;          // 4 wavefronts x 32 query rows
    constexpr int BK = 64;           // keys per LDS tile
    constexpr int KS = D / 16;       // k-steps over the Q/K head dimension
    constexpr int DB = DV / 32;      // 32-row blocks of O^T
    constexpr int KP = D + 8;        // padded row stride of Ks  [key][d]
    constexpr int VP = BK + 8;       // padded row stride of VT  [dv][key]
    __shared__ __align__(16) uint16_t Ks[BK * KP];
    __shared__ __align__(16) uint16_t VT[DV * VP];

    const int tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6;
    const int g = lane >> 5, c = lane & 31;
    const int bh = blockIdx.y;
    const int b = bh / p.Hq, h = bh % p.Hq;
    const int hk = h / (p.Hq / p.Hkv);
    int q0 = 0, k0 = 0, lq = p.Sq, lk = p.Sk;
    if (p.varlen) seq_get(p.seqs, b, q0, k0, lq, lk);
    const int i0 = blockIdx.x * BQ;
    if (i0 >= lq) return;

    const uint16_t* qp = p.q.p + b * p.q.sb + h * p.q.sh + (int64_t)q0 * p.q.ss;
    const uint16_t* kp = p.k.p + b * p.k.sb + hk * p.k.sh + (int64_t)k0 * p.k.ss;
    const uint16_t* vp = p.v.p + b * p.v.sb + hk * p.v.sh + (int64_t)k0 * p.v.ss;

    const int my_i = i0 + 32 * w + c;
    const bool row_ok = my_i < lq;
    u32x4 qreg[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) {
        u32x4 z = {0u, 0u, 0u, 0u};
        qreg[s] = row_ok ? ld16(qp + (int64_t)my_i * p.q.ss + 16 * s + 8 * g) : z;
    }

    float m = -INFINITY, l = 0.f;
    f32x16 o[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) o[db] = zero16();

    const int kend = CAUSAL ? min(lk, i0 + BQ) : lk;
    for (int j0 = 0; j0 < kend; j0 += BK) {
        __syncthreads();
        for (int e = tid; e < BK * D / 8; e += 256) {
            const int r = e / (D / 8), cc = (e % (D / 8)) * 8;
            const int j = j0 + r;
            u32x4 kv = {0u, 0u, 0u, 0u}, vv = {0u, 0u, 0u, 0u};
            if (j < lk) {
                kv = ld16(kp + (int64_t)j * p.k.ss + cc);
                if (DV == D) vv = ld16(vp + (int64_t)j * p.v.ss + cc);
            }
            st16(&Ks[r * KP + cc], kv);
            if (DV == D) {
#pragma unroll
                for (int t = 0; t < 8; ++t) VT[(cc + t) * VP + r] = elem16(vv, t);
            }
        }
        if (DV != D) {
            for (int e = tid; e < BK * DV / 8; e += 256) {
                const int r = e / (DV / 8), cc = (e % (DV / 8)) * 8;
                const int j = j0 + r;
                u32x4 vv = {0u, 0u, 0u, 0u};
                if (j < lk) vv = ld16(vp + (int64_t)j * p.v.ss + cc);
#pragma unroll
                for (int t = 0; t < 8; ++t) VT[(cc + t) * VP + r] = elem16(vv, t);
            }
        }
        __syncthreads();

        f32x16 s[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            s[kb] = zero16();
#pragma unroll
            for (int st = 0; st < KS; ++st)
                s[kb] = T::mma(ld16(&Ks[(kb * 32 + c) * KP + 16 * st + 8 * g]), qreg[st], s[kb]);
        }
        // scale into the log2 domain, mask, and find the tile's row max
        float tmax = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int rg = 0; rg < 16; ++rg) {
                const int j = j0 + kb * 32 + 8 * (rg >> 2) + 4 * g + (rg & 3);
                float x = s[kb][rg] * p.scale_log2;
                if (j >= lk || (CAUSAL && j > my_i)) x = -INFINITY;
                s[kb][rg] = x;
                tmax = fmaxf(tmax, x);
            }
        tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
        const float m_new = fmaxf(m, tmax);
        const float msub = (m_new == -INFINITY) ? 0.f : m_new;
        const float alpha = (m == -INFINITY) ? 0.f : fast_exp2(m - m_new);
        float rs = 0.f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int rg = 0; rg < 16; ++rg) {
                const float pv = fast_exp2(s[kb][rg] - msub);
                s[kb][rg] = pv;
                rs += pv;
            }
        rs += __shfl_xor(rs, 32);
        l = l * alpha + rs;
        m = m_new;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int rg = 0; rg < 16; ++rg) o[db][rg] *= alpha;
        // O^T += V^T P^T, contracted over the 64 keys in four 16-key steps
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                const u32x4 bop = acc_to_operand<T>(s[kb], hh);
#pragma unroll
                for (int db = 0; db < DB; ++db)
                    o[db] = T::mma(ld_acc_slots(&VT[(db * 32 + c) * VP + kb * 32 + 16 * hh], g), bop, o[db]);
            }
    }

    if (!row_ok) return;
    const float inv_l = l > 0.f ? 1.f / l : 0.f;
    uint16_t* op = p.o.p + b * p.o.sb + h * p.o.sh + (int64_t)(q0 + my_i) * p.o.ss;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            u32x2 v2;
            v2[0] = T::pack(o[db][4 * q + 0] * inv_l, o[db][4 * q + 1] * inv_l);
            v2[1] = T::pack(o[db][4 * q + 2] * inv_l, o[db][4 * q + 3] * inv_l);
            st8(op + db * 32 + 8 * q + 4 * g, v2);
        }
    if (g == 0) {
        const float lse = l > 0.f ? (m + log2f(l)) * kLn2 : -INFINITY;
        p.lse[b * p.lse_sb + h * p.lse_sh + (int64_t)(q0 + my_i) * p.lse_ss] = lse;
    }
}

// grid.x covers the longest sequence (dense: Sq) in 128-row tiles
template <class T, int D, int DV>
static hipError_t launch_fwd_t(const FwdParams& p, int max_lq, bool causal, hipStream_t st) {
    dim3 grid((max_lq + 127) / 128, p.B * p.Hq);
    if (causal)
        PROF_LAUNCH(KID_FWD, st, (fwd_kernel<T, D, DV, true>), grid, dim3(256), 0, st, p);
    else
        PROF_LAUNCH(KID_FWD, st, (fwd_kernel<T, D, DV, false>), grid, dim3(256), 0, st, p);
    return hipGetLastError();
}

template <class T>
static hipError_t launch_fwd_dt(const FwdParams& p, int D, int Dv, int max_lq, bool causal, hipStream_t st) {
    if (D == 64) return launch_fwd_t<T, 64, 64>(p, max_lq, causal, st);
    if (D == 128) return launch_fwd_t<T, 128, 128>(p, max_lq, causal, st);
    if (Dv == 128) return launch_fwd_t<T, 192, 128>(p, max_lq, causal, st);
    return launch_fwd_t<T, 192, 192>(p, max_lq, causal, st);
}

hipError_t launch_fwd(const FwdParams& p, int dtype, int D, int Dv, int max_lq, bool causal, hipStream_t st) {
    return dtype == 0 ? launch_fwd_dt<F16>(p, D, Dv, max_lq, causal, st)
                      : launch_fwd_dt<BF16>(p, D, Dv, max_lq, causal, st);
}

}  // namespace sdpa
