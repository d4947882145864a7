// SDPA backward, FlashAttention-2 style, for gfx950.
//
// Kernels (all on the caller's stream):
//   bwd_pre_kernel     per row: Delta = sum_d dO*O, the statistics turned into
//                      log2-domain LSE, and (atomic mode) the fp32 dQ
//                      accumulator row cleared.                   [HBM-bound]
//   bwd_main_kernel    one workgroup per (sequence, KV head, 128-key tile): K
//                      and V of the tile stay in registers, dK and dV
//                      accumulate in registers across every query tile of
//                      every query head of the group; per 64-row query tile it
//                      runs the five contractions S = Q K^T, dP = dO V^T,
//                      dV += P^T dO, dK += dS^T Q, dQ += dS K (the last through
//                      fp32 atomics, or skipped in deterministic mode). [MFMA]
//   bwd_dq_convert     dQ = scale * accumulator, rounded to the I/O type.
//   bwd_dq_kernel      deterministic dQ: query-tile outer, recomputes S, P, dP
//                      and dS per key tile and keeps dQ in registers.
//
// The formulas: dV = P^T dO, dQ = s dS K, dK = s dS^T Q (Ascend
// aclnnNsaSelectedAttentionGrad page, "Formula" section), with
// dS = P o (dP - Delta), Delta_i = sum_j P_ij dP_ij = sum_d dO_id O_id, the
// softmax gradient written with the forward output instead of P.
#include "common.h"
#include "kernels.h"
#include "prof.h"

namespace sdpa {

// ---------------------------------------------------------------------------
// Row location helpers
// ---------------------------------------------------------------------------

struct RowLoc {
    int64_t b, h, i;   // dense: batch, head, row; packed: b = 0, i = token
};

__device__ __forceinline__ RowLoc row_of(const BwdParams& p, int64_t R) {
    RowLoc L;
    if (p.varlen) {
        L.b = 0; L.h = R % p.Hq; L.i = R / p.Hq;
    } else {
        L.i = R % p.Sq;
        const int64_t bh = R / p.Sq;
        L.h = bh % p.Hq; L.b = bh / p.Hq;
    }
    return L;
}

__device__ __forceinline__ int64_t toff(const TensorArg& t, const RowLoc& L) {
    return L.b * t.sb + L.h * t.sh + L.i * t.ss;
}

// ---------------------------------------------------------------------------
// Preprocess
// ---------------------------------------------------------------------------

template <class T, int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(BwdParams p, int zero_dq) {
    constexpr int LPR = D / 8;   // lanes per row, 8 elements (16 bytes) each
    const int64_t gt = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t R = gt / LPR;
    const int part = (int)(gt % LPR);
    const bool ok = R < p.rows;
    float acc = 0.f;
    RowLoc L{0, 0, 0};
    if (ok) {
        L = row_of(p, R);
        const u32x4 ov = ld16(p.o.p + toff(p.o, L) + part * 8);
        const u32x4 dv = ld16(p.dout.p + toff(p.dout, L) + part * 8);
#pragma unroll
        for (int t = 0; t < 8; ++t) acc += T::to_f32(elem16(ov, t)) * T::to_f32(elem16(dv, t));
    }
#pragma unroll
    for (int off = LPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
    if (!ok) return;
    if (part == 0) {
        p.delta[R] = acc;
        const int64_t so = L.b * p.st_sb + L.h * p.st_sh + L.i * p.st_ss;
        float l2;
        if (p.stats_kind == 0) {
            const float x = p.st_a[so];
            l2 = (x == -INFINITY) ? INFINITY : x * kLog2e;
        } else {
            const float mx = p.st_a[so], sm = p.st_b[so];
            l2 = (sm > 0.f) ? mx * kLog2e + log2f(sm) : INFINITY;
        }
        p.lse2[R] = l2;
    }
    if (zero_dq) {
        f32x4 z = {0.f, 0.f, 0.f, 0.f};
        f32x4* dst = reinterpret_cast<f32x4*>(p.dqacc + R * D + part * 8);
        dst[0] = z;
        dst[1] = z;
    }
}

// ---------------------------------------------------------------------------
// Main backward kernel (KV-tile outer)
// ---------------------------------------------------------------------------

template <class T, int D, bool CAUSAL, bool DQ_ATOMIC>
__global__ __launch_bounds__(256) void bwd_main_kernel(BwdParams p) {
    constexpr int BC = 128;          // keys per workgroup: 4 wavefronts x 32
    constexpr int BR = 64;           // query rows per inner step
    constexpr int NW = 4;
    constexpr int KS = D / 16;       // k-steps over the head dimension
    constexpr int MB = BR / 32;      // 32-row blocks of the query tile
    constexpr int DB = D / 32;       // 32-row blocks of dK^T / dV^T
    constexpr int QP = D + 8;        // row stride of Qs, dOs     [i][d]
    constexpr int TP = BR + 8;       // row stride of QT, dOT     [d][i]
    constexpr int SP = BC + 8;       // row stride of dSs [i][j], KT [d][j]
    __shared__ __align__(16) uint16_t Qs[BR * QP];
    __shared__ __align__(16) uint16_t dOs[BR * QP];
    __shared__ __align__(16) uint16_t QT[D * TP];
    __shared__ __align__(16) uint16_t dOT[D * TP];
    __shared__ __align__(16) uint16_t dSs[DQ_ATOMIC ? BR * SP : 8];
    __shared__ __align__(16) uint16_t KT[DQ_ATOMIC ? D * SP : 8];
    __shared__ __align__(16) float lse_s[BR];
    __shared__ __align__(16) float dlt_s[BR];

    const int tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6;
    const int g = lane >> 5, c = lane & 31;
    const int b = blockIdx.x / p.Hkv, hk = blockIdx.x % p.Hkv;
    const int G = p.Hq / p.Hkv;
    int q0 = 0, k0 = 0, lq = p.Sq, lk = p.Sk;
    if (p.varlen) seq_get(p.seqs, b, q0, k0, lq, lk);
    const int j0 = blockIdx.y * BC;
    if (j0 >= lk) return;

    const uint16_t* kbase = p.k.p + b * p.k.sb + hk * p.k.sh + (int64_t)k0 * p.k.ss;
    const uint16_t* vbase = p.v.p + b * p.v.sb + hk * p.v.sh + (int64_t)k0 * p.v.ss;

    const int my_j = j0 + 32 * w + c;
    const bool col_ok = my_j < lk;
    u32x4 kreg[KS], vreg[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) {
        u32x4 z = {0u, 0u, 0u, 0u};
        kreg[s] = col_ok ? ld16(kbase + (int64_t)my_j * p.k.ss + 16 * s + 8 * g) : z;
        vreg[s] = col_ok ? ld16(vbase + (int64_t)my_j * p.v.ss + 16 * s + 8 * g) : z;
    }
    if (DQ_ATOMIC) {
#pragma unroll
        for (int s = 0; s < KS; ++s)
#pragma unroll
            for (int t = 0; t < 8; ++t) KT[(16 * s + 8 * g + t) * SP + 32 * w + c] = elem16(kreg[s], t);
    }

    f32x16 dva[DB], dka[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) { dva[db] = zero16(); dka[db] = zero16(); }

    const int i_begin = CAUSAL ? (j0 / BR) * BR : 0;
    for (int gh = 0; gh < G; ++gh) {
        const int h = hk * G + gh;
        const uint16_t* qbase = p.q.p + b * p.q.sb + h * p.q.sh + (int64_t)q0 * p.q.ss;
        const uint16_t* dobase = p.dout.p + b * p.dout.sb + h * p.dout.sh + (int64_t)q0 * p.dout.ss;
        const int64_t ws_base = p.varlen ? (int64_t)q0 * p.Hq + h : ((int64_t)b * p.Hq + h) * p.Sq;
        const int64_t ws_step = p.varlen ? p.Hq : 1;

        for (int i0 = i_begin; i0 < lq; i0 += BR) {
            __syncthreads();
            for (int e = tid; e < BR * D / 8; e += 256) {
                const int r = e / (D / 8), cc = (e % (D / 8)) * 8;
                const int i = i0 + r;
                u32x4 qv = {0u, 0u, 0u, 0u}, dv = {0u, 0u, 0u, 0u};
                if (i < lq) {
                    qv = ld16(qbase + (int64_t)i * p.q.ss + cc);
                    dv = ld16(dobase + (int64_t)i * p.dout.ss + cc);
                }
                st16(&Qs[r * QP + cc], qv);
                st16(&dOs[r * QP + cc], dv);
#pragma unroll
                for (int t = 0; t < 8; ++t) {
                    QT[(cc + t) * TP + r] = elem16(qv, t);
                    dOT[(cc + t) * TP + r] = elem16(dv, t);
                }
            }
            if (tid < BR) {
                const int i = i0 + tid;
                lse_s[tid] = i < lq ? p.lse2[ws_base + i * ws_step] : INFINITY;
                dlt_s[tid] = i < lq ? p.delta[ws_base + i * ws_step] : 0.f;
            }
            __syncthreads();

            f32x16 sa[MB], pa[MB];
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) {
                sa[mb] = zero16();
                pa[mb] = zero16();
#pragma unroll
                for (int s = 0; s < KS; ++s) {
                    sa[mb] = T::mma(ld16(&Qs[(mb * 32 + c) * QP + 16 * s + 8 * g]), kreg[s], sa[mb]);
                    pa[mb] = T::mma(ld16(&dOs[(mb * 32 + c) * QP + 16 * s + 8 * g]), vreg[s], pa[mb]);
                }
            }
            const bool diag = CAUSAL && (i0 < j0 + BC);
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const f32x4 Lr = *reinterpret_cast<const f32x4*>(&lse_s[mb * 32 + 8 * q + 4 * g]);
                    const f32x4 Dr = *reinterpret_cast<const f32x4*>(&dlt_s[mb * 32 + 8 * q + 4 * g]);
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int rg = 4 * q + r;
                        const int i = i0 + mb * 32 + 8 * q + 4 * g + r;
                        float pv = fast_exp2(sa[mb][rg] * p.scale_log2 - Lr[r]);
                        if (!col_ok || (diag && my_j > i)) pv = 0.f;
                        sa[mb][rg] = pv;
                        pa[mb][rg] = pv * (pa[mb][rg] - Dr[r]);
                    }
                }
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    const u32x4 bP = acc_to_operand<T>(sa[mb], hh);
                    const u32x4 bS = acc_to_operand<T>(pa[mb], hh);
#pragma unroll
                    for (int db = 0; db < DB; ++db) {
                        const int d = db * 32 + c;
                        dva[db] = T::mma(ld_acc_slots(&dOT[d * TP + mb * 32 + 16 * hh], g), bP, dva[db]);
                        dka[db] = T::mma(ld_acc_slots(&QT[d * TP + mb * 32 + 16 * hh], g), bS, dka[db]);
                    }
                }
            if (DQ_ATOMIC) {
#pragma unroll
                for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                    for (int rg = 0; rg < 16; ++rg)
                        dSs[(mb * 32 + 8 * (rg >> 2) + 4 * g + (rg & 3)) * SP + 32 * w + c] = T::cvt(pa[mb][rg]);
                __syncthreads();
                for (int blk = w; blk < MB * DB; blk += NW) {
                    const int ib = blk / DB, db = blk % DB;
                    f32x16 acc = zero16();
#pragma unroll
                    for (int ks = 0; ks < BC / 16; ++ks)
                        acc = T::mma(ld16(&dSs[(ib * 32 + c) * SP + 16 * ks + 8 * g]),
                                     ld16(&KT[(db * 32 + c) * SP + 16 * ks + 8 * g]), acc);
#pragma unroll
                    for (int rg = 0; rg < 16; ++rg) {
                        const int i = i0 + ib * 32 + 8 * (rg >> 2) + 4 * g + (rg & 3);
                        if (i < lq)
                            atomicAdd(&p.dqacc[(ws_base + i * ws_step) * D + db * 32 + c], acc[rg]);
                    }
                }
            }
        }
    }

    if (!col_ok) return;
    uint16_t* dkp = p.dk.p + b * p.dk.sb + hk * p.dk.sh + (int64_t)(k0 + my_j) * p.dk.ss;
    uint16_t* dvp = p.dv.p + b * p.dv.sb + hk * p.dv.sh + (int64_t)(k0 + my_j) * p.dv.ss;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            u32x2 a, v;
            a[0] = T::pack(dka[db][4 * q + 0] * p.scale, dka[db][4 * q + 1] * p.scale);
            a[1] = T::pack(dka[db][4 * q + 2] * p.scale, dka[db][4 * q + 3] * p.scale);
            v[0] = T::pack(dva[db][4 * q + 0], dva[db][4 * q + 1]);
            v[1] = T::pack(dva[db][4 * q + 2], dva[db][4 * q + 3]);
            st8(dkp + db * 32 + 8 * q + 4 * g, a);
            st8(dvp + db * 32 + 8 * q + 4 * g, v);
        }
}

// ---------------------------------------------------------------------------
// dQ finalisation (atomic mode)
// ---------------------------------------------------------------------------

template <class T, int D>
__global__ __launch_bounds__(256) void bwd_dq_convert_kernel(BwdParams p) {
    constexpr int LPR = D / 8;
    const int64_t gt = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t R = gt / LPR;
    const int part = (int)(gt % LPR);
    if (R >= p.rows) return;
    const RowLoc L = row_of(p, R);
    const f32x4* src = reinterpret_cast<const f32x4*>(p.dqacc + R * D + part * 8);
    const f32x4 a = src[0], c = src[1];
    u32x4 o;
    o[0] = T::pack(a[0] * p.scale, a[1] * p.scale);
    o[1] = T::pack(a[2] * p.scale, a[3] * p.scale);
    o[2] = T::pack(c[0] * p.scale, c[1] * p.scale);
    o[3] = T::pack(c[2] * p.scale, c[3] * p.scale);
    st16(p.dq.p + toff(p.dq, L) + part * 8, o);
}

// ---------------------------------------------------------------------------
// Deterministic dQ (query-tile outer)
// ---------------------------------------------------------------------------

template <class T, int D, bool CAUSAL>
__global__ __launch_bounds__(256) void bwd_dq_kernel(BwdParams p) {
    constexpr int BQ = 128;          // 4 wavefronts x 32 query rows
    constexpr int BK = 64;           // keys per LDS tile
    constexpr int KS = D / 16;
    constexpr int DB = D / 32;
    constexpr int KP = D + 8;        // Ks, Vs  [key][d]
    constexpr int TP = BK + 8;       // KT      [d][key]
    __shared__ __align__(16) uint16_t Ks[BK * KP];
    __shared__ __align__(16) uint16_t Vs[BK * KP];
    __shared__ __align__(16) uint16_t KT[D * TP];

    const int tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6;
    const int g = lane >> 5, c = lane & 31;
    const int b = blockIdx.y / p.Hq, h = blockIdx.y % p.Hq;
    const int hk = h / (p.Hq / p.Hkv);
    int q0 = 0, k0 = 0, lq = p.Sq, lk = p.Sk;
    if (p.varlen) seq_get(p.seqs, b, q0, k0, lq, lk);
    const int i0 = blockIdx.x * BQ;
    if (i0 >= lq) return;

    const uint16_t* qbase = p.q.p + b * p.q.sb + h * p.q.sh + (int64_t)q0 * p.q.ss;
    const uint16_t* dobase = p.dout.p + b * p.dout.sb + h * p.dout.sh + (int64_t)q0 * p.dout.ss;
    const uint16_t* kbase = p.k.p + b * p.k.sb + hk * p.k.sh + (int64_t)k0 * p.k.ss;
    const uint16_t* vbase = p.v.p + b * p.v.sb + hk * p.v.sh + (int64_t)k0 * p.v.ss;
    const int64_t ws_base = p.varlen ? (int64_t)q0 * p.Hq + h : ((int64_t)b * p.Hq + h) * p.Sq;
    const int64_t ws_step = p.varlen ? p.Hq : 1;

    const int my_i = i0 + 32 * w + c;
    const bool row_ok = my_i < lq;
    u32x4 qreg[KS], doreg[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) {
        u32x4 z = {0u, 0u, 0u, 0u};
        qreg[s] = row_ok ? ld16(qbase + (int64_t)my_i * p.q.ss + 16 * s + 8 * g) : z;
        doreg[s] = row_ok ? ld16(dobase + (int64_t)my_i * p.dout.ss + 16 * s + 8 * g) : z;
    }
    const float l2 = row_ok ? p.lse2[ws_base + my_i * ws_step] : INFINITY;
    const float dl = row_ok ? p.delta[ws_base + my_i * ws_step] : 0.f;

    f32x16 dq[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) dq[db] = zero16();

    const int kend = CAUSAL ? min(lk, i0 + BQ) : lk;
    for (int j0 = 0; j0 < kend; j0 += BK) {
        __syncthreads();
        for (int e = tid; e < BK * D / 8; e += 256) {
            const int r = e / (D / 8), cc = (e % (D / 8)) * 8;
            const int j = j0 + r;
            u32x4 kv = {0u, 0u, 0u, 0u}, vv = {0u, 0u, 0u, 0u};
            if (j < lk) {
                kv = ld16(kbase + (int64_t)j * p.k.ss + cc);
                vv = ld16(vbase + (int64_t)j * p.v.ss + cc);
            }
            st16(&Ks[r * KP + cc], kv);
            st16(&Vs[r * KP + cc], vv);
#pragma unroll
            for (int t = 0; t < 8; ++t) KT[(cc + t) * TP + r] = elem16(kv, t);
        }
        __syncthreads();
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            f32x16 s = zero16(), dp = zero16();
#pragma unroll
            for (int st = 0; st < KS; ++st) {
                s = T::mma(ld16(&Ks[(kb * 32 + c) * KP + 16 * st + 8 * g]), qreg[st], s);
                dp = T::mma(ld16(&Vs[(kb * 32 + c) * KP + 16 * st + 8 * g]), doreg[st], dp);
            }
#pragma unroll
            for (int rg = 0; rg < 16; ++rg) {
                const int j = j0 + kb * 32 + 8 * (rg >> 2) + 4 * g + (rg & 3);
                float pv = fast_exp2(s[rg] * p.scale_log2 - l2);
                if (j >= lk || (CAUSAL && j > my_i)) pv = 0.f;
                dp[rg] = pv * (dp[rg] - dl);
            }
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                const u32x4 bS = acc_to_operand<T>(dp, hh);
#pragma unroll
                for (int db = 0; db < DB; ++db)
                    dq[db] = T::mma(ld_acc_slots(&KT[(db * 32 + c) * TP + kb * 32 + 16 * hh], g), bS, dq[db]);
            }
        }
    }
    if (!row_ok) return;
    uint16_t* dqp = p.dq.p + b * p.dq.sb + h * p.dq.sh + (int64_t)(q0 + my_i) * p.dq.ss;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            u32x2 v;
            v[0] = T::pack(dq[db][4 * q + 0] * p.scale, dq[db][4 * q + 1] * p.scale);
            v[1] = T::pack(dq[db][4 * q + 2] * p.scale, dq[db][4 * q + 3] * p.scale);
            st8(dqp + db * 32 + 8 * q + 4 * g, v);
        }
}

// ---------------------------------------------------------------------------
// Launch
// ---------------------------------------------------------------------------

template <class T, int D, bool CAUSAL>
static hipError_t launch_bwd_t(const BwdParams& p, const BwdLaunch& L, hipStream_t st) {
    const int64_t row_threads = p.rows * (D / 8);
    const dim3 row_grid((unsigned)((row_threads + 255) / 256));
    const bool have_rows = p.rows > 0;
    if ((L.phase & BwdLaunch::kFirst) && have_rows)
        PROF_LAUNCH(KID_BWD_PRE, st, (bwd_pre_kernel<T, D>), row_grid, dim3(256), 0, st, p, L.deterministic ? 0 : 1);
    const dim3 main_grid(L.n_seq * p.Hkv, L.max_kv_tiles);
    const bool have_main = main_grid.x > 0 && main_grid.y > 0;
    if (L.deterministic) {
        if (have_main)
            PROF_LAUNCH(KID_BWD_MAIN, st, (bwd_main_kernel<T, D, CAUSAL, false>), main_grid, dim3(256), 0, st, p);
        const dim3 dq_grid(L.max_q_tiles128, L.n_seq * p.Hq);
        if (dq_grid.x > 0 && dq_grid.y > 0)
            PROF_LAUNCH(KID_BWD_DQ_DET, st, (bwd_dq_kernel<T, D, CAUSAL>), dq_grid, dim3(256), 0, st, p);
    } else {
        if (have_main)
            PROF_LAUNCH(KID_BWD_MAIN, st, (bwd_main_kernel<T, D, CAUSAL, true>), main_grid, dim3(256), 0, st, p);
        if ((L.phase & BwdLaunch::kLast) && have_rows)
            PROF_LAUNCH(KID_BWD_DQ_CONVERT, st, (bwd_dq_convert_kernel<T, D>), row_grid, dim3(256), 0, st, p);
    }
    return hipGetLastError();
}

template <class T, int D>
static hipError_t launch_bwd_d(const BwdParams& p, const BwdLaunch& L, hipStream_t st) {
    return L.causal ? launch_bwd_t<T, D, true>(p, L, st) : launch_bwd_t<T, D, false>(p, L, st);
}

hipError_t launch_bwd(const BwdParams& p, const BwdLaunch& L, hipStream_t st) {
    if (L.dtype == 0)
        return L.D == 64 ? launch_bwd_d<F16, 64>(p, L, st) : launch_bwd_d<F16, 128>(p, L, st);
    return L.D == 64 ? launch_bwd_d<BF16, 64>(p, L, st) : launch_bwd_d<BF16, 128>(p, L, st);
}

}  // namespace sdpa
