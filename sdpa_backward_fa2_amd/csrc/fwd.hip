// Attention forward in training mode: O and the natural-log LSE per row.
//
// This produces the statistics the backward consumes (the cuDNN SDPA sample's
// forward graph with is_inference=False emits o and stats; forward-graph cell).
// It is a FlashAttention-style forward: each wavefront owns 32 query rows,
// keys stream through double-buffered LDS tiles 64 at a time, and a running
// max and sum give the softmax without materialising it.  Packed batches read each sequence's
// token range from the sequence table.  Scores are computed transposed
// (S^T = K Q^T) so that every lane holds one query column: row statistics are
// lane-local and need a single exchange with the other lane half.
#include "common.h"
#include "kernels.h"
#include "prof.h"

namespace sdpa {

// One workgroup of NW wavefronts per 32*NW query rows of one (batch, head);
// wavefront w owns rows 32w .. 32w+31 of the tile and holds their Q in
// registers (the B operand of S^T = K Q^T).  Key tiles of 64 rows of K and V
// are double-buffered in LDS, the next tile loaded into registers while the
// current one is used.  O^T += V^T P^T takes V^T from ds_read_b64_tr_b16 on
// the row-major V tile in the order of P^T's accumulator registers, so P^T
// feeds the product without leaving registers.  Masks are evaluated only on
// tiles that need them; keys past the end re-read the last key and are
// masked, rows past the end re-read the last row and are not stored.
template <int D, int DV>
struct FwdLds {
    // SWV: at D = DV = 128 the V tiles are unpadded with their chunks
    // swizzled (swz128), so that the transposing reads meet distinct banks:
    // S=4096 causal 235 -> 229 us.  (At (192, 128) it was slower, 341 -> 353
    // us, and a 64-column swizzle at D = 64 changed nothing.)
    static constexpr bool SWV = D == 128 && DV == 128;
    static constexpr int BK = 64, KP = D + 8, VP = SWV ? DV : DV + 8;
};

// D: head dim of Q and K; DV: of V and O.
template <class T, int D, int DV, bool CAUSAL, int NW>
__global__ __launch_bounds__(64 * NW, 8 / NW) void fwd_kernel(FwdParams p) {
    constexpr int NT = 64 * NW;      // threads
    constexpr int BQ = 32 * NW;      // query rows per workgroup
    constexpr int BK = FwdLds<D, DV>::BK;
    constexpr int KS = D / 16;       // k-steps of S over the Q/K head dimension
    constexpr int DB = DV / 32;      // 32-row blocks of O^T
    constexpr int KP = FwdLds<D, DV>::KP, VP = FwdLds<D, DV>::VP;   // row strides [key][d]
    constexpr bool SWV = FwdLds<D, DV>::SWV;
    constexpr int CHK = BK * D / 8 / NT, CHV = BK * DV / 8 / NT;    // 16-byte chunks per thread per tile
    static_assert(CHK * NT * 8 == BK * D && CHV * NT * 8 == BK * DV, "whole chunks per thread");
    __shared__ __align__(16) uint16_t Ks[2][BK * KP];
    __shared__ __align__(16) uint16_t Vs[2][BK * VP];

    const int tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6;
    const int g = lane >> 5, c = lane & 31;
    // a head's query tiles stay on one XCD (its K and V in that L2), the
    // longest causal ranges first
    int bh, item;
    xcd_unit_order(gridDim.y, gridDim.x, blockIdx.y * gridDim.x + blockIdx.x, bh, item);
    const int bx = CAUSAL ? gridDim.x - 1 - item : item;
    const int b = bh / p.Hq, h = bh % p.Hq;
    const int hk = h / (p.Hq / p.Hkv);
    int q0 = 0, k0 = 0, lq = p.Sq, lk = p.Sk;
    if (p.varlen) seq_get(p.seqs, b, q0, k0, lq, lk);
    const int i0 = bx * BQ;
    if (i0 >= lq) return;

    const uint16_t* qp = p.q.p + b * p.q.sb + h * p.q.sh + (int64_t)q0 * p.q.ss;
    const uint16_t* kp = p.k.p + b * p.k.sb + hk * p.k.sh + (int64_t)k0 * p.k.ss;
    const uint16_t* vp = p.v.p + b * p.v.sb + hk * p.v.sh + (int64_t)k0 * p.v.ss;

    const int kend = CAUSAL ? min(lk, i0 + BQ) : lk;
    const int n_steps = (kend + BK - 1) / BK;

    int krow[CHK], kcol[CHK], vrow[CHV], vcol[CHV];
#pragma unroll
    for (int x = 0; x < CHK; ++x) {
        const int e = tid + NT * x;
        krow[x] = e / (D / 8);
        kcol[x] = (e % (D / 8)) * 8;
    }
#pragma unroll
    for (int x = 0; x < CHV; ++x) {
        const int e = tid + NT * x;
        vrow[x] = e / (DV / 8);
        vcol[x] = (e % (DV / 8)) * 8;
    }
    auto vcol_lds = [&](int x) { return SWV ? swz128_col(vrow[x], vcol[x]) : vcol[x]; };
    u32x4 pk[CHK], pv[CHV];
    auto load_tile = [&](int st) {
        const int j0 = st * BK, last = lk - 1 - j0;
        const uint16_t* kt = kp + (int64_t)j0 * p.k.ss;
        const uint16_t* vt = vp + (int64_t)j0 * p.v.ss;
#pragma unroll
        for (int x = 0; x < CHK; ++x) pk[x] = ld16(kt + (int64_t)min(krow[x], last) * p.k.ss + kcol[x]);
#pragma unroll
        for (int x = 0; x < CHV; ++x) pv[x] = ld16(vt + (int64_t)min(vrow[x], last) * p.v.ss + vcol[x]);
    };
    auto store_tile = [&](int buf) {
#pragma unroll
        for (int x = 0; x < CHK; ++x) st16(&Ks[buf][krow[x] * KP + kcol[x]], pk[x]);
#pragma unroll
        for (int x = 0; x < CHV; ++x) st16(&Vs[buf][vrow[x] * VP + vcol_lds(x)], pv[x]);
    };

    if (n_steps > 0) load_tile(0);
    const int my_i = i0 + 32 * w + c;
    const bool row_ok = my_i < lq;
    const int my_ic = min(my_i, lq - 1);
    u32x4 qreg[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) qreg[s] = ld16(qp + (int64_t)my_ic * p.q.ss + 16 * s + 8 * g);
    if (n_steps > 0) store_tile(0);
    __syncthreads();

    float m = -INFINITY, l = 0.f;
    f32x16 o[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) o[db] = zero16();
    // last key this lane's row keeps, relative to the 4g part of a tile row
    const int t_row = min(lk - 1, CAUSAL ? my_i : INT_MAX) - 4 * g;
    const int w_row0 = i0 + 32 * w;   // the wavefront's first row

    for (int st = 0; st < n_steps; ++st) {
        const int buf = st & 1;
        const int j0 = st * BK;
        const bool has_next = st + 1 < n_steps;
        if (has_next) load_tile(st + 1);
        const uint16_t* Kb = Ks[buf];
        const uint16_t* Vb = Vs[buf];

        // S^T of the tile's two 32-key blocks: element (kb, rg) is key
        // j0 + 32kb + 8(rg/4) + 4g + rg%4 of this lane's query row
        f32x16 s[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            s[kb] = zero16();
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                s[kb] = T::mma(ld16(&Kb[(32 * kb + c) * KP + 16 * ks + 8 * g]), qreg[ks], s[kb]);
        }
        const bool masked = (CAUSAL && j0 + BK - 1 > w_row0) || (j0 + BK > lk);
        float tmax = -INFINITY;
        if (masked) {
            const int t = t_row - j0;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int rg = 0; rg < 16; ++rg) {
                    const float x = (32 * kb + 8 * (rg >> 2) + (rg & 3) <= t) ? s[kb][rg] * p.scale_log2 : -INFINITY;
                    s[kb][rg] = x;
                    tmax = fmaxf(tmax, x);
                }
        } else {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int rg = 0; rg < 16; ++rg) {
                    const float x = s[kb][rg] * p.scale_log2;
                    s[kb][rg] = x;
                    tmax = fmaxf(tmax, x);
                }
        }
        tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
        const float m_new = fmaxf(m, tmax);
        const float msub = (m_new == -INFINITY) ? 0.f : m_new;
        const float alpha = fast_exp2(m - msub);   // 0 while the row had no key
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
        // rescale O only when some row's maximum moved
        if (__any(alpha != 1.f)) {
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int rg = 0; rg < 16; ++rg) o[db][rg] *= alpha;
        }
        // O^T += V^T P^T over the tile's keys, 16 at a time
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                const u32x4 bop = acc_to_operand<T>(s[kb], hh);
#pragma unroll
                for (int db = 0; db < DB; ++db) {
                    u32x4 a;
                    if constexpr (SWV) a = ld_tr_swz128<true>(Vb, 32 * kb + 16 * hh, db * 32, lane);
                    else a = ld_tr<true>(Vb, VP, 32 * kb + 16 * hh, db * 32, lane);
                    o[db] = T::mma(a, bop, o[db]);
                }
            }
        if (has_next) store_tile(buf ^ 1);
        __syncthreads();
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

// grid: (query tiles of the longest sequence, batch x heads).  Four
// wavefronts (128-row tiles) at every head dim: at D = 64 two-wavefront
// workgroups, twice as many, were no faster on the GPT-2 shape (31.0 against
// 30.3 us).
template <class T, int D, int DV>
static hipError_t launch_fwd_t(const FwdParams& p, int max_lq, bool causal, hipStream_t st) {
    constexpr int NW = 4;
    dim3 grid((max_lq + 32 * NW - 1) / (32 * NW), p.B * p.Hq);
    if (causal)
        PROF_LAUNCH(KID_FWD, st, (fwd_kernel<T, D, DV, true, NW>), grid, dim3(64 * NW), 0, st, p);
    else
        PROF_LAUNCH(KID_FWD, st, (fwd_kernel<T, D, DV, false, NW>), grid, dim3(64 * NW), 0, st, p);
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
