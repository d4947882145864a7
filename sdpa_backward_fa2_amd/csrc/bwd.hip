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

// log2-domain LSE of one row straight from the caller's statistics: LSE*log2e,
// or m*log2e + log2(l) for the max/sum form; +inf for a row without keys.
__device__ __forceinline__ float stats_lse2(const BwdParams& p, int64_t so) {
    if (p.stats_kind == 0) {
        const float x = p.st_a[so];
        return (x == -INFINITY) ? INFINITY : x * kLog2e;
    }
    const float mx = p.st_a[so], sm = p.st_b[so];
    return (sm > 0.f) ? mx * kLog2e + log2f(sm) : INFINITY;
}

template <class T>
__device__ __forceinline__ float dot8(u32x4 a, u32x4 b) {
    float acc = 0.f;
#pragma unroll
    for (int t = 0; t < 8; ++t) acc += T::to_f32(elem16(a, t)) * T::to_f32(elem16(b, t));
    return acc;
}

// dQ accumulator row of statistics row R (head-major; see BwdParams)
__device__ __forceinline__ int64_t acc_row(const BwdParams& p, const RowLoc& L, int64_t R) {
    return p.varlen ? L.h * p.Sq + L.i : R;
}

__device__ __forceinline__ int64_t toff(const TensorArg& t, const RowLoc& L) {
    return L.b * t.sb + L.h * t.sh + L.i * t.ss;
}

// ---------------------------------------------------------------------------
// Preprocess
// ---------------------------------------------------------------------------

template <class T, int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(BwdParams p, int zero_dq) {
    constexpr int LPR = D / 16;  // lanes per row, 16 elements (two 16-byte chunks) each
    const int64_t gt = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t R = gt / LPR;
    const int part = (int)(gt % LPR);
    const bool ok = R < p.rows;
    float acc = 0.f;
    RowLoc L{0, 0, 0};
    if (ok) {
        L = row_of(p, R);
        const uint16_t* op = p.o.p + toff(p.o, L) + part * 16;
        const uint16_t* dp = p.dout.p + toff(p.dout, L) + part * 16;
        const u32x4 o0 = ld16(op), o1 = ld16(op + 8);
        const u32x4 d0 = ld16(dp), d1 = ld16(dp + 8);
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            acc += T::to_f32(elem16(o0, t)) * T::to_f32(elem16(d0, t));
            acc += T::to_f32(elem16(o1, t)) * T::to_f32(elem16(d1, t));
        }
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
        f32x4* dst = reinterpret_cast<f32x4*>(p.dqacc + acc_row(p, L, R) * D + part * 16);
        dst[0] = z;
        dst[1] = z;
        dst[2] = z;
        dst[3] = z;
    }
}

// ---------------------------------------------------------------------------
// Main backward kernel (KV-tile outer)
// ---------------------------------------------------------------------------
//
// Per step (one 64-row query tile of one query head) each wavefront, owning 32
// of the workgroup's 128 keys, computes S and dP (32 x 32 per half tile), P and
// dS, then dV^T += dO^T P and dK^T += Q^T dS.  Q and dO tiles sit row-major in
// LDS; the transposed operands of the dV/dK products come from
// ds_read_b64_tr_b16.  The next tile's Q/dO rows are loaded into registers
// while the current one is consumed and written to the other half of a double
// buffer.  In atomic mode dS^T goes to LDS and the four wavefronts split
// dQ_tile = dS K (64 x D) between them, adding it to the fp32 accumulator with
// global atomics.  Masks are evaluated only on tiles that need them (the
// causal diagonal, a ragged last key tile); ragged query rows carry LSE = +inf
// and so contribute P = 0 without a mask.

// P = exp2(S*scale*log2e - LSE*log2e) and dS = P * (dP - Delta) for one 32x32
// C tile held as (sa, pa); rows i = i_base + 8q + 4g + r, this lane's key my_j.
template <bool MASKED, bool CAUSAL>
__device__ __forceinline__ void softmax_grad_tile(f32x16& sa, f32x16& pa, const float* lse_row,
                                                  const float* dlt_row, float scale_log2, int g,
                                                  int i_base, int my_j, bool col_ok) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const f32x4 Lr = *reinterpret_cast<const f32x4*>(&lse_row[8 * q + 4 * g]);
        const f32x4 Dr = *reinterpret_cast<const f32x4*>(&dlt_row[8 * q + 4 * g]);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int rg = 4 * q + r;
            float pv = fast_exp2(__builtin_fmaf(sa[rg], scale_log2, -Lr[r]));
            if (MASKED) {
                // branch-free: keep = key valid and (not causal or key <= row)
                const int i = i_base + 8 * q + 4 * g + r;
                const bool keep = col_ok & (!CAUSAL | (my_j <= i));
                pv = keep ? pv : 0.f;
            }
            sa[rg] = pv;
            pa[rg] = pv * (pa[rg] - Dr[r]);
        }
    }
}

template <class T, int D, bool CAUSAL, bool DQ_ATOMIC>
__global__ __launch_bounds__(256, (D == 64 ? 2 : 1)) void bwd_main_kernel(BwdParams p) {
    constexpr int BC = 128;          // keys per workgroup: 4 wavefronts x 32
    constexpr int BR = 64;           // query rows per step
    constexpr int NW = 4;
    constexpr int KS = D / 16;       // k-steps over the head dimension
    constexpr int MB = BR / 32;      // 32-row blocks of the query tile
    constexpr int DB = D / 32;       // 32-row blocks of dK^T / dV^T
    constexpr int QP = D + 8;        // row stride of Qs, dOs, Ks  [row][d]
    constexpr int SP = BR + 8;       // row stride of dST          [j][i]
    constexpr int CH = BR * D / 8 / 256;     // 16-byte chunks per thread per tile
    constexpr int NBLK = MB * DB / NW;       // dQ 32x32 blocks per wavefront
    static_assert(CH >= 1 && NBLK >= 1, "tile shape");
    __shared__ __align__(16) uint16_t Qs[2][BR * QP];
    __shared__ __align__(16) uint16_t dOs[2][BR * QP];
    __shared__ __align__(16) uint16_t Ks[DQ_ATOMIC ? BC * QP : 8];
    __shared__ __align__(16) uint16_t dST[DQ_ATOMIC ? BC * SP : 8];
    __shared__ __align__(16) float lse_s[2][BR];
    __shared__ __align__(16) float dlt_s[2][BR];

    const int tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6;
    const int g = lane >> 5, c = lane & 31;
    const int b = blockIdx.x / p.Hkv, hk = blockIdx.x % p.Hkv;
    const int G = p.Hq / p.Hkv;
    int q0 = 0, k0 = 0, lq = p.Sq, lk = p.Sk;
    if (p.varlen) seq_get(p.seqs, b, q0, k0, lq, lk);
    const int j0 = blockIdx.y * BC;
    if (j0 >= lk) return;
    const bool full_cols = j0 + BC <= lk;

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
        if (DQ_ATOMIC) st16(&Ks[(32 * w + c) * QP + 16 * s + 8 * g], kreg[s]);
    }

    f32x16 dva[DB], dka[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) { dva[db] = zero16(); dka[db] = zero16(); }

    // steps: query heads of the group outer, query tiles from the causal start inner
    const int i_begin = CAUSAL ? (j0 / BR) * BR : 0;
    const int per_head = lq > i_begin ? (lq - i_begin + BR - 1) / BR : 0;
    const int n_steps = G * per_head;

    // per-thread element offsets of its 16-byte chunks inside a tile (row r, column cc)
    int qoff[CH], dooff[CH], crow[CH];
#pragma unroll
    for (int x = 0; x < CH; ++x) {
        const int e = tid + 256 * x;
        const int r = e / (D / 8), cc = (e % (D / 8)) * 8;
        crow[x] = r;
        qoff[x] = r * (int)p.q.ss + cc;
        dooff[x] = r * (int)p.dout.ss + cc;
    }
    const int64_t ws_step = p.varlen ? p.Hq : 1;

    u32x4 pq[CH], pdo[CH];
    float pl = INFINITY, pd = 0.f;
    auto load_tile = [&](int st) {
        const int h = hk * G + st / per_head;
        const int i0 = i_begin + (st % per_head) * BR;
        const uint16_t* qb = p.q.p + b * p.q.sb + h * p.q.sh + (int64_t)(q0 + i0) * p.q.ss;
        const uint16_t* dob = p.dout.p + b * p.dout.sb + h * p.dout.sh + (int64_t)(q0 + i0) * p.dout.ss;
        if (i0 + BR <= lq) {
#pragma unroll
            for (int x = 0; x < CH; ++x) {
                pq[x] = ld16(qb + qoff[x]);
                pdo[x] = ld16(dob + dooff[x]);
            }
        } else {
#pragma unroll
            for (int x = 0; x < CH; ++x) {
                u32x4 z = {0u, 0u, 0u, 0u};
                const bool ok = i0 + crow[x] < lq;
                pq[x] = ok ? ld16(qb + qoff[x]) : z;
                pdo[x] = ok ? ld16(dob + dooff[x]) : z;
            }
        }
        if (tid < BR) {
            const int i = i0 + tid;
            const int64_t ws = p.varlen ? ((int64_t)(q0 + i) * p.Hq + h) : (((int64_t)b * p.Hq + h) * p.Sq + i);
            pl = i < lq ? p.lse2[ws] : INFINITY;
            pd = i < lq ? p.delta[ws] : 0.f;
        }
    };
    auto store_tile = [&](int buf) {
#pragma unroll
        for (int x = 0; x < CH; ++x) {
            const int e = tid + 256 * x;
            const int r = e / (D / 8), cc = (e % (D / 8)) * 8;
            st16(&Qs[buf][r * QP + cc], pq[x]);
            st16(&dOs[buf][r * QP + cc], pdo[x]);
        }
        if (tid < BR) {
            lse_s[buf][tid] = pl;
            dlt_s[buf][tid] = pd;
        }
    };

    if (n_steps > 0) {
        load_tile(0);
        store_tile(0);
    }
    __syncthreads();

    for (int st = 0; st < n_steps; ++st) {
        const int buf = st & 1;
        const int h = hk * G + st / per_head;
        const int i0 = i_begin + (st % per_head) * BR;
        const bool has_next = st + 1 < n_steps;
        if (has_next) load_tile(st + 1);

        const uint16_t* Qb = Qs[buf];
        const uint16_t* dOb = dOs[buf];
        const bool masked = (CAUSAL && i0 < j0 + BC) || !full_cols;
        // one 32-row half of the query tile at a time keeps S and dP at 32 registers
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            f32x16 sa = zero16(), pa = zero16();
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                sa = T::mma(ld16(&Qb[(mb * 32 + c) * QP + 16 * s + 8 * g]), kreg[s], sa);
                pa = T::mma(ld16(&dOb[(mb * 32 + c) * QP + 16 * s + 8 * g]), vreg[s], pa);
            }
            if (masked)
                softmax_grad_tile<true, CAUSAL>(sa, pa, &lse_s[buf][mb * 32], &dlt_s[buf][mb * 32],
                                                p.scale_log2, g, i0 + mb * 32, my_j, col_ok);
            else
                softmax_grad_tile<false, CAUSAL>(sa, pa, &lse_s[buf][mb * 32], &dlt_s[buf][mb * 32],
                                                 p.scale_log2, g, i0 + mb * 32, my_j, col_ok);
            if (mb == MB - 1 && has_next) store_tile(buf ^ 1);
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                const u32x4 bP = acc_to_operand<T>(sa, hh);
                const u32x4 bS = acc_to_operand<T>(pa, hh);
#pragma unroll
                for (int db = 0; db < DB; ++db) {
                    dva[db] = T::mma(ld_tr<true>(dOb, QP, mb * 32 + 16 * hh, db * 32, lane), bP, dva[db]);
                    dka[db] = T::mma(ld_tr<true>(Qb, QP, mb * 32 + 16 * hh, db * 32, lane), bS, dka[db]);
                }
                if (DQ_ATOMIC) {
                    // dS^T rows j = 32w + c; bS holds query rows 16hh + 4g + 0..3 and
                    // 16hh + 8 + 4g + 0..3 of this half tile, packed in pairs
                    u32x2 lo, hi;
                    lo[0] = bS[0]; lo[1] = bS[1]; hi[0] = bS[2]; hi[1] = bS[3];
                    st8(&dST[(32 * w + c) * SP + mb * 32 + 16 * hh + 4 * g], lo);
                    st8(&dST[(32 * w + c) * SP + mb * 32 + 16 * hh + 8 + 4 * g], hi);
                }
            }
        }

        if (DQ_ATOMIC) {
            __syncthreads();
            f32x16 acc[NBLK];
#pragma unroll
            for (int x = 0; x < NBLK; ++x) acc[x] = zero16();
#pragma unroll
            for (int ks = 0; ks < BC / 16; ++ks)
#pragma unroll
                for (int x = 0; x < NBLK; ++x) {
                    const int blk = w + x * NW, ib = blk / DB, db = blk % DB;
                    acc[x] = T::mma(ld_tr<false>(dST, SP, 16 * ks, ib * 32, lane),
                                    ld_tr<false>(Ks, QP, 16 * ks, db * 32, lane), acc[x]);
                }
            // accumulator rows of this (sequence, head): head-major, row stride D floats
            const int64_t arow0 = p.varlen ? ((int64_t)h * p.Sq + q0) : (((int64_t)b * p.Hq + h) * p.Sq);
            float* dqa = p.dqacc + (arow0 + i0) * D + c;
            const bool full_rows = i0 + BR <= lq;
#pragma unroll
            for (int x = 0; x < NBLK; ++x) {
                const int blk = w + x * NW, ib = blk / DB, db = blk % DB;
                float* base = dqa + (ib * 32 + 4 * g) * D + db * 32;
                if (full_rows) {
#pragma unroll
                    for (int rg = 0; rg < 16; ++rg)
                        atomicAdd(base + (8 * (rg >> 2) + (rg & 3)) * D, acc[x][rg]);
                } else {
#pragma unroll
                    for (int rg = 0; rg < 16; ++rg) {
                        const int i = i0 + ib * 32 + 8 * (rg >> 2) + 4 * g + (rg & 3);
                        if (i < lq) atomicAdd(base + (8 * (rg >> 2) + (rg & 3)) * D, acc[x][rg]);
                    }
                }
            }
        }
        __syncthreads();
    }
    (void)ws_step;

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
// Main backward kernel, eight wavefronts (two per SIMD)
// ---------------------------------------------------------------------------
//
// Same work item as bwd_main_kernel (128 keys of one KV head, every query tile
// of every query head of its group) with eight wavefronts: wavefront
// w = kw + 4*rh owns keys 32*kw .. 32*kw+31 and rows 32*rh .. 32*rh+31 of each
// 64-row query tile.  Each SIMD thus runs two wavefronts, so the matrix core
// and the vector ALU of a SIMD overlap, and every wavefront carries half the
// softmax work.  dK/dV accumulate per wavefront over its row half; the two
// halves are summed through LDS once, at the end.  dQ_tile = dS K uses
// v_mfma_f32_16x16x32: wavefront w owns query rows 16*(w/2) .. +15 and head
// dims 32*(w%2) .. +31 of the tile, with its K operand held in registers for
// the whole kernel, so only dS^T is read from LDS per step.

template <int D>
struct Main8Lds {
    static constexpr int BC = 128, BR = 64, QP = D + 8, SP = BR + 8, DB = D / 32;
    static constexpr int TILE_B = BR * QP * 2;
    static constexpr int OFF_ST = 4 * TILE_B;
    static constexpr int OFF_STAT = OFF_ST + BC * (QP > SP ? QP : SP) * 2;
    static constexpr int LOOP_B = OFF_STAT + 4 * BR * 4;
    static constexpr int RED_B = 4 * 64 * (2 * DB * 16) * 4;
    static constexpr int BYTES = LOOP_B > RED_B ? LOOP_B : RED_B;
};

template <class T, int D, bool CAUSAL, bool DQ_ATOMIC>
__device__ __forceinline__ void bwd_main8_body(const BwdParams& p, unsigned char* arena, int bx, int by) {
    constexpr int BC = 128;          // keys per workgroup
    constexpr int BR = 64;           // query rows per step
    constexpr int KS = D / 16;       // k-steps over the head dimension (32x32x16)
    constexpr int DB = D / 32;       // 32-row blocks of dK^T / dV^T
    constexpr int QP = D + 8;        // row stride of Qs, dOs, Ks  [row][d]
    constexpr int SP = BR + 8;       // row stride of dST          [j][i]
    constexpr int CH = BR * D / 8 / 512;     // 16-byte chunks per thread per tile
    constexpr int NQB = D / 32;      // 16-wide head-dim blocks of dQ per wavefront (2 for D=64)
    static_assert(CH >= 1, "tile shape");
    constexpr int TILE_B = BR * QP * 2;                  // bytes of one Q (or dO) tile
    constexpr int OFF_Q = 0, OFF_DO = 2 * TILE_B, OFF_ST = 4 * TILE_B;
    constexpr int OFF_STAT = OFF_ST + BC * (QP > SP ? QP : SP) * 2;
    constexpr int LOOP_B = OFF_STAT + 4 * BR * 4;
    constexpr int RED_B = 4 * 64 * (2 * DB * 16) * 4;   // dK/dV partials of four wavefronts
    static_assert(Main8Lds<D>::BYTES == (LOOP_B > RED_B ? LOOP_B : RED_B), "arena size");
    uint16_t* Qs0 = reinterpret_cast<uint16_t*>(arena + OFF_Q);
    uint16_t* dOs0 = reinterpret_cast<uint16_t*>(arena + OFF_DO);
    uint16_t* dST = reinterpret_cast<uint16_t*>(arena + OFF_ST);
    float* lse_s = reinterpret_cast<float*>(arena + OFF_STAT);          // [2][BR]
    float* dlt_s = lse_s + 2 * BR;                                        // [2][BR]

    const int tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6;
    const int kw = w & 3, rh = w >> 2;
    const int g = lane >> 5, c = lane & 31;
    const int b = bx / p.Hkv, hk = bx % p.Hkv;
    const int G = p.Hq / p.Hkv;
    int q0 = 0, k0 = 0, lq = p.Sq, lk = p.Sk;
    if (p.varlen) seq_get(p.seqs, b, q0, k0, lq, lk);
    const int j0 = by * BC;
    if (j0 >= lk) return;
    const bool full_cols = j0 + BC <= lk;

    const uint16_t* kbase = p.k.p + b * p.k.sb + hk * p.k.sh + (int64_t)k0 * p.k.ss;
    const uint16_t* vbase = p.v.p + b * p.v.sb + hk * p.v.sh + (int64_t)k0 * p.v.ss;

    const int my_j = j0 + 32 * kw + c;
    const bool col_ok = my_j < lk;
    u32x4 kreg[KS], vreg[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) {
        u32x4 z = {0u, 0u, 0u, 0u};
        kreg[s] = col_ok ? ld16(kbase + (int64_t)my_j * p.k.ss + 16 * s + 8 * g) : z;
        vreg[s] = col_ok ? ld16(vbase + (int64_t)my_j * p.v.ss + 16 * s + 8 * g) : z;
    }
    // K operand of the dQ product (k = key, column = head dim), via a row-major
    // staging copy of the key tile in the dS^T area
    u32x4 kop[BC / 32][NQB];
    if (DQ_ATOMIC) {
        uint16_t* Ks = dST;
        if (rh == 0) {
#pragma unroll
            for (int s = 0; s < KS; ++s) st16(&Ks[(32 * kw + c) * QP + 16 * s + 8 * g], kreg[s]);
        }
        __syncthreads();
#pragma unroll
        for (int ks = 0; ks < BC / 32; ++ks)
#pragma unroll
            for (int nb = 0; nb < NQB; ++nb)
                kop[ks][nb] = ld_tr16x16(Ks, QP, 32 * ks, (w & 1) * (16 * NQB) + 16 * nb, lane);
        __syncthreads();
    }

    f32x16 dva[DB], dka[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) { dva[db] = zero16(); dka[db] = zero16(); }

    const int i_begin = CAUSAL ? (j0 / BR) * BR : 0;
    const int per_head = lq > i_begin ? (lq - i_begin + BR - 1) / BR : 0;
    const int n_steps = G * per_head;

    int qoff[CH], dooff[CH], ooff[CH], crow[CH];
#pragma unroll
    for (int x = 0; x < CH; ++x) {
        const int e = tid + 512 * x;
        const int r = e / (D / 8), cc = (e % (D / 8)) * 8;
        crow[x] = r;
        qoff[x] = r * (int)p.q.ss + cc;
        dooff[x] = r * (int)p.dout.ss + cc;
        ooff[x] = r * (int)p.o.ss + cc;
    }

    // Each step's 64 rows arrive as 16-byte chunks of Q, dO and O; the row's
    // Delta = sum_d dO*O is reduced across the D/8 consecutive lanes holding
    // it, and its LSE is read from the caller's statistics: no separate pass.
    u32x4 pq[CH], pdo[CH], po[CH];
    float pl = INFINITY;
    auto load_tile = [&](int st) {
        const int h = hk * G + st / per_head;
        const int i0 = i_begin + (st % per_head) * BR;
        const uint16_t* qb = p.q.p + b * p.q.sb + h * p.q.sh + (int64_t)(q0 + i0) * p.q.ss;
        const uint16_t* dob = p.dout.p + b * p.dout.sb + h * p.dout.sh + (int64_t)(q0 + i0) * p.dout.ss;
        const uint16_t* ob = p.o.p + b * p.o.sb + h * p.o.sh + (int64_t)(q0 + i0) * p.o.ss;
        if (i0 + BR <= lq) {
#pragma unroll
            for (int x = 0; x < CH; ++x) {
                pq[x] = ld16(qb + qoff[x]);
                pdo[x] = ld16(dob + dooff[x]);
                po[x] = ld16(ob + ooff[x]);
            }
        } else {
#pragma unroll
            for (int x = 0; x < CH; ++x) {
                u32x4 z = {0u, 0u, 0u, 0u};
                const bool ok = i0 + crow[x] < lq;
                pq[x] = ok ? ld16(qb + qoff[x]) : z;
                pdo[x] = ok ? ld16(dob + dooff[x]) : z;
                po[x] = ok ? ld16(ob + ooff[x]) : z;
            }
        }
        if (tid < BR) {
            const int i = i0 + tid;
            pl = i < lq ? stats_lse2(p, b * p.st_sb + h * p.st_sh + (int64_t)(q0 + i) * p.st_ss) : INFINITY;
        }
    };
    auto store_tile = [&](int buf) {
        uint16_t* Qd = Qs0 + buf * (BR * QP);
        uint16_t* dOd = dOs0 + buf * (BR * QP);
#pragma unroll
        for (int x = 0; x < CH; ++x) {
            const int e = tid + 512 * x;
            const int r = e / (D / 8), cc = (e % (D / 8)) * 8;
            st16(&Qd[r * QP + cc], pq[x]);
            st16(&dOd[r * QP + cc], pdo[x]);
            float dsum = dot8<T>(pdo[x], po[x]);
#pragma unroll
            for (int o = D / 16; o > 0; o >>= 1) dsum += __shfl_xor(dsum, o);
            if (cc == 0) dlt_s[buf * BR + r] = dsum;
        }
        if (tid < BR) lse_s[buf * BR + tid] = pl;
    };

    if (n_steps > 0) {
        load_tile(0);
        store_tile(0);
    }
    __syncthreads();

    for (int st = 0; st < n_steps; ++st) {
        const int buf = st & 1;
        const int h = hk * G + st / per_head;
        const int i0 = i_begin + (st % per_head) * BR;
        const bool has_next = st + 1 < n_steps;
        if (has_next) load_tile(st + 1);

        const uint16_t* Qb = Qs0 + buf * (BR * QP);
        const uint16_t* dOb = dOs0 + buf * (BR * QP);
        const bool masked = (CAUSAL && i0 < j0 + BC) || !full_cols;
        f32x16 sa = zero16(), pa = zero16();
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            sa = T::mma(ld16(&Qb[(32 * rh + c) * QP + 16 * s + 8 * g]), kreg[s], sa);
            pa = T::mma(ld16(&dOb[(32 * rh + c) * QP + 16 * s + 8 * g]), vreg[s], pa);
        }
        if (masked)
            softmax_grad_tile<true, CAUSAL>(sa, pa, &lse_s[buf * BR + 32 * rh], &dlt_s[buf * BR + 32 * rh],
                                            p.scale_log2, g, i0 + 32 * rh, my_j, col_ok);
        else
            softmax_grad_tile<false, CAUSAL>(sa, pa, &lse_s[buf * BR + 32 * rh], &dlt_s[buf * BR + 32 * rh],
                                             p.scale_log2, g, i0 + 32 * rh, my_j, col_ok);
        if (has_next) store_tile(buf ^ 1);
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            const u32x4 bP = acc_to_operand<T>(sa, hh);
            const u32x4 bS = acc_to_operand<T>(pa, hh);
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                dva[db] = T::mma(ld_tr<true>(dOb, QP, 32 * rh + 16 * hh, db * 32, lane), bP, dva[db]);
                dka[db] = T::mma(ld_tr<true>(Qb, QP, 32 * rh + 16 * hh, db * 32, lane), bS, dka[db]);
            }
            if (DQ_ATOMIC) {
                u32x2 lo, hi;
                lo[0] = bS[0]; lo[1] = bS[1]; hi[0] = bS[2]; hi[1] = bS[3];
                st8(&dST[(32 * kw + c) * SP + 32 * rh + 16 * hh + 4 * g], lo);
                st8(&dST[(32 * kw + c) * SP + 32 * rh + 16 * hh + 8 + 4 * g], hi);
            }
        }

        if (DQ_ATOMIC) {
            __syncthreads();
            const int ib = w >> 1;                 // query rows 16*ib .. +15 of the tile
            f32x4 acc[NQB];
#pragma unroll
            for (int nb = 0; nb < NQB; ++nb) acc[nb] = zero4();
#pragma unroll
            for (int ks = 0; ks < BC / 32; ++ks) {
                const u32x4 a = ld_tr16x16(dST, SP, 32 * ks, 16 * ib, lane);
#pragma unroll
                for (int nb = 0; nb < NQB; ++nb) acc[nb] = T::mma16(a, kop[ks][nb], acc[nb]);
            }
            const int64_t arow0 = p.varlen ? ((int64_t)h * p.Sq + q0) : (((int64_t)b * p.Hq + h) * p.Sq);
            const int G16 = lane >> 4, col = lane & 15;
            float* base = p.dqacc + (arow0 + i0 + 16 * ib + 4 * G16) * D + (w & 1) * (16 * NQB) + col;
            if (i0 + BR <= lq) {
#pragma unroll
                for (int nb = 0; nb < NQB; ++nb)
#pragma unroll
                    for (int r = 0; r < 4; ++r) atomicAdd(base + r * D + 16 * nb, acc[nb][r]);
            } else {
#pragma unroll
                for (int nb = 0; nb < NQB; ++nb)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        if (i0 + 16 * ib + 4 * G16 + r < lq) atomicAdd(base + r * D + 16 * nb, acc[nb][r]);
            }
        }
        __syncthreads();
    }

    // sum the two row halves' dK/dV partials through LDS, then store
    float* red = reinterpret_cast<float*>(arena);
    if (rh == 1) {
#pragma unroll
        for (int a = 0; a < 2 * DB; ++a) {
            const f32x16& v = a < DB ? dva[a] : dka[a - DB];
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                f32x4 x = {v[4 * r4 + 0], v[4 * r4 + 1], v[4 * r4 + 2], v[4 * r4 + 3]};
                *reinterpret_cast<f32x4*>(&red[(((kw * 2 * DB + a) * 4 + r4) * 64 + lane) * 4]) = x;
            }
        }
    }
    __syncthreads();
    if (rh == 1 || !col_ok) return;
#pragma unroll
    for (int a = 0; a < 2 * DB; ++a) {
        f32x16& v = a < DB ? dva[a] : dka[a - DB];
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
            const f32x4 x = *reinterpret_cast<const f32x4*>(&red[(((kw * 2 * DB + a) * 4 + r4) * 64 + lane) * 4]);
            v[4 * r4 + 0] += x[0]; v[4 * r4 + 1] += x[1]; v[4 * r4 + 2] += x[2]; v[4 * r4 + 3] += x[3];
        }
    }
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

template <class T, int D, bool CAUSAL, bool DQ_ATOMIC>
__global__ __launch_bounds__(512) void bwd_main8_kernel(BwdParams p) {
    __shared__ __align__(16) unsigned char arena[Main8Lds<D>::BYTES];
    bwd_main8_body<T, D, CAUSAL, DQ_ATOMIC>(p, arena, blockIdx.x, blockIdx.y);
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
    const f32x4* src = reinterpret_cast<const f32x4*>(p.dqacc + acc_row(p, L, R) * D + part * 8);
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
// dQ pass without atomics, eight wavefronts (query-tile outer)
// ---------------------------------------------------------------------------
//
// One workgroup per (sequence, query head, 64-row query tile); it walks the
// 128-key tiles the tile can see.  Wavefront w = kw + 4*rh owns query rows
// 32*rh .. +31 and keys 32*kw .. +31 of every key tile.  Scores are computed
// transposed, S^T = K Q^T and dP^T = V dO^T, so that each lane holds one query
// column: its LSE and Delta are lane-uniform, and dS^T feeds
// dQ^T += K^T dS^T directly as the B operand.  Q and dO stay in registers for
// the whole kernel; key tiles stream through a double-buffered LDS copy whose
// next tile is loaded into registers while the current one is used.  Each
// wavefront accumulates dQ^T over its key slices; the four slices are summed
// through LDS at the end and dQ is written once, scaled and rounded.

template <int D>
struct Dq8Lds {
    static constexpr int BK = 128, KP = D + 8, DB = D / 32;
    static constexpr int TILE_B = BK * KP * 2;
    static constexpr int LOOP_B = 4 * TILE_B;
    static constexpr int RED_B = 3 * 2 * 64 * (DB * 16) * 4;
    static constexpr int BYTES = LOOP_B > RED_B ? LOOP_B : RED_B;
};

template <class T, int D, bool CAUSAL>
__device__ __forceinline__ void bwd_dq8_body(const BwdParams& p, unsigned char* arena, int bx, int by) {
    constexpr int BQ = 64;           // query rows per workgroup
    constexpr int BK = 128;          // keys per step
    constexpr int KS = D / 16;       // k-steps over the head dimension (32x32x16)
    constexpr int DB = D / 32;       // 32-row blocks of dQ^T
    constexpr int KP = D + 8;        // row stride of Ks, Vs  [key][d]
    constexpr int CH = BK * D / 8 / 512;     // 16-byte chunks per thread per key tile
    constexpr int TILE_B = BK * KP * 2;
    constexpr int OFF_K = 0, OFF_V = 2 * TILE_B;
    constexpr int LOOP_B = 4 * TILE_B;
    constexpr int RED_B = 3 * 2 * 64 * (DB * 16) * 4;    // three key slices of both row halves
    static_assert(Dq8Lds<D>::BYTES == (LOOP_B > RED_B ? LOOP_B : RED_B), "arena size");
    uint16_t* Ks0 = reinterpret_cast<uint16_t*>(arena + OFF_K);
    uint16_t* Vs0 = reinterpret_cast<uint16_t*>(arena + OFF_V);

    const int tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6;
    const int kw = w & 3, rh = w >> 2;
    const int g = lane >> 5, c = lane & 31;
    const int b = by / p.Hq, h = by % p.Hq;
    const int hk = h / (p.Hq / p.Hkv);
    int q0 = 0, k0 = 0, lq = p.Sq, lk = p.Sk;
    if (p.varlen) seq_get(p.seqs, b, q0, k0, lq, lk);
    const int i0 = bx * BQ;
    if (i0 >= lq) return;

    const uint16_t* qbase = p.q.p + b * p.q.sb + h * p.q.sh + (int64_t)q0 * p.q.ss;
    const uint16_t* dobase = p.dout.p + b * p.dout.sb + h * p.dout.sh + (int64_t)q0 * p.dout.ss;
    const uint16_t* kbase = p.k.p + b * p.k.sb + hk * p.k.sh + (int64_t)k0 * p.k.ss;
    const uint16_t* vbase = p.v.p + b * p.v.sb + hk * p.v.sh + (int64_t)k0 * p.v.ss;

    const int my_i = i0 + 32 * rh + c;
    const bool row_ok = my_i < lq;
    u32x4 qreg[KS], doreg[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) {
        u32x4 z = {0u, 0u, 0u, 0u};
        qreg[s] = row_ok ? ld16(qbase + (int64_t)my_i * p.q.ss + 16 * s + 8 * g) : z;
        doreg[s] = row_ok ? ld16(dobase + (int64_t)my_i * p.dout.ss + 16 * s + 8 * g) : z;
    }
    // this row's LSE from the caller's statistics and Delta = sum_d dO*O: the two
    // lane halves hold alternate 8-element chunks of the row
    const float l2 = row_ok ? stats_lse2(p, b * p.st_sb + h * p.st_sh + (int64_t)(q0 + my_i) * p.st_ss) : INFINITY;
    float dl = 0.f;
    {
        const uint16_t* orow = p.o.p + b * p.o.sb + h * p.o.sh + (int64_t)(q0 + my_i) * p.o.ss;
#pragma unroll
        for (int s = 0; s < KS; ++s)
            if (row_ok) dl += dot8<T>(doreg[s], ld16(orow + 16 * s + 8 * g));
        dl += __shfl_xor(dl, 32);
    }

    f32x16 dq[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) dq[db] = zero16();

    const int kend = CAUSAL ? min(lk, i0 + BQ) : lk;
    const int n_steps = (kend + BK - 1) / BK;

    int koff[CH], voff[CH], crow[CH];
#pragma unroll
    for (int x = 0; x < CH; ++x) {
        const int e = tid + 512 * x;
        const int r = e / (D / 8), cc = (e % (D / 8)) * 8;
        crow[x] = r;
        koff[x] = r * (int)p.k.ss + cc;
        voff[x] = r * (int)p.v.ss + cc;
    }
    u32x4 pk[CH], pv[CH];
    auto load_tile = [&](int st) {
        const int j0 = st * BK;
        const uint16_t* kb = kbase + (int64_t)j0 * p.k.ss;
        const uint16_t* vb = vbase + (int64_t)j0 * p.v.ss;
        if (j0 + BK <= lk) {
#pragma unroll
            for (int x = 0; x < CH; ++x) {
                pk[x] = ld16(kb + koff[x]);
                pv[x] = ld16(vb + voff[x]);
            }
        } else {
#pragma unroll
            for (int x = 0; x < CH; ++x) {
                u32x4 z = {0u, 0u, 0u, 0u};
                const bool ok = j0 + crow[x] < lk;
                pk[x] = ok ? ld16(kb + koff[x]) : z;
                pv[x] = ok ? ld16(vb + voff[x]) : z;
            }
        }
    };
    auto store_tile = [&](int buf) {
        uint16_t* Kd = Ks0 + buf * (BK * KP);
        uint16_t* Vd = Vs0 + buf * (BK * KP);
#pragma unroll
        for (int x = 0; x < CH; ++x) {
            const int e = tid + 512 * x;
            const int r = e / (D / 8), cc = (e % (D / 8)) * 8;
            st16(&Kd[r * KP + cc], pk[x]);
            st16(&Vd[r * KP + cc], pv[x]);
        }
    };

    if (n_steps > 0) {
        load_tile(0);
        store_tile(0);
    }
    __syncthreads();

    for (int st = 0; st < n_steps; ++st) {
        const int buf = st & 1;
        const int j0 = st * BK;
        const bool has_next = st + 1 < n_steps;
        if (has_next) load_tile(st + 1);
        const uint16_t* Kb = Ks0 + buf * (BK * KP);
        const uint16_t* Vb = Vs0 + buf * (BK * KP);

        f32x16 s = zero16(), dp = zero16();
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            s = T::mma(ld16(&Kb[(32 * kw + c) * KP + 16 * ks + 8 * g]), qreg[ks], s);
            dp = T::mma(ld16(&Vb[(32 * kw + c) * KP + 16 * ks + 8 * g]), doreg[ks], dp);
        }
        // element (rg): key j = j0 + 32kw + 8(rg/4) + 4g + rg%4, query my_i
        const bool masked = (CAUSAL && j0 + BK > i0) || (j0 + BK > lk);
        if (masked) {
#pragma unroll
            for (int rg = 0; rg < 16; ++rg) {
                const int j = j0 + 32 * kw + 8 * (rg >> 2) + 4 * g + (rg & 3);
                float pvv = fast_exp2(__builtin_fmaf(s[rg], p.scale_log2, -l2));
                const bool keep = (j < lk) & (!CAUSAL | (j <= my_i));
                pvv = keep ? pvv : 0.f;
                dp[rg] = pvv * (dp[rg] - dl);
            }
        } else {
#pragma unroll
            for (int rg = 0; rg < 16; ++rg) {
                const float pvv = fast_exp2(__builtin_fmaf(s[rg], p.scale_log2, -l2));
                dp[rg] = pvv * (dp[rg] - dl);
            }
        }
        if (has_next) store_tile(buf ^ 1);
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            const u32x4 bS = acc_to_operand<T>(dp, hh);
#pragma unroll
            for (int db = 0; db < DB; ++db)
                dq[db] = T::mma(ld_tr<true>(Kb, KP, 32 * kw + 16 * hh, db * 32, lane), bS, dq[db]);
        }
        __syncthreads();
    }

    // sum the four key slices through LDS (slices 1..3 write, slice 0 adds)
    float* red = reinterpret_cast<float*>(arena);
    if (kw != 0) {
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                f32x4 x = {dq[db][4 * r4 + 0], dq[db][4 * r4 + 1], dq[db][4 * r4 + 2], dq[db][4 * r4 + 3]};
                *reinterpret_cast<f32x4*>(&red[(((((kw - 1) * 2 + rh) * DB + db) * 4 + r4) * 64 + lane) * 4]) = x;
            }
    }
    __syncthreads();
    if (kw != 0 || !row_ok) return;
#pragma unroll
    for (int sl = 0; sl < 3; ++sl)
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const f32x4 x = *reinterpret_cast<const f32x4*>(&red[((((sl * 2 + rh) * DB + db) * 4 + r4) * 64 + lane) * 4]);
                dq[db][4 * r4 + 0] += x[0]; dq[db][4 * r4 + 1] += x[1];
                dq[db][4 * r4 + 2] += x[2]; dq[db][4 * r4 + 3] += x[3];
            }
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

template <class T, int D, bool CAUSAL>
__global__ __launch_bounds__(512) void bwd_dq8_kernel(BwdParams p) {
    __shared__ __align__(16) unsigned char arena[Dq8Lds<D>::BYTES];
    bwd_dq8_body<T, D, CAUSAL>(p, arena, blockIdx.x, blockIdx.y);
}

// dK/dV and dQ in one launch: the first n_main workgroups run the key-tile
// outer kernel (key tiles in ascending order, so the longest causal ranges
// start first), the rest the query-tile outer dQ kernel (query tiles in
// descending order).  The dQ workgroups fill the CUs the long dK/dV
// workgroups leave idle near the end.
template <class T, int D, bool CAUSAL>
__global__ __launch_bounds__(512) void bwd_fused8_kernel(BwdParams p, int main_x, int main_y, int dq_x, int dq_y) {
    constexpr int A = Main8Lds<D>::BYTES > Dq8Lds<D>::BYTES ? Main8Lds<D>::BYTES : Dq8Lds<D>::BYTES;
    __shared__ __align__(16) unsigned char arena[A];
    const int id = blockIdx.x;
    const int n_main = main_x * main_y;
    if (id < n_main) {
        bwd_main8_body<T, D, CAUSAL, false>(p, arena, id % main_x, id / main_x);
    } else {
        const int r = id - n_main;
        bwd_dq8_body<T, D, CAUSAL>(p, arena, dq_x - 1 - r / dq_y, r % dq_y);
    }
}

// fp32 zero fill (16 bytes per thread) of the dQ accumulator in atomic mode
__global__ __launch_bounds__(256) void fill_zero_kernel(float* dst, int64_t n4) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n4) {
        f32x4 z = {0.f, 0.f, 0.f, 0.f};
        reinterpret_cast<f32x4*>(dst)[i] = z;
    }
}

// ---------------------------------------------------------------------------
// Launch
// ---------------------------------------------------------------------------

template <class T, int D, bool CAUSAL>
static hipError_t launch_bwd_t(const BwdParams& p, const BwdLaunch& L, hipStream_t st) {
    const int64_t row_threads = p.rows * (D / 8);
    const dim3 row_grid((unsigned)((row_threads + 255) / 256));   // dQ conversion: 8 elements per thread
    const bool have_rows = p.rows > 0;
    constexpr bool W8 = D == 64;   // eight-wavefront kernels read the statistics and O themselves
    if ((L.phase & BwdLaunch::kFirst) && have_rows) {
        if constexpr (W8) {
            if (!L.deterministic) {
                const int64_t n4 = p.rows * D / 4;
                PROF_LAUNCH(KID_BWD_PRE, st, fill_zero_kernel, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, st,
                            p.dqacc, n4);
            }
        } else {
            PROF_LAUNCH(KID_BWD_PRE, st, (bwd_pre_kernel<T, D>), dim3((unsigned)((p.rows * (D / 16) + 255) / 256)),
                        dim3(256), 0, st, p, L.deterministic ? 0 : 1);
        }
    }
    const dim3 main_grid(L.n_seq * p.Hkv, L.max_kv_tiles);
    const bool have_main = main_grid.x > 0 && main_grid.y > 0;
    const dim3 main_block(W8 ? 512 : 256);
    if (L.deterministic) {
        if constexpr (W8) {
            const int mx = (int)main_grid.x, my = (int)main_grid.y;
            const int qx = L.max_q_tiles64, qy = L.n_seq * p.Hq;
            const int n = mx * my + qx * qy;
            if (n > 0)
                PROF_LAUNCH(KID_BWD_MAIN, st, (bwd_fused8_kernel<T, D, CAUSAL>), dim3(n), dim3(512), 0, st, p,
                            mx, my, qx, qy);
        } else {
            if (have_main)
                PROF_LAUNCH(KID_BWD_MAIN, st, (bwd_main_kernel<T, D, CAUSAL, false>), main_grid, main_block, 0, st, p);
            const dim3 dq_grid(L.max_q_tiles128, L.n_seq * p.Hq);
            if (dq_grid.x > 0 && dq_grid.y > 0)
                PROF_LAUNCH(KID_BWD_DQ_DET, st, (bwd_dq_kernel<T, D, CAUSAL>), dq_grid, dim3(256), 0, st, p);
        }
    } else {
        if constexpr (W8) {
            if (have_main)
                PROF_LAUNCH(KID_BWD_MAIN, st, (bwd_main8_kernel<T, D, CAUSAL, true>), main_grid, main_block, 0, st, p);
        } else if (have_main) {
            PROF_LAUNCH(KID_BWD_MAIN, st, (bwd_main_kernel<T, D, CAUSAL, true>), main_grid, main_block, 0, st, p);
        }
        if ((L.phase & BwdLaunch::kLast) && have_rows)
            PROF_LAUNCH(KID_BWD_DQ_CONVERT, st, (bwd_dq_convert_kernel<T, D>), row_grid, dim3(256), 0, st, p);
    }
    return hipGetLastError();
}

template <class T, int D>
static hipError_t launch_bwd_d(const BwdParams& p, const BwdLaunch& L, hipStream_t st) {
    return L.causal ? launch_bwd_t<T, D, true>(p, L, st) : launch_bwd_t<T, D, false>(p, L, st);
}

template <class T, int D>
static hipError_t launch_pre_t(const BwdParams& p, bool zero_dq, hipStream_t st) {
    const int64_t row_threads = p.rows * (D / 16);
    if (row_threads > 0)
        PROF_LAUNCH(KID_BWD_PRE, st, (bwd_pre_kernel<T, D>), dim3((unsigned)((row_threads + 255) / 256)), dim3(256),
                    0, st, p, zero_dq ? 1 : 0);
    return hipGetLastError();
}

hipError_t launch_bwd_pre(const BwdParams& p, int dtype, int D, bool zero_dq, hipStream_t st) {
    if (dtype == 0) return D == 64 ? launch_pre_t<F16, 64>(p, zero_dq, st) : launch_pre_t<F16, 128>(p, zero_dq, st);
    return D == 64 ? launch_pre_t<BF16, 64>(p, zero_dq, st) : launch_pre_t<BF16, 128>(p, zero_dq, st);
}

hipError_t launch_bwd(const BwdParams& p, const BwdLaunch& L, hipStream_t st) {
    if (L.dtype == 0)
        return L.D == 64 ? launch_bwd_d<F16, 64>(p, L, st) : launch_bwd_d<F16, 128>(p, L, st);
    return L.D == 64 ? launch_bwd_d<BF16, 64>(p, L, st) : launch_bwd_d<BF16, 128>(p, L, st);
}

}  // namespace sdpa
