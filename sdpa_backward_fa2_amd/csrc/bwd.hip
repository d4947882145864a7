// SDPA backward, FlashAttention-2 style, for gfx950.
//
// Kernels (all on the caller's stream):
//   bwd_pre_kernel     per row: Delta = sum_d dO*O, the statistics as
//                      log2-domain LSE, and (D=128 atomic mode) the fp32 dQ
//                      accumulator row cleared.                   [HBM-bound]
//   bwd_fused8_kernel  D=64: one launch of four-wavefront workgroups, two per
//                      CU, running work items of two kinds: the key-tile
//                      outer body (dK, dV of 64 keys over every query tile of
//                      every query head of the group) and a query-tile outer
//                      body (dQ of 64 rows, or of 128 rows in the wide form
//                      for large causal problems, over the key tiles they
//                      see).  No atomics.                                [MFMA]
//   bwd_main_kernel    D=128: one four-wavefront workgroup per (sequence, KV
//                      head, 128-key tile); dK and dV accumulate in registers
//                      across every query tile of every query head of the
//                      group; per 64-row query tile S, dP, dV, dK and, in
//                      atomic mode, dQ += dS K through fp32 atomics.     [MFMA]
//   bwd_dq_convert     D=128 atomic mode: dQ = scale * accumulator, rounded.
//   bwd_dq8_kernel     D=128 deterministic mode: the query-tile outer dQ body
//                      as its own launch.                                [MFMA]
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

// log2-domain LSE of one row from the caller's statistics (a = LSE, or a = row
// max and b = row sum): LSE*log2e, or m*log2e + log2(l); +inf for a row
// without keys, so that its P is exactly zero.
__device__ __forceinline__ float stats_to_lse2(int kind, float a, float b) {
    if (kind == 0) return (a == -INFINITY) ? INFINITY : a * kLog2e;
    return (b > 0.f) ? a * kLog2e + log2f(b) : INFINITY;
}

template <class T>
__device__ __forceinline__ float dot8(u32x4 a, u32x4 b, float acc = 0.f) {
    acc = T::dot2(a[0], b[0], acc);
    acc = T::dot2(a[1], b[1], acc);
    acc = T::dot2(a[2], b[2], acc);
    return T::dot2(a[3], b[3], acc);
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

// Grid, LPR lanes per row (a power of two; 16 elements per lane at D=64 and
// 128, 24 at D=192): dense, x = chunks of rows of one (batch, head) = y;
// packed, x = chunks of the (token, head) rows in memory order (the heads of
// a token are adjacent in the packed layout).
template <int D>
constexpr int pre_lanes() { return D == 64 ? 4 : 8; }
template <int D>
constexpr int pre_rows_per_block() { return 256 / pre_lanes<D>(); }

template <class T, int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(BwdParams p, int zero_dq) {
    constexpr int LPR = pre_lanes<D>();
    constexpr int EPL = D / LPR;                 // elements per lane
    constexpr int NC = EPL / 8;                  // 16-byte chunks per lane
    static_assert(EPL % 8 == 0 && (LPR & (LPR - 1)) == 0, "row split");
    constexpr int RPB = pre_rows_per_block<D>();
    const int part = threadIdx.x % LPR;
    int64_t R;
    bool ok;
    RowLoc L;
    if (p.varlen) {
        R = (int64_t)blockIdx.x * RPB + threadIdx.x / LPR;
        ok = R < p.rows;
        const int64_t Rc = ok ? R : p.rows - 1;           // rows past the end re-read the last
        L = RowLoc{0, Rc % p.Hq, Rc / p.Hq};
    } else {
        const int i = blockIdx.x * RPB + threadIdx.x / LPR;
        const int y = blockIdx.y;
        ok = i < p.Sq;
        R = (int64_t)y * p.Sq + i;
        L = RowLoc{y / p.Hq, y % p.Hq, min(i, p.Sq - 1)};
    }
    const uint16_t* op = p.o.p + toff(p.o, L) + part * EPL;
    const uint16_t* dp = p.dout.p + toff(p.dout, L) + part * EPL;
    u32x4 oc[NC], dc[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        oc[c] = ld16(op + 8 * c);
        dc[c] = ld16(dp + 8 * c);
    }
    const int64_t so = L.b * p.st_sb + L.h * p.st_sh + L.i * p.st_ss;
    const float sa = p.st_a[so];
    const float sb = p.stats_kind ? p.st_b[so] : 0.f;
    float acc = 0.f;
#pragma unroll
    for (int c = 0; c < NC; ++c) acc = dot8<T>(dc[c], oc[c], acc);
#pragma unroll
    for (int off = LPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
    if (!ok) return;
    if (part == 0) {
        p.delta[R] = acc;
        p.lse2[R] = stats_to_lse2(p.stats_kind, sa, sb);
    }
    if (zero_dq) {
        f32x4 z = {0.f, 0.f, 0.f, 0.f};
        f32x4* dst = reinterpret_cast<f32x4*>(p.dqacc + acc_row(p, L, R) * D + part * EPL);
#pragma unroll
        for (int c = 0; c < EPL / 4; ++c) dst[c] = z;
    }
}

template <class T, int D>
static void launch_pre(const BwdParams& p, int zero_dq, hipStream_t st) {
    constexpr int RPB = pre_rows_per_block<D>();
    const dim3 grid = p.varlen ? dim3((unsigned)((p.rows + RPB - 1) / RPB), 1)
                               : dim3((unsigned)((p.Sq + RPB - 1) / RPB), (unsigned)(p.B * p.Hq));
    if (grid.x > 0 && grid.y > 0)
        PROF_LAUNCH(KID_BWD_PRE, st, (bwd_pre_kernel<T, D>), grid, dim3(256), 0, st, p, zero_dq);
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
// C tile held as (sa, pa), whose dP accumulator started from -Delta (pa
// already holds dP - Delta); rows 8q + 4g + r of the tile, this lane's key.  Element (q, r) is kept when 8q + r >= t, with t the first
// kept row offset of this lane's key (INT_MAX for a key past the end).
template <bool MASKED>
__device__ __forceinline__ void softmax_grad_tile_nd(f32x16& sa, f32x16& pa, const float* lse_row,
                                                     float scale_log2, int g, int t) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const f32x4 Lr = *reinterpret_cast<const f32x4*>(&lse_row[8 * q + 4 * g]);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int rg = 4 * q + r;
            float pv = fast_exp2(__builtin_fmaf(sa[rg], scale_log2, -Lr[r]));
            if (MASKED) pv = (8 * q + r >= t) ? pv : 0.f;
            sa[rg] = pv;
            pa[rg] = pv * pa[rg];
        }
    }
}

// Dispatch places consecutive workgroups (x fastest) on consecutive XCDs of
// the eight.  For a grid of n_unit units (heads, whose workgroups share their
// tensors) of n_item items each, linear slot L is mapped so that XCD L % 8
// runs the items of one unit after another: its concurrently running
// workgroups then share a unit's data in that XCD's L2, instead of every XCD
// reading every unit.  Needs n_unit % 8 == 0 (else the plain mapping).  A
// bijection on [0, n_unit * n_item).
__device__ __forceinline__ void xcd_unit_order(int n_unit, int n_item, int L, int& unit, int& item) {
    if (n_unit & 7) {
        unit = L % n_unit;
        item = L / n_unit;
        return;
    }
    const int xcd = L & 7, slot = L >> 3;
    unit = (slot / n_item) * 8 + xcd;
    item = slot % n_item;
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
    // Grid (sequence x KV head, key tile): the key tiles go out longest causal
    // range first, and with gridDim.x a multiple of 8 each (sequence, KV head)
    // stays on one XCD, whose L2 its workgroups share.  (Ordering one unit's
    // tiles together instead, as the dQ kernel does, was measured 7-9 % slower
    // here: this kernel runs one workgroup per CU and needs the longest-first
    // order more than the locality.)
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

    // per-thread byte offsets of its 16-byte chunks inside a tile (row r,
    // column cc); row strides are below 2^23 elements, so they fit 32 bits
    const uint32_t qss = 2u * (uint32_t)p.q.ss, doss = 2u * (uint32_t)p.dout.ss;
    const int64_t ws_ss = p.varlen ? p.Hq : 1;      // row stride of lse2 / delta
    const uint32_t wss = 4u * (uint32_t)ws_ss;
    uint32_t qoff[CH], dooff[CH];
    int crow[CH], ccol[CH];
#pragma unroll
    for (int x = 0; x < CH; ++x) {
        const int e = tid + 256 * x;
        const int r = e / (D / 8), cc = (e % (D / 8)) * 8;
        crow[x] = r;
        ccol[x] = cc;
        qoff[x] = r * qss + 2 * cc;
        dooff[x] = r * doss + 2 * cc;
    }

    // Cursor of the tile to load next (head ld_h, rows from ld_i0): the query
    // rows of one head from i_begin to the end, then the next head of the
    // group; pointers advance in scalar registers.
    int ld_h = hk * G, ld_i0 = i_begin;
    const uint16_t *ld_q, *ld_do;
    const float *ld_l, *ld_d;
    auto seek = [&]() {
        ld_q = p.q.p + b * p.q.sb + ld_h * p.q.sh + (int64_t)(q0 + ld_i0) * p.q.ss;
        ld_do = p.dout.p + b * p.dout.sb + ld_h * p.dout.sh + (int64_t)(q0 + ld_i0) * p.dout.ss;
        const int64_t ws = p.varlen ? (int64_t)(q0 + ld_i0) * p.Hq + ld_h : ((int64_t)b * p.Hq + ld_h) * p.Sq + ld_i0;
        ld_l = p.lse2 + ws;
        ld_d = p.delta + ws;
    };
    seek();

    // Tile loads are unconditional (rows past the end re-read the last row),
    // and nothing loaded is used before store_tile, so the prefetch of the next
    // tile is not waited for until the current step's products are issued.
    u32x4 pq[CH], pdo[CH];
    float pl = INFINITY, pd = 0.f;
    int pi0 = 0;
    auto load_tile = [&]() {
        uint32_t oq[CH], odo[CH];
        uint32_t so = (uint32_t)(tid & (BR - 1)) * wss;
        if (ld_i0 + BR <= lq) {
#pragma unroll
            for (int x = 0; x < CH; ++x) { oq[x] = qoff[x]; odo[x] = dooff[x]; }
        } else {
            const int last = lq - 1 - ld_i0;
#pragma unroll
            for (int x = 0; x < CH; ++x) {
                const uint32_t r = min(crow[x], last);
                oq[x] = r * qss + 2 * ccol[x];
                odo[x] = r * doss + 2 * ccol[x];
            }
            so = (uint32_t)min(tid & (BR - 1), last) * wss;
        }
#pragma unroll
        for (int x = 0; x < CH; ++x) {
            pq[x] = ld16_at(ld_q, oq[x]);
            pdo[x] = ld16_at(ld_do, odo[x]);
        }
        pl = ldf_at(ld_l, so);
        pd = ldf_at(ld_d, so);
        pi0 = ld_i0;
        ld_i0 += BR;
        if (ld_i0 >= lq) {
            ld_i0 = i_begin;
            ++ld_h;
            seek();
        } else {
            ld_q += BR * p.q.ss; ld_do += BR * p.dout.ss; ld_l += BR * ws_ss; ld_d += BR * ws_ss;
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
            const bool ok = pi0 + tid < lq;     // a row past the end has P = 0
            lse_s[buf][tid] = ok ? pl : INFINITY;
            dlt_s[buf][tid] = ok ? -pd : 0.f;       // stored negated: it seeds dP - Delta
        }
    };

    if (n_steps > 0) {
        load_tile();
        store_tile(0);
    }
    wait_all_memory();
    __syncthreads();

    // first kept row offset of this lane's key within a 32-row half, before
    // the 8q+4g part: key my_j needs row >= my_j; a key past the end keeps nothing
    const int t_key = col_ok ? (CAUSAL ? my_j - 4 * g : INT_MIN / 2) : INT_MAX / 2;

    int h = hk * G, i0 = i_begin;          // the step's tile
    for (int st = 0; st < n_steps; ++st) {
        const int buf = st & 1;
        const bool has_next = st + 1 < n_steps;
        if (has_next) load_tile();

        const uint16_t* Qb = Qs[buf];
        const uint16_t* dOb = dOs[buf];
        const bool masked = (CAUSAL && i0 < j0 + BC) || !full_cols;
        if constexpr (!DQ_ATOMIC) {
            // S^T and dP^T of both 32-row halves of the query tile first, then
            // each half's softmax gradient and dV/dK products: the matrix
            // cores work through the second half's S and dP while the vector
            // ALUs run the first half's softmax, and the first half's dV/dK
            // products while they run the second's.  With one wavefront per
            // SIMD this overlap has to come from within the wavefront.  dP^T
            // accumulates onto the rows' -Delta: pa ends as dP - Delta.
            f32x16 sa[MB], pa[MB];
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) {
                sa[mb] = zero16();
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const f32x4 nd = *reinterpret_cast<const f32x4*>(&dlt_s[buf][mb * 32 + 8 * q + 4 * g]);
#pragma unroll
                    for (int r = 0; r < 4; ++r) pa[mb][4 * q + r] = nd[r];
                }
#pragma unroll
                for (int s = 0; s < KS; ++s) {
                    sa[mb] = T::mma(ld16(&Qb[(mb * 32 + c) * QP + 16 * s + 8 * g]), kreg[s], sa[mb]);
                    pa[mb] = T::mma(ld16(&dOb[(mb * 32 + c) * QP + 16 * s + 8 * g]), vreg[s], pa[mb]);
                }
            }
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) {
                if (masked)
                    softmax_grad_tile_nd<true>(sa[mb], pa[mb], &lse_s[buf][mb * 32], p.scale_log2, g, t_key - i0 - mb * 32);
                else
                    softmax_grad_tile_nd<false>(sa[mb], pa[mb], &lse_s[buf][mb * 32], p.scale_log2, g, 0);
                if (mb == MB - 1 && has_next) store_tile(buf ^ 1);
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    const u32x4 bP = acc_to_operand<T>(sa[mb], hh);
                    const u32x4 bS = acc_to_operand<T>(pa[mb], hh);
#pragma unroll
                    for (int db = 0; db < DB; ++db) {
                        dva[db] = T::mma(ld_tr<true>(dOb, QP, mb * 32 + 16 * hh, db * 32, lane), bP, dva[db]);
                        dka[db] = T::mma(ld_tr<true>(Qb, QP, mb * 32 + 16 * hh, db * 32, lane), bS, dka[db]);
                    }
                }
            }
        } else {
            // Atomic mode, which also stages dS^T for its dQ product: one 32-row
            // half at a time (S and dP of both halves first was 6 % slower
            // here on the packed workload).
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) {
                f32x16 sa = zero16(), pa;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const f32x4 nd = *reinterpret_cast<const f32x4*>(&dlt_s[buf][mb * 32 + 8 * q + 4 * g]);
#pragma unroll
                    for (int r = 0; r < 4; ++r) pa[4 * q + r] = nd[r];
                }
#pragma unroll
                for (int s = 0; s < KS; ++s) {
                    sa = T::mma(ld16(&Qb[(mb * 32 + c) * QP + 16 * s + 8 * g]), kreg[s], sa);
                    pa = T::mma(ld16(&dOb[(mb * 32 + c) * QP + 16 * s + 8 * g]), vreg[s], pa);
                }
                if (masked)
                    softmax_grad_tile_nd<true>(sa, pa, &lse_s[buf][mb * 32], p.scale_log2, g, t_key - i0 - mb * 32);
                else
                    softmax_grad_tile_nd<false>(sa, pa, &lse_s[buf][mb * 32], p.scale_log2, g, 0);
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
        i0 += BR;
        if (i0 >= lq) { i0 = i_begin; ++h; }
    }

    if (!col_ok) return;
    const int64_t dko = b * p.dk.sb + hk * p.dk.sh + (int64_t)(k0 + my_j) * p.dk.ss;
    const int64_t dvo = b * p.dv.sb + hk * p.dv.sh + (int64_t)(k0 + my_j) * p.dv.ss;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int e = db * 32 + 8 * q + 4 * g;
            st_grad4<T>(p.dk.p, dko + e, p.grad_f32, dka[db][4 * q + 0] * p.scale, dka[db][4 * q + 1] * p.scale,
                        dka[db][4 * q + 2] * p.scale, dka[db][4 * q + 3] * p.scale);
            st_grad4<T>(p.dv.p, dvo + e, p.grad_f32, dva[db][4 * q + 0], dva[db][4 * q + 1], dva[db][4 * q + 2],
                        dva[db][4 * q + 3]);
        }
}

// ---------------------------------------------------------------------------
// dK/dV body, four wavefronts (two workgroups per CU), software-pipelined
// ---------------------------------------------------------------------------
//
// Work item: 64 keys of one KV head against every 64-row query tile of every
// query head of its group (causal: from the tile holding the diagonal on).
// Wavefront w = kw + 2*rh owns keys 32*kw .. +31 and rows 32*rh .. +31 of each
// tile; K and V of its keys stay in registers and dK^T, dV^T accumulate in
// registers across all tiles.  Step k runs the softmax gradient of tile k
// (vector ALU) next to S^T and dP^T of tile k+1 (matrix cores, independent of
// it), then dV^T += P^T dO and dK^T += dS^T Q of tile k; P^T and dS^T feed the
// B operand straight from the accumulator layout.  Q/dO tiles rotate through
// three LDS buffers: tile k (read by dV/dK), k+1 (read by S/dP), and k+2, which
// is loaded into registers at the start of the step and stored at its end with
// its rows' log2-domain LSE and negated Delta from the row pass.  The two row
// halves' dK/dV partials are summed through LDS at the end.  dQ is left to
// the query-outer body.

// Wavefronts per workgroup of the D=64 kernel and the dQ body: two row halves
// of kKeySlices key slices.  Four wavefronts let two workgroups share a CU (two
// wavefronts per SIMD), so one workgroup's memory waits and barriers overlap
// the other's arithmetic.
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kKeySlices = kWaves / 2;

template <int D>
struct Main8Lds {
    static constexpr int BR = 64, QP = D + 8, DB = D / 32, NBUF = 3;
    static constexpr int TILE_B = BR * QP * 2;            // one Q or dO tile
    static constexpr int OFF_STAT = 2 * NBUF * TILE_B;    // lse [NBUF][BR], -Delta [NBUF][BR]
    static constexpr int LOOP_B = OFF_STAT + 2 * NBUF * BR * 4;
    static constexpr int RED_B = kKeySlices * 64 * (2 * DB * 16) * 4;   // dK/dV partials of one row half
    static constexpr int BYTES = LOOP_B > RED_B ? LOOP_B : RED_B;
};

template <class T, int D, bool CAUSAL>
__device__ __forceinline__ void bwd_main8_body(const BwdParams& p, unsigned char* arena, int bx, int by) {
    using L = Main8Lds<D>;
    constexpr int BC = 32 * kKeySlices;   // keys per workgroup
    constexpr int BR = L::BR;        // query rows per step
    constexpr int KS = D / 16;       // k-steps over the head dimension (32x32x16)
    constexpr int DB = L::DB;        // 32-row blocks of dK^T / dV^T
    constexpr int QP = L::QP;        // row stride of the Q and dO tiles  [row][d]
    constexpr int TILE = BR * QP;    // elements of one tile
    constexpr int CH = BR * D / 8 / kThreads;   // 16-byte chunks per thread per tile
    static_assert(CH >= 1, "tile shape");
    uint16_t* Qs0 = reinterpret_cast<uint16_t*>(arena);
    uint16_t* dOs0 = Qs0 + L::NBUF * TILE;
    float* lse_s = reinterpret_cast<float*>(arena + L::OFF_STAT);
    float* dlt_s = lse_s + L::NBUF * BR;

    const int tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6;
    const int kw = w % kKeySlices, rh = w / kKeySlices;
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

    f32x16 dva[DB], dka[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) { dva[db] = zero16(); dka[db] = zero16(); }

    const int i_begin = CAUSAL ? (j0 / BR) * BR : 0;
    const int per_head = lq > i_begin ? (lq - i_begin + BR - 1) / BR : 0;
    const int n_steps = G * per_head;

    // byte offsets of this thread's chunks within a tile (row strides are
    // below 2^23 elements, so 128 rows fit in 32 bits)
    const uint32_t qss = 2u * (uint32_t)p.q.ss, doss = 2u * (uint32_t)p.dout.ss;
    uint32_t qoff[CH], dooff[CH];
    int crow[CH], ccol[CH];
#pragma unroll
    for (int x = 0; x < CH; ++x) {
        const int e = tid + kThreads * x;
        const int r = e / (D / 8), cc = (e % (D / 8)) * 8;
        crow[x] = r;
        ccol[x] = cc;
        qoff[x] = r * qss + 2 * cc;
        dooff[x] = r * doss + 2 * cc;
    }

    // Pointers of the tile being loaded (head ld_h, rows from ld_i0), advanced
    // by one tile per step in scalar registers.
    const uint16_t* const q_seq = p.q.p + b * p.q.sb + (int64_t)q0 * p.q.ss;
    const uint16_t* const do_seq = p.dout.p + b * p.dout.sb + (int64_t)q0 * p.dout.ss;
    // per-row log2-domain LSE and Delta from the row pass, rows (token, head)
    // when packed, (batch, head, row) when dense
    const int64_t ws_ss = p.varlen ? p.Hq : 1;
    const int64_t q_step = BR * p.q.ss, do_step = BR * p.dout.ss, st_step = BR * ws_ss;
    int ld_h = hk * G, ld_i0 = i_begin;
    const uint16_t *ld_q, *ld_do;
    const float *ld_sa, *ld_sb;
    auto seek = [&]() {
        ld_q = q_seq + ld_h * p.q.sh + (int64_t)ld_i0 * p.q.ss;
        ld_do = do_seq + ld_h * p.dout.sh + (int64_t)ld_i0 * p.dout.ss;
        const int64_t ws = p.varlen ? (int64_t)(q0 + ld_i0) * p.Hq + ld_h
                                    : ((int64_t)b * p.Hq + ld_h) * p.Sq + ld_i0;
        ld_sa = p.lse2 + ws;
        ld_sb = p.delta + ws;
    };
    // the query rows of one head from i_begin to the end of the sequence, then
    // the next head of the group
    auto advance = [&]() {
        ld_i0 += BR;
        if (ld_i0 >= lq) {
            ld_i0 = i_begin;
            ++ld_h;
            seek();
        } else {
            ld_q += q_step; ld_do += do_step; ld_sa += st_step; ld_sb += st_step;
        }
    };
    seek();

    // Tile loads are unconditional: rows past the end of the sequence re-read
    // its last row and get LSE = +inf when stored, so their P is exactly zero.
    // Nothing loaded is used before the tile is stored.
    struct TileRegs { u32x4 q[CH], d[CH]; float sa, sb; };
    const int srow = tid & (BR - 1);
    const uint32_t sss = 4u * (uint32_t)ws_ss;
    const uint32_t srow_off = srow * sss;
    auto load_tile = [&](TileRegs& t) {
        uint32_t oq[CH], odo[CH], so = srow_off;
        if (ld_i0 + BR <= lq) {
#pragma unroll
            for (int x = 0; x < CH; ++x) { oq[x] = qoff[x]; odo[x] = dooff[x]; }
        } else {
            const int last = lq - 1 - ld_i0;
#pragma unroll
            for (int x = 0; x < CH; ++x) {
                const uint32_t r = min(crow[x], last);
                oq[x] = r * qss + 2 * ccol[x];
                odo[x] = r * doss + 2 * ccol[x];
            }
            so = (uint32_t)min(srow, last) * sss;
        }
#pragma unroll
        for (int x = 0; x < CH; ++x) {
            t.q[x] = ld16_at(ld_q, oq[x]);
            t.d[x] = ld16_at(ld_do, odo[x]);
        }
        t.sa = ldf_at(ld_sa, so);
        t.sb = ldf_at(ld_sb, so);
    };
    auto store_tile = [&](const TileRegs& t, int buf, int i0) {
        uint16_t* Qd = Qs0 + buf * TILE;
        uint16_t* dOd = dOs0 + buf * TILE;
#pragma unroll
        for (int x = 0; x < CH; ++x) {
            st16(&Qd[crow[x] * QP + ccol[x]], t.q[x]);
            st16(&dOd[crow[x] * QP + ccol[x]], t.d[x]);
        }
        if (tid < BR) {
            const bool ok = i0 + tid < lq;      // a row past the end has P = 0
            lse_s[buf * BR + tid] = ok ? t.sa : INFINITY;
            dlt_s[buf * BR + tid] = ok ? -t.sb : 0.f;   // stored negated: it seeds dP - Delta
        }
    };
    u32x4 kreg[KS], vreg[KS];            // this wavefront's keys, loaded in the prologue
    // S^T and dP^T - Delta of the tile in buffer buf; dP^T accumulates onto
    // the rows' -Delta
    auto s_dp = [&](int buf, f32x16& sa, f32x16& pa) {
        const uint16_t* Qb = Qs0 + buf * TILE;
        const uint16_t* dOb = dOs0 + buf * TILE;
        sa = zero16();
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const f32x4 nd = *reinterpret_cast<const f32x4*>(&dlt_s[buf * BR + 32 * rh + 8 * q + 4 * g]);
#pragma unroll
            for (int r = 0; r < 4; ++r) pa[4 * q + r] = nd[r];
        }
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            sa = T::mma(ld16(&Qb[(32 * rh + c) * QP + 16 * s + 8 * g]), kreg[s], sa);
            pa = T::mma(ld16(&dOb[(32 * rh + c) * QP + 16 * s + 8 * g]), vreg[s], pa);
        }
    };

    // Prologue: the first two tiles and this wavefront's K and V rows are all
    // requested before anything waits for memory.
    int i0_k = i_begin, i0_k1 = i_begin;   // first rows of tiles k and k+1
    TileRegs tr0, tr1;
    if (n_steps > 0) { load_tile(tr0); i0_k = ld_i0; advance(); }
    if (n_steps > 1) { load_tile(tr1); i0_k1 = ld_i0; advance(); }
    {
        const int jr = min(my_j, lk - 1);   // keys past the end are masked and not stored
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            kreg[s] = ld16(kbase + (int64_t)jr * p.k.ss + 16 * s + 8 * g);
            vreg[s] = ld16(vbase + (int64_t)jr * p.v.ss + 16 * s + 8 * g);
        }
    }
    if (n_steps > 0) store_tile(tr0, 0, i0_k);
    if (n_steps > 1) store_tile(tr1, 1, i0_k1);
    wait_all_memory();
    __syncthreads();

    // this lane's first kept row offset within its 32-row half, before the
    // 8q+4g part: key my_j needs row >= my_j; a key past the end keeps nothing
    const int t_key = col_ok ? (CAUSAL ? my_j - 32 * rh - 4 * g : INT_MIN / 2) : INT_MAX / 2;

    f32x16 sa, pa;
    if (n_steps > 0) s_dp(0, sa, pa);
    int bk = 0, bk1 = 1, bk2 = 2;          // buffers of tiles k, k+1, k+2
    for (int k = 0; k < n_steps; ++k) {
        const bool has2 = k + 2 < n_steps;
        int i0_k2 = i0_k1;
        TileRegs trn;
        if (has2) { load_tile(trn); i0_k2 = ld_i0; advance(); }

        // softmax gradient of tile k next to S^T/dP^T of tile k+1 (on the last
        // step the latter reads a stale buffer and is discarded)
        const bool masked = (CAUSAL && i0_k < j0 + BC) || !full_cols;
        u32x4 bP[2], bS[2];
        if (masked) {
            softmax_grad_tile_nd<true>(sa, pa, &lse_s[bk * BR + 32 * rh], p.scale_log2, g, t_key - i0_k);
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) { bP[hh] = acc_to_operand<T>(sa, hh); bS[hh] = acc_to_operand<T>(pa, hh); }
            s_dp(bk1, sa, pa);
        } else {
            softmax_grad_tile_nd<false>(sa, pa, &lse_s[bk * BR + 32 * rh], p.scale_log2, g, 0);
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) { bP[hh] = acc_to_operand<T>(sa, hh); bS[hh] = acc_to_operand<T>(pa, hh); }
            s_dp(bk1, sa, pa);
        }

        // dV^T += P^T dO, dK^T += dS^T Q of tile k
        const uint16_t* Qb = Qs0 + bk * TILE;
        const uint16_t* dOb = dOs0 + bk * TILE;
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                dva[db] = T::mma(ld_tr<true>(dOb, QP, 32 * rh + 16 * hh, db * 32, lane), bP[hh], dva[db]);
                dka[db] = T::mma(ld_tr<true>(Qb, QP, 32 * rh + 16 * hh, db * 32, lane), bS[hh], dka[db]);
            }
        __builtin_amdgcn_s_setprio(0);
        if (has2) store_tile(trn, bk2, i0_k2);
        __syncthreads();
        const int t = bk; bk = bk1; bk1 = bk2; bk2 = t;
        i0_k = i0_k1;
        i0_k1 = i0_k2;
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
    const int64_t dko = b * p.dk.sb + hk * p.dk.sh + (int64_t)(k0 + my_j) * p.dk.ss;
    const int64_t dvo = b * p.dv.sb + hk * p.dv.sh + (int64_t)(k0 + my_j) * p.dv.ss;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int e = db * 32 + 8 * q + 4 * g;
            st_grad4<T>(p.dk.p, dko + e, p.grad_f32, dka[db][4 * q + 0] * p.scale, dka[db][4 * q + 1] * p.scale,
                        dka[db][4 * q + 2] * p.scale, dka[db][4 * q + 3] * p.scale);
            st_grad4<T>(p.dv.p, dvo + e, p.grad_f32, dva[db][4 * q + 0], dva[db][4 * q + 1], dva[db][4 * q + 2],
                        dva[db][4 * q + 3]);
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
    const f32x4* src = reinterpret_cast<const f32x4*>(p.dqacc + acc_row(p, L, R) * D + part * 8);
    const f32x4 a = src[0], c = src[1];
    const float x[8] = {a[0] * p.scale, a[1] * p.scale, a[2] * p.scale, a[3] * p.scale,
                        c[0] * p.scale, c[1] * p.scale, c[2] * p.scale, c[3] * p.scale};
    st_grad8<T>(p.dq.p, toff(p.dq, L) + part * 8, p.grad_f32, x);
}

// ---------------------------------------------------------------------------
// dQ pass without atomics, four wavefronts (query-tile outer)
// ---------------------------------------------------------------------------
//
// One workgroup per (sequence, query head, 64-row query tile); it walks the
// 64-key tiles the tile can see.  Wavefront w = kw + 2*rh owns query rows
// 32*rh .. +31 and keys 32*kw .. +31 of every key tile.  Scores are computed
// transposed, S^T = K Q^T and dP^T = V dO^T, so that each lane holds one query
// column: its LSE and Delta are lane-uniform, and dS^T feeds
// dQ^T += K^T dS^T directly as the B operand.  Q and dO stay in registers for
// the whole kernel; key tiles stream through a double-buffered LDS copy whose
// next tile is loaded into registers while the current one is used.  Each
// wavefront accumulates dQ^T over its key slice; the two slices' partials are
// summed through LDS at the end and dQ is written once, scaled and rounded.

template <int D>
struct Dq8Lds {
    static constexpr int BK = 32 * kKeySlices, KP = D + 8, DB = D / 32;
    static constexpr int TILE_B = BK * KP * 2;
    static constexpr int LOOP_B = 4 * TILE_B;
    static constexpr int RED_B = (kKeySlices - 1) * 2 * 64 * (DB * 16) * 4;
    static constexpr int BYTES = LOOP_B > RED_B ? LOOP_B : RED_B;
};

template <class T, int D, bool CAUSAL>
__device__ __forceinline__ void bwd_dq8_body(const BwdParams& p, unsigned char* arena, int bx, int by) {
    constexpr int BQ = 64;           // query rows per workgroup
    constexpr int BK = 32 * kKeySlices;   // keys per step
    constexpr int KS = D / 16;       // k-steps over the head dimension (32x32x16)
    constexpr int DB = D / 32;       // 32-row blocks of dQ^T
    constexpr int KP = D + 8;        // row stride of Ks, Vs  [key][d]
    constexpr int CH = BK * D / 8 / kThreads;   // 16-byte chunks per thread per key tile
    constexpr int TILE_B = BK * KP * 2;
    constexpr int OFF_K = 0, OFF_V = 2 * TILE_B;
    constexpr int LOOP_B = 4 * TILE_B;
    constexpr int RED_B = (kKeySlices - 1) * 2 * 64 * (DB * 16) * 4;   // key slices 1.. of both row halves
    static_assert(Dq8Lds<D>::BYTES == (LOOP_B > RED_B ? LOOP_B : RED_B), "arena size");
    uint16_t* Ks0 = reinterpret_cast<uint16_t*>(arena + OFF_K);
    uint16_t* Vs0 = reinterpret_cast<uint16_t*>(arena + OFF_V);

    const int tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6;
    const int kw = w % kKeySlices, rh = w / kKeySlices;
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

    const int kend = CAUSAL ? min(lk, i0 + BQ) : lk;
    const int n_steps = (kend + BK - 1) / BK;

    // byte offsets of this thread's chunks within a key tile
    const uint32_t kss = 2u * (uint32_t)p.k.ss, vss = 2u * (uint32_t)p.v.ss;
    uint32_t koff[CH], voff[CH];
    int crow[CH], ccol[CH];
#pragma unroll
    for (int x = 0; x < CH; ++x) {
        const int e = tid + kThreads * x;
        const int r = e / (D / 8), cc = (e % (D / 8)) * 8;
        crow[x] = r;
        ccol[x] = cc;
        koff[x] = r * kss + 2 * cc;
        voff[x] = r * vss + 2 * cc;
    }
    // Unconditional loads: keys past the end of the sequence re-read its last
    // key and are masked out (P = 0), so nothing is waited for before the tile
    // is stored after the step's products.
    u32x4 pk[CH], pv[CH];
    const uint16_t* kb = kbase;          // key tile being loaded, advanced per step
    const uint16_t* vb = vbase;
    const int64_t k_step = BK * p.k.ss, v_step = BK * p.v.ss;
    auto load_tile = [&](int st) {
        const int j0 = st * BK;
        uint32_t ok_[CH], ov_[CH];
        if (j0 + BK <= lk) {
#pragma unroll
            for (int x = 0; x < CH; ++x) { ok_[x] = koff[x]; ov_[x] = voff[x]; }
        } else {
            const int last = lk - 1 - j0;
#pragma unroll
            for (int x = 0; x < CH; ++x) {
                const uint32_t r = min(crow[x], last);
                ok_[x] = r * kss + 2 * ccol[x];
                ov_[x] = r * vss + 2 * ccol[x];
            }
        }
#pragma unroll
        for (int x = 0; x < CH; ++x) {
            pk[x] = ld16_at(kb, ok_[x]);
            pv[x] = ld16_at(vb, ov_[x]);
        }
        kb += k_step;
        vb += v_step;
    };
    auto store_tile = [&](int buf) {
        uint16_t* Kd = Ks0 + buf * (BK * KP);
        uint16_t* Vd = Vs0 + buf * (BK * KP);
#pragma unroll
        for (int x = 0; x < CH; ++x) {
            st16(&Kd[crow[x] * KP + ccol[x]], pk[x]);
            st16(&Vd[crow[x] * KP + ccol[x]], pv[x]);
        }
    };

    // Prologue: the first key tile and this lane's query row are requested
    // before anything waits for memory.
    if (n_steps > 0) load_tile(0);
    const int my_i = i0 + 32 * rh + c;
    const bool row_ok = my_i < lq;
    // a row past the end of the sequence re-reads its last row; its LSE is
    // +inf (P = 0) and its dQ is not stored
    const int my_ic = min(my_i, lq - 1);
    u32x4 qreg[KS], doreg[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) {
        qreg[s] = ld16(qbase + (int64_t)my_ic * p.q.ss + 16 * s + 8 * g);
        doreg[s] = ld16(dobase + (int64_t)my_ic * p.dout.ss + 16 * s + 8 * g);
    }
    // this row's log2-domain LSE and Delta from the row pass
    const int64_t ws = p.varlen ? (int64_t)(q0 + my_ic) * p.Hq + h : ((int64_t)b * p.Hq + h) * p.Sq + my_ic;
    const float l2 = row_ok ? p.lse2[ws] : INFINITY;
    const float dl = p.delta[ws];

    f32x16 dq[DB], ndl16;
#pragma unroll
    for (int db = 0; db < DB; ++db) dq[db] = zero16();
#pragma unroll
    for (int r = 0; r < 16; ++r) ndl16[r] = -dl;

    if (n_steps > 0) store_tile(0);
    wait_all_memory();
    __syncthreads();

    // last key this lane's row keeps, relative to the 8q+4g part of a tile row
    const int t_row = min(lk - 1, CAUSAL ? my_i : INT_MAX) - 32 * kw - 4 * g;

    for (int st = 0; st < n_steps; ++st) {
        const int buf = st & 1;
        const int j0 = st * BK;
        const bool has_next = st + 1 < n_steps;
        if (has_next) load_tile(st + 1);
        const uint16_t* Kb = Ks0 + buf * (BK * KP);
        const uint16_t* Vb = Vs0 + buf * (BK * KP);

        f32x16 s = zero16(), dp = ndl16;   // dP^T accumulates onto -Delta
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            s = T::mma(ld16(&Kb[(32 * kw + c) * KP + 16 * ks + 8 * g]), qreg[ks], s);
            dp = T::mma(ld16(&Vb[(32 * kw + c) * KP + 16 * ks + 8 * g]), doreg[ks], dp);
        }
        // element (rg): key j = j0 + 32kw + 8(rg/4) + 4g + rg%4, query my_i
        const bool masked = (CAUSAL && j0 + BK > i0) || (j0 + BK > lk);
        if (masked) {
            const int t = t_row - j0;
#pragma unroll
            for (int rg = 0; rg < 16; ++rg) {
                float pvv = fast_exp2(__builtin_fmaf(s[rg], p.scale_log2, -l2));
                pvv = (8 * (rg >> 2) + (rg & 3) <= t) ? pvv : 0.f;
                dp[rg] = pvv * dp[rg];
            }
        } else {
#pragma unroll
            for (int rg = 0; rg < 16; ++rg) {
                const float pvv = fast_exp2(__builtin_fmaf(s[rg], p.scale_log2, -l2));
                dp[rg] = pvv * dp[rg];
            }
        }
        if (has_next) store_tile(buf ^ 1);
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            const u32x4 bS = acc_to_operand<T>(dp, hh);
#pragma unroll
            for (int db = 0; db < DB; ++db)
                dq[db] = T::mma(ld_tr<true>(Kb, KP, 32 * kw + 16 * hh, db * 32, lane), bS, dq[db]);
        }
        __builtin_amdgcn_s_setprio(0);
        __syncthreads();
    }

    // sum the key slices through LDS (slices 1..3 write, slice 0 adds)
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
    for (int sl = 0; sl < kKeySlices - 1; ++sl)
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const f32x4 x = *reinterpret_cast<const f32x4*>(&red[((((sl * 2 + rh) * DB + db) * 4 + r4) * 64 + lane) * 4]);
                dq[db][4 * r4 + 0] += x[0]; dq[db][4 * r4 + 1] += x[1];
                dq[db][4 * r4 + 2] += x[2]; dq[db][4 * r4 + 3] += x[3];
            }
    const int64_t dqo = b * p.dq.sb + h * p.dq.sh + (int64_t)(q0 + my_i) * p.dq.ss;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int q = 0; q < 4; ++q)
            st_grad4<T>(p.dq.p, dqo + db * 32 + 8 * q + 4 * g, p.grad_f32, dq[db][4 * q + 0] * p.scale,
                        dq[db][4 * q + 1] * p.scale, dq[db][4 * q + 2] * p.scale, dq[db][4 * q + 3] * p.scale);
}

// ---------------------------------------------------------------------------
// Wide query-tile body of the D=64 kernel: dQ of 128 query rows
// ---------------------------------------------------------------------------
//
// Wavefront w owns rows 32w .. +31 of the tile against all 64 keys of each
// step, so there are no key-slice partials to sum at the end: per step, S^T
// and dP^T of the two 32-key halves (v_mfma_f32_32x32x16; dP^T accumulates
// onto -Delta), P and dS, then dQ^T += K^T dS^T.  K and V tiles are double
// buffered in LDS and the next one is loaded into registers during the step.
// With twice the rows of the 64-row body an item covers twice the work, so
// the per-item costs (first loads, dispatch, epilogue) are paid half as
// often.  On a causal diagonal, a wavefront whose rows all precede the step's
// keys skips the step's products (its P is zero there).

template <int D>
struct DqwLds {
    static constexpr int BK = 64, KP = D + 8;
    static constexpr int TILE_B = BK * KP * 2;
    static constexpr int BYTES = 4 * TILE_B;   // K and V, two buffers each
};

template <class T, int D, bool CAUSAL>
__device__ __forceinline__ void bwd_dqw_body(const BwdParams& p, unsigned char* arena, int bx, int by) {
    static_assert(D == 64, "wide dQ body: D=64");
    constexpr int BQ = 128;                 // query rows per workgroup
    constexpr int BK = DqwLds<D>::BK;       // keys per step
    constexpr int KS = D / 16;              // k-steps over the head dimension (32x32x16)
    constexpr int DB = D / 32;              // 32-row blocks of dQ^T
    constexpr int KP = DqwLds<D>::KP;       // row stride of the K and V tiles  [key][d]
    constexpr int TILE = BK * KP;           // elements of one tile
    constexpr int CH = BK * D / 8 / kThreads;   // 16-byte chunks per thread per tile
    uint16_t* Ks0 = reinterpret_cast<uint16_t*>(arena);
    uint16_t* Vs0 = Ks0 + 2 * TILE;

    const int tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6;
    const int g = lane >> 5, c = lane & 31;
    const int b = by / p.Hq, h = by % p.Hq;
    const int hk = h / (p.Hq / p.Hkv);
    int q0 = 0, k0 = 0, lq = p.Sq, lk = p.Sk;
    if (p.varlen) seq_get(p.seqs, b, q0, k0, lq, lk);
    const int i0 = bx * BQ;
    if (i0 >= lq) return;

    const uint16_t* qbase = p.q.p + b * p.q.sb + h * p.q.sh + (int64_t)q0 * p.q.ss;
    const uint16_t* dobase = p.dout.p + b * p.dout.sb + h * p.dout.sh + (int64_t)q0 * p.dout.ss;
    const uint16_t* kb = p.k.p + b * p.k.sb + hk * p.k.sh + (int64_t)k0 * p.k.ss;   // tile being loaded
    const uint16_t* vb = p.v.p + b * p.v.sb + hk * p.v.sh + (int64_t)k0 * p.v.ss;
    const int64_t k_step = BK * p.k.ss, v_step = BK * p.v.ss;

    const int kend = CAUSAL ? min(lk, i0 + BQ) : lk;
    const int n_steps = (kend + BK - 1) / BK;

    // byte offsets of this thread's chunks within a key tile
    const uint32_t kss = 2u * (uint32_t)p.k.ss, vss = 2u * (uint32_t)p.v.ss;
    uint32_t koff[CH], voff[CH];
    int crow[CH], ccol[CH];
#pragma unroll
    for (int x = 0; x < CH; ++x) {
        const int e = tid + kThreads * x;
        const int r = e / (D / 8), cc = (e % (D / 8)) * 8;
        crow[x] = r;
        ccol[x] = cc;
        koff[x] = r * kss + 2 * cc;
        voff[x] = r * vss + 2 * cc;
    }
    // Unconditional loads: keys past the end of the sequence re-read its last
    // key and are masked out (P = 0); nothing loaded is used before the tile
    // is stored after the step's products.
    u32x4 pk[CH], pv[CH];
    auto load_tile = [&](int st) {
        const int j0 = st * BK;
        uint32_t ok_[CH], ov_[CH];
        if (j0 + BK <= lk) {
#pragma unroll
            for (int x = 0; x < CH; ++x) { ok_[x] = koff[x]; ov_[x] = voff[x]; }
        } else {
            const int last = lk - 1 - j0;
#pragma unroll
            for (int x = 0; x < CH; ++x) {
                const uint32_t r = min(crow[x], last);
                ok_[x] = r * kss + 2 * ccol[x];
                ov_[x] = r * vss + 2 * ccol[x];
            }
        }
#pragma unroll
        for (int x = 0; x < CH; ++x) {
            pk[x] = ld16_at(kb, ok_[x]);
            pv[x] = ld16_at(vb, ov_[x]);
        }
        kb += k_step;
        vb += v_step;
    };
    auto store_tile = [&](int buf) {
        uint16_t* Kd = Ks0 + buf * TILE;
        uint16_t* Vd = Vs0 + buf * TILE;
#pragma unroll
        for (int x = 0; x < CH; ++x) {
            st16(&Kd[crow[x] * KP + ccol[x]], pk[x]);
            st16(&Vd[crow[x] * KP + ccol[x]], pv[x]);
        }
    };

    // Prologue: the first key tile and this lane's query row are requested
    // before anything waits for memory.
    if (n_steps > 0) load_tile(0);
    const int my_i = i0 + 32 * w + c;
    const bool row_ok = my_i < lq;
    // a row past the end of the sequence re-reads its last row; its LSE is
    // +inf (P = 0) and its dQ is not stored
    const int my_ic = min(my_i, lq - 1);
    u32x4 qreg[KS], doreg[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) {
        qreg[s] = ld16(qbase + (int64_t)my_ic * p.q.ss + 16 * s + 8 * g);
        doreg[s] = ld16(dobase + (int64_t)my_ic * p.dout.ss + 16 * s + 8 * g);
    }
    // this row's log2-domain LSE and Delta from the row pass
    const int64_t ws = p.varlen ? (int64_t)(q0 + my_ic) * p.Hq + h : ((int64_t)b * p.Hq + h) * p.Sq + my_ic;
    const float l2 = row_ok ? p.lse2[ws] : INFINITY;
    const float dl = p.delta[ws];

    f32x16 dq[DB], ndl16;
#pragma unroll
    for (int db = 0; db < DB; ++db) dq[db] = zero16();
#pragma unroll
    for (int r = 0; r < 16; ++r) ndl16[r] = -dl;

    if (n_steps > 0) store_tile(0);
    wait_all_memory();
    __syncthreads();

    // last key this lane's row keeps, relative to the 8q+4g part of a tile row
    const int t_row = min(lk - 1, CAUSAL ? my_i : INT_MAX) - 4 * g;
    const int w_row0 = i0 + 32 * w;   // the wavefront's first row

    for (int st = 0; st < n_steps; ++st) {
        const int buf = st & 1;
        const int j0 = st * BK;
        const bool has_next = st + 1 < n_steps;
        if (has_next) load_tile(st + 1);
        const uint16_t* Kb = Ks0 + buf * TILE;
        const uint16_t* Vb = Vs0 + buf * TILE;
        // every key of the step after every row of this wavefront: P = 0
        const bool dead = CAUSAL && j0 > w_row0 + 31;

        f32x16 ds[2];
        if (!dead) {
#pragma unroll
            for (int kh = 0; kh < 2; ++kh) {
                f32x16 s = zero16(), dp = ndl16;   // dP^T accumulates onto -Delta
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    s = T::mma(ld16(&Kb[(32 * kh + c) * KP + 16 * ks + 8 * g]), qreg[ks], s);
                    dp = T::mma(ld16(&Vb[(32 * kh + c) * KP + 16 * ks + 8 * g]), doreg[ks], dp);
                }
                // element rg: key j0 + 32kh + 8(rg/4) + 4g + rg%4, query my_i
                const int jh = j0 + 32 * kh;
                const bool masked = (CAUSAL && jh + 31 > w_row0) || (jh + 32 > lk);
                if (masked) {
                    const int t = t_row - jh;
#pragma unroll
                    for (int rg = 0; rg < 16; ++rg) {
                        float pvv = fast_exp2(__builtin_fmaf(s[rg], p.scale_log2, -l2));
                        pvv = (8 * (rg >> 2) + (rg & 3) <= t) ? pvv : 0.f;
                        dp[rg] = pvv * dp[rg];
                    }
                } else {
#pragma unroll
                    for (int rg = 0; rg < 16; ++rg)
                        dp[rg] = fast_exp2(__builtin_fmaf(s[rg], p.scale_log2, -l2)) * dp[rg];
                }
                ds[kh] = dp;
            }
        }
        if (has_next) store_tile(buf ^ 1);
        if (!dead) {
            __builtin_amdgcn_s_setprio(1);
#pragma unroll
            for (int kh = 0; kh < 2; ++kh)
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    const u32x4 bS = acc_to_operand<T>(ds[kh], hh);
#pragma unroll
                    for (int db = 0; db < DB; ++db)
                        dq[db] = T::mma(ld_tr<true>(Kb, KP, 32 * kh + 16 * hh, db * 32, lane), bS, dq[db]);
                }
            __builtin_amdgcn_s_setprio(0);
        }
        __syncthreads();
    }

    if (!row_ok) return;
    const int64_t dqo = b * p.dq.sb + h * p.dq.sh + (int64_t)(q0 + my_i) * p.dq.ss;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int q = 0; q < 4; ++q)
            st_grad4<T>(p.dq.p, dqo + db * 32 + 8 * q + 4 * g, p.grad_f32, dq[db][4 * q + 0] * p.scale,
                        dq[db][4 * q + 1] * p.scale, dq[db][4 * q + 2] * p.scale, dq[db][4 * q + 3] * p.scale);
}

template <class T, int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 2) void bwd_dq8_kernel(BwdParams p) {
    __shared__ __align__(16) unsigned char arena[Dq8Lds<D>::BYTES];
    // units: (sequence, query head), sharing K and V; items: query tiles,
    // the longest causal range (the last tile) first.  With the plain grid
    // each XCD took every eighth query tile of every head and so read every
    // head's K and V; per-unit order took the S=4096, D=128 dQ pass from 325
    // to 236 us.
    int unit, item;
    xcd_unit_order(gridDim.y, gridDim.x, blockIdx.y * gridDim.x + blockIdx.x, unit, item);
    bwd_dq8_body<T, D, CAUSAL>(p, arena, gridDim.x - 1 - item, unit);
}

// dK/dV and dQ in one launch: key-tile items (the key-tile outer body, dK and
// dV of 64 keys) and query-tile items, dQ of 64 rows or, causal with more
// items than the GPU has workgroup slots, of 128 rows with the wide body
// (half the items, so half the per-item costs; with fewer items the time is
// the longest item's, and non-causal the wide step's lower efficiency is not
// paid back: measured).  Item order, longest first so the dQ items fill the
// CUs that the long dK/dV items leave idle near the end: causal with one
// query head per KV head and equal lengths, key tile k has n_k - k steps and
// query tile m has m + 1 (64 rows) or 2m + 2 (128 rows), so segments of two
// items (key tile k, query tile n_q - 1 - k) or of three (key tiles 2j and
// 2j + 1 around query tile n_q - 1 - j), each over every (sequence, head), go
// out in decreasing length; otherwise the key tiles, then the query tiles in
// descending order.
// The two forms are separate instantiations (WIDE): one kernel holding both
// query-tile bodies spilled registers.
struct Fused8Map {
    int main_x, main_y, dq_x, dq_y;
    int alternate;   // the two- or three-item segment order
};

template <class T, int D, bool CAUSAL, bool WIDE>
__device__ __forceinline__ void fused8_dq(const BwdParams& p, unsigned char* arena, int bx, int by) {
    if constexpr (WIDE) bwd_dqw_body<T, D, CAUSAL>(p, arena, bx, by);
    else bwd_dq8_body<T, D, CAUSAL>(p, arena, bx, by);
}

template <class T, int D, bool CAUSAL, bool WIDE>
__global__ __launch_bounds__(kThreads, 2) void bwd_fused8_kernel(BwdParams p, Fused8Map m) {
    constexpr int A = Main8Lds<D>::BYTES > (WIDE ? DqwLds<D>::BYTES : Dq8Lds<D>::BYTES)
                          ? Main8Lds<D>::BYTES : (WIDE ? DqwLds<D>::BYTES : Dq8Lds<D>::BYTES);
    __shared__ __align__(16) unsigned char arena[A];
    const int id = blockIdx.x;
    constexpr bool wide = WIDE;
    if (m.alternate) {
        // main_x == dq_y; main_y == dq_x (64-row items) or 2 * dq_x (wide)
        const int seg = id / m.main_x, within = id % m.main_x;
        if constexpr (wide) {
            const int j = seg / 3, r = seg % 3;
            if (r == 1) bwd_dqw_body<T, D, CAUSAL>(p, arena, m.dq_x - 1 - j, within);
            else bwd_main8_body<T, D, CAUSAL>(p, arena, within, 2 * j + (r >> 1));
        } else {
            if (!(seg & 1)) bwd_main8_body<T, D, CAUSAL>(p, arena, within, seg >> 1);
            else bwd_dq8_body<T, D, CAUSAL>(p, arena, m.dq_x - 1 - (seg >> 1), within);
        }
        return;
    }
    const int n_main = m.main_x * m.main_y;
    if (id < n_main) {
        bwd_main8_body<T, D, CAUSAL>(p, arena, id % m.main_x, id / m.main_x);
    } else {
        const int r = id - n_main;
        fused8_dq<T, D, CAUSAL, WIDE>(p, arena, m.dq_x - 1 - r / m.dq_y, r % m.dq_y);
    }
}

// Workgroup slots of the D=64 fused kernel on the current device: two per
// compute unit (0 if the count is unknown).
static int fused8_slots() {
    constexpr int kMaxDev = 64;
    static int cached[kMaxDev] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev) return 0;
    if (cached[dev] == 0) {
        int cu = 0;
        if (hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cu <= 0) return 0;
        cached[dev] = 2 * cu;
    }
    return cached[dev];
}

// ---------------------------------------------------------------------------
// Launch
// ---------------------------------------------------------------------------

template <class T, int D, bool CAUSAL>
static hipError_t launch_bwd_t(const BwdParams& p, const BwdLaunch& L, hipStream_t st) {
    if constexpr (D == 64) {
        // The row pass, then one launch of both bodies; dQ is computed without
        // atomics, so the result is deterministic whatever the caller asked for.
        if (L.phase & BwdLaunch::kFirst) launch_pre<T, D>(p, 0, st);
        const int mx = L.n_seq * p.Hkv, my = L.max_kv_tiles64;
        static_assert(32 * kKeySlices == 64, "key tile of the fused kernel");
        const int qy = L.n_seq * p.Hq;
        // 128-row dQ items, causal, when the 64-row form has more items than slots
        const int slots = fused8_slots();
        const long n64 = (long)mx * my + (long)L.max_q_tiles64 * qy;
        const bool wide = CAUSAL && slots > 0 && n64 > slots;
        Fused8Map m{mx, my, wide ? L.max_q_tiles128 : L.max_q_tiles64, qy, 0};
        const int n = mx * my + m.dq_x * qy;
        if (n > 0) {
            m.alternate = (CAUSAL && mx == qy && my == (wide ? 2 : 1) * m.dq_x) ? 1 : 0;
            if (wide)
                PROF_LAUNCH(KID_BWD_FUSED, st, (bwd_fused8_kernel<T, D, CAUSAL, true>), dim3(n), dim3(kThreads), 0, st, p, m);
            else
                PROF_LAUNCH(KID_BWD_FUSED, st, (bwd_fused8_kernel<T, D, CAUSAL, false>), dim3(n), dim3(kThreads), 0, st, p, m);
        }
        return hipGetLastError();
    } else {
        const int64_t row_threads = p.rows * (D / 8);
        const dim3 row_grid((unsigned)((row_threads + 255) / 256));   // dQ conversion: 8 elements per thread
        const bool have_rows = p.rows > 0;
        if ((L.phase & BwdLaunch::kFirst) && have_rows) launch_pre<T, D>(p, L.deterministic ? 0 : 1, st);
        const dim3 main_grid(L.n_seq * p.Hkv, L.max_kv_tiles);
        const bool have_main = main_grid.x > 0 && main_grid.y > 0;
        if (L.deterministic) {
            if (have_main)
                PROF_LAUNCH(KID_BWD_MAIN, st, (bwd_main_kernel<T, D, CAUSAL, false>), main_grid, dim3(256), 0, st, p);
            const dim3 dq_grid(L.max_q_tiles64, L.n_seq * p.Hq);
            if (dq_grid.x > 0 && dq_grid.y > 0)
                PROF_LAUNCH(KID_BWD_DQ_DET, st, (bwd_dq8_kernel<T, D, CAUSAL>), dq_grid, dim3(kThreads), 0, st, p);
        } else {
            if (have_main)
                PROF_LAUNCH(KID_BWD_MAIN, st, (bwd_main_kernel<T, D, CAUSAL, true>), main_grid, dim3(256), 0, st, p);
            if ((L.phase & BwdLaunch::kLast) && have_rows)
                PROF_LAUNCH(KID_BWD_DQ_CONVERT, st, (bwd_dq_convert_kernel<T, D>), row_grid, dim3(256), 0, st, p);
        }
        return hipGetLastError();
    }
}

template <class T, int D>
static hipError_t launch_bwd_d(const BwdParams& p, const BwdLaunch& L, hipStream_t st) {
    return L.causal ? launch_bwd_t<T, D, true>(p, L, st) : launch_bwd_t<T, D, false>(p, L, st);
}

template <class T, int D>
static hipError_t launch_pre_t(const BwdParams& p, bool zero_dq, hipStream_t st) {
    launch_pre<T, D>(p, zero_dq ? 1 : 0, st);
    return hipGetLastError();
}

hipError_t launch_bwd_pre(const BwdParams& p, int dtype, int D, bool zero_dq, hipStream_t st) {
    if (dtype == 0) {
        if (D == 192) return launch_pre_t<F16, 192>(p, zero_dq, st);
        return D == 64 ? launch_pre_t<F16, 64>(p, zero_dq, st) : launch_pre_t<F16, 128>(p, zero_dq, st);
    }
    if (D == 192) return launch_pre_t<BF16, 192>(p, zero_dq, st);
    return D == 64 ? launch_pre_t<BF16, 64>(p, zero_dq, st) : launch_pre_t<BF16, 128>(p, zero_dq, st);
}

hipError_t launch_bwd(const BwdParams& p, const BwdLaunch& L, hipStream_t st) {
    if (L.dtype == 0)
        return L.D == 64 ? launch_bwd_d<F16, 64>(p, L, st) : launch_bwd_d<F16, 128>(p, L, st);
    return L.D == 64 ? launch_bwd_d<BF16, 64>(p, L, st) : launch_bwd_d<BF16, 128>(p, L, st);
}

}  // namespace sdpa
