// The key-tile backward kernel and the atomic-free dQ pass for D = 128 and
// D = 192 (and the key-tile kernel at D = 64 in the atomic dQ mode), as
// templates: bwd128.hip instantiates D = 64 and 128, bwd192.hip D = 192, each
// in a translation unit of its own so that each takes its own
// machine-scheduler strategy.
//
// Kernels (all on the caller's stream; the row pass is bwd.hip's):
//   bwd_main_kernel    one four-wavefront workgroup per (sequence, KV head,
//                      128-key tile); D=128 in every dQ mode, D=192 in the
//                      atomic-free modes, D=64 in the atomic mode; dK and dV accumulate in registers
//                      across every query tile of every query head of the
//                      group; per 64-row query tile S, dP, dV, dK and, in
//                      atomic mode, dQ += dS K through fp32 atomics.     [MFMA]
//   bwd_dq_convert     atomic mode: dQ = scale * accumulator, rounded.
//   bwd_dq8_kernel     atomic-free modes: the query-tile outer dQ body as its
//                      own launch.                                       [MFMA]
#pragma once

#include "bwd_shared.h"
#include "common.h"
#include "kernels.h"
#include "prof.h"

namespace sdpa {

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

// DK: head dim of Q and K; DV: of V, O and dO (equal unless (192, 128)).
template <class T, int DK, int DV, bool CAUSAL, bool DQ_ATOMIC>
__global__ __launch_bounds__(256, (DK == 64 ? 2 : 1)) void bwd_main_kernel(BwdParams p) {
    static_assert(!DQ_ATOMIC || DK == DV, "the atomic dQ form takes equal head dims");
    constexpr int D = DK;            // the atomic form's head dim
    constexpr int BC = 128;          // keys per workgroup: 4 wavefronts x 32
    constexpr int BR = 64;           // query rows per step
    constexpr int NW = 4;
    constexpr int KSK = DK / 16, KSV = DV / 16;   // k-steps of S (over DK) and dP (over DV)
    constexpr int KSM = KSK > KSV ? KSK : KSV;
    constexpr int MB = BR / 32;      // 32-row blocks of the query tile
    constexpr int DBK = DK / 32, DBV = DV / 32;   // 32-row blocks of dK^T and dV^T
    constexpr int DBM = DBK > DBV ? DBK : DBV;
    // row strides of Qs (and Ks) and dOs [row][d]: 128-column tiles are
    // unpadded and chunk-swizzled (swz128), the others padded by 8 columns
    constexpr bool SWQ = DK == 128, SWO = DV == 128;
    constexpr int QPK = SWQ ? DK : DK + 8, QPV = SWO ? DV : DV + 8;
    constexpr int SP = BR + 8;       // row stride of dST          [j][i]
    constexpr int CHK = BR * DK / 8 / 256, CHV = BR * DV / 8 / 256;   // 16-byte chunks per thread per tile
    constexpr int NBLK = MB * DBK / NW;      // dQ 32x32 blocks per wavefront
    static_assert(CHK >= 1 && CHV >= 1 && NBLK >= 1, "tile shape");
    __shared__ __align__(16) uint16_t Qs[2][BR * QPK];
    __shared__ __align__(16) uint16_t dOs[2][BR * QPV];
    __shared__ __align__(16) uint16_t Ks[DQ_ATOMIC ? BC * QPK : 8];
    __shared__ __align__(16) uint16_t dST[DQ_ATOMIC ? BC * SP : 8];
    __shared__ __align__(16) float lse_s[2][BR];
    __shared__ __align__(16) float dlt_s[2][BR];
    // column position of (row, col) in a tile, and the transposed operand read
    auto tcolq = [](int row, int col) { return SWQ ? swz128_col(row, col) : col; };
    auto tcolo = [](int row, int col) { return SWO ? swz128_col(row, col) : col; };
    auto ldt_q = [&](const uint16_t* X, int k0, int n0, int ln) {
        if constexpr (SWQ) return ld_tr_swz128<true>(X, k0, n0, ln);
        else return ld_tr<true>(X, QPK, k0, n0, ln);
    };
    auto ldt_o = [&](const uint16_t* X, int k0, int n0, int ln) {
        if constexpr (SWO) return ld_tr_swz128<true>(X, k0, n0, ln);
        else return ld_tr<true>(X, QPV, k0, n0, ln);
    };
    auto ldt_row = [&](const uint16_t* X, int k0, int n0, int ln) {
        if constexpr (SWQ) return ld_tr_swz128<false>(X, k0, n0, ln);
        else return ld_tr<false>(X, QPK, k0, n0, ln);
    };

    const int tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6;
    const int g = lane >> 5, c = lane & 31;
    // Grid (sequence x KV head, key tile), taken in XCD groups: each XCD runs
    // the key tiles of kXcdGroup of its units at a time, longest causal range
    // first (see xcd_group_order).
    int unit, tile;
    xcd_group_order(gridDim.x, gridDim.y, blockIdx.y * gridDim.x + blockIdx.x, unit, tile);
    const int b = unit / p.Hkv, hk = unit % p.Hkv;
    const int G = p.Hq / p.Hkv;
    int q0 = 0, k0 = 0, lq = p.Sq, lk = p.Sk;
    if (p.varlen) seq_get(p.seqs, b, q0, k0, lq, lk);
    const int j0 = tile * BC;
    if (j0 >= lk) return;
    const bool full_cols = j0 + BC <= lk;

    const uint16_t* kbase = p.k.p + b * p.k.sb + hk * p.k.sh + (int64_t)k0 * p.k.ss;
    const uint16_t* vbase = p.v.p + b * p.v.sb + hk * p.v.sh + (int64_t)k0 * p.v.ss;

    const int my_j = j0 + 32 * w + c;
    const bool col_ok = my_j < lk;
    u32x4 kreg[KSK], vreg[KSV];
#pragma unroll
    for (int s = 0; s < KSM; ++s) {
        u32x4 z = {0u, 0u, 0u, 0u};
        if (s < KSK) kreg[s] = col_ok ? ld16(kbase + (int64_t)my_j * p.k.ss + 16 * s + 8 * g) : z;
        if (s < KSV) vreg[s] = col_ok ? ld16(vbase + (int64_t)my_j * p.v.ss + 16 * s + 8 * g) : z;
        if (DQ_ATOMIC && s < KSK) st16(&Ks[(32 * w + c) * QPK + tcolq(32 * w + c, 16 * s + 8 * g)], kreg[s]);
    }

    f32x16 dva[DBV], dka[DBK];
#pragma unroll
    for (int db = 0; db < DBM; ++db) {
        if (db < DBV) dva[db] = zero16();
        if (db < DBK) dka[db] = zero16();
    }

    // steps: query heads of the group outer, query tiles from the causal start inner
    const int i_begin = CAUSAL ? (j0 / BR) * BR : 0;
    const int per_head = lq > i_begin ? (lq - i_begin + BR - 1) / BR : 0;
    const int n_steps = G * per_head;

    // per-thread byte offsets of its 16-byte chunks inside a tile (row r,
    // column cc); row strides are below 2^23 elements, so they fit 32 bits
    const uint32_t qss = 2u * (uint32_t)p.q.ss, doss = 2u * (uint32_t)p.dout.ss;
    const int64_t ws_ss = p.varlen ? p.Hq : 1;      // row stride of lse2 / delta
    const uint32_t wss = 4u * (uint32_t)ws_ss;
    // (chunk x of a Q tile: row e / (DK/8); of a dO tile: row e / (DV/8))
    auto qrow = [&](int x) { return (tid + 256 * x) / (DK / 8); };
    auto qcol = [&](int x) { return ((tid + 256 * x) % (DK / 8)) * 8; };
    auto orow = [&](int x) { return (tid + 256 * x) / (DV / 8); };
    auto ocol = [&](int x) { return ((tid + 256 * x) % (DV / 8)) * 8; };
    uint32_t qoff[CHK], dooff[CHV];
#pragma unroll
    for (int x = 0; x < CHK; ++x) qoff[x] = qrow(x) * qss + 2 * qcol(x);
#pragma unroll
    for (int x = 0; x < CHV; ++x) dooff[x] = orow(x) * doss + 2 * ocol(x);

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
    u32x4 pq[CHK], pdo[CHV];
    float pl = INFINITY, pd = 0.f;
    int pi0 = 0;
    auto load_tile = [&]() {
        uint32_t oq[CHK], odo[CHV];
        uint32_t so = (uint32_t)(tid & (BR - 1)) * wss;
        if (ld_i0 + BR <= lq) {
#pragma unroll
            for (int x = 0; x < CHK; ++x) oq[x] = qoff[x];
#pragma unroll
            for (int x = 0; x < CHV; ++x) odo[x] = dooff[x];
        } else {
            const int last = lq - 1 - ld_i0;
#pragma unroll
            for (int x = 0; x < CHK; ++x) oq[x] = (uint32_t)min(qrow(x), last) * qss + 2 * qcol(x);
#pragma unroll
            for (int x = 0; x < CHV; ++x) odo[x] = (uint32_t)min(orow(x), last) * doss + 2 * ocol(x);
            so = (uint32_t)min(tid & (BR - 1), last) * wss;
        }
#pragma unroll
        for (int x = 0; x < CHK; ++x) pq[x] = ld16_at(ld_q, oq[x]);
#pragma unroll
        for (int x = 0; x < CHV; ++x) pdo[x] = ld16_at(ld_do, odo[x]);
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
        for (int x = 0; x < CHK; ++x) st16(&Qs[buf][qrow(x) * QPK + tcolq(qrow(x), qcol(x))], pq[x]);
#pragma unroll
        for (int x = 0; x < CHV; ++x) st16(&dOs[buf][orow(x) * QPV + tcolo(orow(x), ocol(x))], pdo[x]);
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
                for (int s = 0; s < KSM; ++s) {
                    const int row = mb * 32 + c, col = 16 * s + 8 * g;
                    if (s < KSK) sa[mb] = T::mma(ld16(&Qb[row * QPK + tcolq(row, col)]), kreg[s], sa[mb]);
                    if (s < KSV) pa[mb] = T::mma(ld16(&dOb[row * QPV + tcolo(row, col)]), vreg[s], pa[mb]);
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
                    for (int db = 0; db < DBM; ++db) {
                        if (db < DBV) dva[db] = T::mma(ldt_o(dOb, mb * 32 + 16 * hh, db * 32, lane), bP, dva[db]);
                        if (db < DBK) dka[db] = T::mma(ldt_q(Qb, mb * 32 + 16 * hh, db * 32, lane), bS, dka[db]);
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
                for (int s = 0; s < KSM; ++s) {
                    const int row = mb * 32 + c, col = 16 * s + 8 * g;
                    if (s < KSK) sa = T::mma(ld16(&Qb[row * QPK + tcolq(row, col)]), kreg[s], sa);
                    if (s < KSV) pa = T::mma(ld16(&dOb[row * QPV + tcolo(row, col)]), vreg[s], pa);
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
                    for (int db = 0; db < DBM; ++db) {
                        if (db < DBV) dva[db] = T::mma(ldt_o(dOb, mb * 32 + 16 * hh, db * 32, lane), bP, dva[db]);
                        if (db < DBK) dka[db] = T::mma(ldt_q(Qb, mb * 32 + 16 * hh, db * 32, lane), bS, dka[db]);
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
                    const int blk = w + x * NW, ib = blk / DBK, db = blk % DBK;
                    acc[x] = T::mma(ld_tr<false>(dST, SP, 16 * ks, ib * 32, lane),
                                    ldt_row(Ks, 16 * ks, db * 32, lane), acc[x]);
                }
            // accumulator rows of this (sequence, head): head-major, row stride D floats
            const int64_t arow0 = p.varlen ? ((int64_t)h * p.Sq + q0) : (((int64_t)b * p.Hq + h) * p.Sq);
            float* dqa = p.dqacc + (arow0 + i0) * D + c;
            const bool full_rows = i0 + BR <= lq;
#pragma unroll
            for (int x = 0; x < NBLK; ++x) {
                const int blk = w + x * NW, ib = blk / DBK, db = blk % DBK;
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

    if (!p.grad_f32) {
        // 16-bit gradients leave through LDS (the Q/dO tiles are free after
        // the loop's last barrier): in the accumulator layout a store
        // instruction covers 8 bytes of each of 32 rows; staged, each covers
        // whole rows.  Row r's 16-byte chunk ch sits at position (ch + r) mod
        // the row's chunk count, so the staging writes of a wavefront's 32
        // rows spread over the banks.
        constexpr int NCK = DK / 8, NCV = DV / 8;
        static_assert(2 * BR * QPK >= BC * DK && 2 * BR * QPV >= BC * DV, "staging fits the tile buffers");
        static_assert((BC * NCK) % 256 == 0 && (BC * NCV) % 256 == 0, "whole chunks per thread");
        uint16_t* sk = &Qs[0][0];       // [BC][DK]
        uint16_t* sv = &dOs[0][0];      // [BC][DV]
        const int r = 32 * w + c;
#pragma unroll
        for (int db = 0; db < DBM; ++db)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int ch = 4 * db + q;
                if (db < DBK) {
                    u32x2 x;
                    x[0] = T::pack(f32_round(dka[db][4 * q + 0] * p.scale), f32_round(dka[db][4 * q + 1] * p.scale));
                    x[1] = T::pack(f32_round(dka[db][4 * q + 2] * p.scale), f32_round(dka[db][4 * q + 3] * p.scale));
                    st8(&sk[r * DK + ((ch + r) % NCK) * 8 + 4 * g], x);
                }
                if (db < DBV) {
                    u32x2 x;
                    x[0] = T::pack(dva[db][4 * q + 0], dva[db][4 * q + 1]);
                    x[1] = T::pack(dva[db][4 * q + 2], dva[db][4 * q + 3]);
                    st8(&sv[r * DV + ((ch + r) % NCV) * 8 + 4 * g], x);
                }
            }
        __syncthreads();
        const int nrow = min(BC, lk - j0);
        uint16_t* dkp = p.dk.p + b * p.dk.sb + hk * p.dk.sh + (int64_t)(k0 + j0) * p.dk.ss;
        uint16_t* dvp = p.dv.p + b * p.dv.sb + hk * p.dv.sh + (int64_t)(k0 + j0) * p.dv.ss;
#pragma unroll
        for (int x = 0; x < BC * NCK / 256; ++x) {
            const int e = tid + 256 * x, row = e / NCK, ch = e % NCK;
            if (row < nrow) st16(dkp + (int64_t)row * p.dk.ss + ch * 8, ld16(&sk[row * DK + ((ch + row) % NCK) * 8]));
        }
#pragma unroll
        for (int x = 0; x < BC * NCV / 256; ++x) {
            const int e = tid + 256 * x, row = e / NCV, ch = e % NCV;
            if (row < nrow) st16(dvp + (int64_t)row * p.dv.ss + ch * 8, ld16(&sv[row * DV + ((ch + row) % NCV) * 8]));
        }
        return;
    }
    if (!col_ok) return;
    const int64_t dko = b * p.dk.sb + hk * p.dk.sh + (int64_t)(k0 + my_j) * p.dk.ss;
    const int64_t dvo = b * p.dv.sb + hk * p.dv.sh + (int64_t)(k0 + my_j) * p.dv.ss;
#pragma unroll
    for (int db = 0; db < DBM; ++db)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int e = db * 32 + 8 * q + 4 * g;
            if (db < DBK)
                st_grad4<T>(p.dk.p, dko + e, p.grad_f32, dka[db][4 * q + 0] * p.scale, dka[db][4 * q + 1] * p.scale,
                            dka[db][4 * q + 2] * p.scale, dka[db][4 * q + 3] * p.scale);
            if (db < DBV)
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

template <class T, int D, int DV, bool CAUSAL>
__global__ __launch_bounds__(kThreads, (D > 128 ? 1 : 2)) void bwd_dq8_kernel(BwdParams p) {
    __shared__ __align__(16) unsigned char arena[Dq8Lds<D, DV>::BYTES];
    // units: (sequence, query head), sharing K and V; items: query tiles,
    // the longest causal range (the last tile) first.  With the plain grid
    // each XCD took every eighth query tile of every head and so read every
    // head's K and V; per-unit order took the S=4096, D=128 dQ pass from 325
    // to 236 us.
    // Dense batches take the key-tile kernel's grouped order (item-major
    // across an XCD's units, so its longest query tiles go first): 225.7 ->
    // 221.9 us at B2 H16 S4096; packed batches, whose units differ in length,
    // keep the unit-major order (249.3 us; grouped, 253.2 us on 8 sequences).
    int unit, item;
    if (p.varlen) xcd_unit_order(gridDim.y, gridDim.x, blockIdx.y * gridDim.x + blockIdx.x, unit, item);
    else xcd_group_order(gridDim.y, gridDim.x, blockIdx.y * gridDim.x + blockIdx.x, unit, item);
    bwd_dq8_body<T, D, CAUSAL, DV>(p, arena, gridDim.x - 1 - item, unit);
}

// ---------------------------------------------------------------------------
// Launch
// ---------------------------------------------------------------------------

// FA2's dQ method: the key-tile kernel adds dS K to a zeroed fp32
// accumulator with atomics, then a row pass scales and rounds it into dQ.
template <class T, int D, bool CAUSAL>
static hipError_t launch_bwd_atomic_t(const BwdParams& p, const BwdLaunch& L, hipStream_t st) {
    const int64_t row_threads = p.rows * (D / 8);
    const dim3 row_grid((unsigned)((row_threads + 255) / 256));   // dQ conversion: 8 elements per thread
    const bool have_rows = p.rows > 0;
    if ((L.phase & BwdLaunch::kFirst) && have_rows) {
        const hipError_t e = launch_bwd_pre(p, L.dtype, D, true, st);
        if (e != hipSuccess) return e;
    }
    const dim3 main_grid(L.n_seq * p.Hkv, L.max_kv_tiles);
    if (main_grid.x > 0 && main_grid.y > 0)
        PROF_LAUNCH(KID_BWD_MAIN, st, (bwd_main_kernel<T, D, D, CAUSAL, true>), main_grid, dim3(256), 0, st, p);
    if ((L.phase & BwdLaunch::kLast) && have_rows)
        PROF_LAUNCH(KID_BWD_DQ_CONVERT, st, (bwd_dq_convert_kernel<T, D>), row_grid, dim3(256), 0, st, p);
    return hipGetLastError();
}

// DK: head dim of Q and K; DV: of V, O and dO.
template <class T, int DK, int DV, bool CAUSAL>
static hipError_t launch_bwd128_t(const BwdParams& p, const BwdLaunch& L, hipStream_t st) {
    // the atomic dQ form exists for equal head dims up to 128 (the host
    // offers dQ mode 2 only there)
    if constexpr (DK == DV && DK <= 128)
        if (!L.deterministic) return launch_bwd_atomic_t<T, DK, CAUSAL>(p, L, st);
    if ((L.phase & BwdLaunch::kFirst) && p.rows > 0) {
        const hipError_t e = launch_bwd_pre(p, L.dtype, DV, false, st);
        if (e != hipSuccess) return e;
    }
    const dim3 main_grid(L.n_seq * p.Hkv, L.max_kv_tiles);
    if (main_grid.x > 0 && main_grid.y > 0)
        PROF_LAUNCH(KID_BWD_MAIN, st, (bwd_main_kernel<T, DK, DV, CAUSAL, false>), main_grid, dim3(256), 0, st, p);
    const dim3 dq_grid(L.max_q_tiles64, L.n_seq * p.Hq);
    if (dq_grid.x > 0 && dq_grid.y > 0)
        PROF_LAUNCH(KID_BWD_DQ_DET, st, (bwd_dq8_kernel<T, DK, DV, CAUSAL>), dq_grid, dim3(kThreads), 0, st, p);
    return hipGetLastError();
}

template <class T, int DK, int DV>
static hipError_t launch_bwd_big_d(const BwdParams& p, const BwdLaunch& L, hipStream_t st) {
    return L.causal ? launch_bwd128_t<T, DK, DV, true>(p, L, st) : launch_bwd128_t<T, DK, DV, false>(p, L, st);
}

}  // namespace sdpa
