// SDPA backward, FlashAttention-2 style, for gfx950: the row pass and the D=64
// kernel.  (The D=128 kernels are in bwd128.hip; the helpers both use in
// bwd_shared.h.)
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
//
// The formulas: dV = P^T dO, dQ = s dS K, dK = s dS^T Q (Ascend
// aclnnNsaSelectedAttentionGrad page, "Formula" section), with
// dS = P o (dP - Delta), Delta_i = sum_j P_ij dP_ij = sum_d dO_id O_id, the
// softmax gradient written with the forward output instead of P.
#include <type_traits>

#include "bwd_shared.h"
#include "common.h"
#include "kernels.h"
#include "prof.h"

namespace sdpa {

// ---------------------------------------------------------------------------
// Preprocess
// ---------------------------------------------------------------------------

template <int D>
constexpr int pre_rows_per_block() { return 256 / pre_lanes<D>(); }

template <class T, int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(BwdParams p, int zero_dq) {
    row_pass_rows<T, D, 256>(p, zero_dq, blockIdx.x, blockIdx.y);
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

// NW: wavefronts of the workgroup (4, or 2 in the two-wavefront form); each
// owns 32 rows, so a workgroup covers 32 * NW rows.
template <class T, int D, bool CAUSAL, int NW = 4>
__device__ __forceinline__ void bwd_dqw_body(const BwdParams& p, unsigned char* arena, int bx, int by) {
    static_assert(D == 64, "wide dQ body: D=64");
    constexpr int NT = 64 * NW;             // threads
    constexpr int BQ = 32 * NW;             // query rows per workgroup
    constexpr int BK = DqwLds<D>::BK;       // keys per step
    constexpr int KS = D / 16;              // k-steps over the head dimension (32x32x16)
    constexpr int DB = D / 32;              // 32-row blocks of dQ^T
    constexpr int KP = DqwLds<D>::KP;       // row stride of the K and V tiles  [key][d]
    constexpr int TILE = BK * KP;           // elements of one tile
    constexpr int CH = BK * D / 8 / NT;   // 16-byte chunks per thread per tile
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
        const int e = tid + NT * x;
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

        // dS^T as 16-bit B operands; fp16 forms it from the 16-bit P and
        // dP - Delta with packed products, bf16 in fp32 then rounds
        constexpr bool PK = std::is_same<T, F16>::value;
        u32x4 ds[2][2];
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
                        if constexpr (PK) s[rg] = pvv;
                        else dp[rg] = pvv * dp[rg];
                    }
                } else {
#pragma unroll
                    for (int rg = 0; rg < 16; ++rg) {
                        const float pvv = fast_exp2(__builtin_fmaf(s[rg], p.scale_log2, -l2));
                        if constexpr (PK) s[rg] = pvv;
                        else dp[rg] = pvv * dp[rg];
                    }
                }
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    if constexpr (PK) ds[kh][hh] = mul_f16x8(acc_to_operand<T>(s, hh), acc_to_operand<T>(dp, hh));
                    else ds[kh][hh] = acc_to_operand<T>(dp, hh);
                }
            }
        }
        if (has_next) store_tile(buf ^ 1);
        if (!dead) {
            __builtin_amdgcn_s_setprio(1);
#pragma unroll
            for (int kh = 0; kh < 2; ++kh)
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    const u32x4 bS = ds[kh][hh];
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

// ---------------------------------------------------------------------------
// Two-wavefront form of the D=64 kernel
// ---------------------------------------------------------------------------
//
// Workgroups of two wavefronts, four per CU (still two wavefronts per SIMD).
// Key-tile item: 64 keys; wavefront kw owns keys 32*kw .. +31 against every
// 32-row query tile, so each wavefront holds the whole dK/dV of its keys and
// stores them itself: no cross-wavefront reduction at the end, and the
// per-step barrier joins two wavefronts instead of four.  Query-tile item: 64
// rows, wavefront rh owns rows 32*rh .. +31 against 64-key tiles (the wide
// body with two wavefronts), again with nothing to reduce.  A key-tile
// wavefront's step (32 keys x 32 rows: S, dP, softmax gradient, dV, dK) is
// twice that of the four-wavefront form per wavefront; an item runs on two
// SIMDs instead of four, so it takes twice as long, and the form pays only
// when there are enough items to fill the CUs (see the launch).
constexpr int k2Threads = 128;

// Key-tile item of the two-wavefront form: 64 keys, wavefront kw owns keys
// 32*kw .. +31 against every 64-row query tile, as two 32-row blocks per step
// (S and dP of both, then each block's softmax gradient and dV/dK products,
// so the matrix cores work on one block while the vector ALUs run the other's
// softmax).  Q/dO tiles are double-buffered in LDS; the next tile is loaded
// into registers during the step.  Against 32-row steps with the next tile's
// S and dP computed during this tile's softmax: GPT-2 shape 41.4 -> 40.1 us.
template <int D>
struct Key2Lds {
    static constexpr int BR = 64, QP = D + 8, NBUF = 2;
    static constexpr int TILE_B = BR * QP * 2;
    static constexpr int OFF_STAT = 2 * NBUF * TILE_B;
    static constexpr int BYTES = OFF_STAT + 2 * NBUF * BR * 4;
};

template <class T, int D, bool CAUSAL>
__device__ __forceinline__ void bwd_key2_body(const BwdParams& p, unsigned char* arena, int bx, int by) {
    using L = Key2Lds<D>;
    constexpr int BC = 64, BR = L::BR, KS = D / 16, DB = D / 32, QP = L::QP, TILE = BR * QP;
    constexpr int CH = BR * D / 8 / k2Threads;
    uint16_t* Qs0 = reinterpret_cast<uint16_t*>(arena);
    uint16_t* dOs0 = Qs0 + L::NBUF * TILE;
    float* lse_s = reinterpret_cast<float*>(arena + L::OFF_STAT);
    float* dlt_s = lse_s + L::NBUF * BR;

    const int tid = threadIdx.x;
    const int lane = tid & 63, kw = tid >> 6;
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

    const int i_begin = CAUSAL ? j0 : 0;     // j0 is a multiple of the 64-row tile
    const int per_head = lq > i_begin ? (lq - i_begin + BR - 1) / BR : 0;
    const int n_steps = G * per_head;

    const uint32_t qss = 2u * (uint32_t)p.q.ss, doss = 2u * (uint32_t)p.dout.ss;
    int crow[CH], ccol[CH];
#pragma unroll
    for (int x = 0; x < CH; ++x) {
        const int e = tid + k2Threads * x;
        crow[x] = e / (D / 8);
        ccol[x] = (e % (D / 8)) * 8;
    }
    const uint16_t* const q_seq = p.q.p + b * p.q.sb + (int64_t)q0 * p.q.ss;
    const uint16_t* const do_seq = p.dout.p + b * p.dout.sb + (int64_t)q0 * p.dout.ss;
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

    struct TileRegs { u32x4 q[CH], d[CH]; float sa, sb; };
    const int srow = tid & (BR - 1);
    const uint32_t sss = 4u * (uint32_t)ws_ss;
    auto load_tile = [&](TileRegs& t) {
        const int last = lq - 1 - ld_i0;     // rows past the end re-read the last row
#pragma unroll
        for (int x = 0; x < CH; ++x) {
            const uint32_t r = min(crow[x], last);
            t.q[x] = ld16_at(ld_q, r * qss + 2 * ccol[x]);
            t.d[x] = ld16_at(ld_do, r * doss + 2 * ccol[x]);
        }
        const uint32_t so = (uint32_t)min(srow, last) * sss;
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
            const bool ok = i0 + tid < lq;
            lse_s[buf * BR + tid] = ok ? t.sa : INFINITY;
            dlt_s[buf * BR + tid] = ok ? -t.sb : 0.f;
        }
    };
    u32x4 kreg[KS], vreg[KS];

    int i0_k = i_begin;
    {
        TileRegs tr0;
        if (n_steps > 0) { load_tile(tr0); i0_k = ld_i0; advance(); }
        const int jr = min(my_j, lk - 1);
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            kreg[s] = ld16(kbase + (int64_t)jr * p.k.ss + 16 * s + 8 * g);
            vreg[s] = ld16(vbase + (int64_t)jr * p.v.ss + 16 * s + 8 * g);
        }
        if (n_steps > 0) store_tile(tr0, 0, i0_k);
    }
    wait_all_memory();
    __syncthreads();

    const int t_key = col_ok ? (CAUSAL ? my_j - 4 * g : INT_MIN / 2) : INT_MAX / 2;
    for (int k = 0; k < n_steps; ++k) {
        const int buf = k & 1;
        const bool has1 = k + 1 < n_steps;
        int i0_k1 = i0_k;
        TileRegs trn;
        if (has1) { load_tile(trn); i0_k1 = ld_i0; advance(); }
        const uint16_t* Qb = Qs0 + buf * TILE;
        const uint16_t* dOb = dOs0 + buf * TILE;
        // S^T and dP^T - Delta of both 32-row blocks
        f32x16 sab[2], pab[2];
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
            sab[rb] = zero16();
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const f32x4 nd = *reinterpret_cast<const f32x4*>(&dlt_s[buf * BR + 32 * rb + 8 * q + 4 * g]);
#pragma unroll
                for (int r = 0; r < 4; ++r) pab[rb][4 * q + r] = nd[r];
            }
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                sab[rb] = T::mma(ld16(&Qb[(32 * rb + c) * QP + 16 * s + 8 * g]), kreg[s], sab[rb]);
                pab[rb] = T::mma(ld16(&dOb[(32 * rb + c) * QP + 16 * s + 8 * g]), vreg[s], pab[rb]);
            }
        }
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
            const int r0 = i0_k + 32 * rb;
            const bool masked = (CAUSAL && r0 < j0 + BC) || !full_cols;
            // fp16: dS from the 16-bit P and dP - Delta operands, two products per instruction
            constexpr bool PK = std::is_same<T, F16>::value;
            if (masked) {
                if constexpr (PK) softmax_p_tile_nd<true>(sab[rb], &lse_s[buf * BR + 32 * rb], p.scale_log2, g, t_key - r0);
                else softmax_grad_tile_nd<true>(sab[rb], pab[rb], &lse_s[buf * BR + 32 * rb], p.scale_log2, g, t_key - r0);
            } else {
                if constexpr (PK) softmax_p_tile_nd<false>(sab[rb], &lse_s[buf * BR + 32 * rb], p.scale_log2, g, 0);
                else softmax_grad_tile_nd<false>(sab[rb], pab[rb], &lse_s[buf * BR + 32 * rb], p.scale_log2, g, 0);
            }
            __builtin_amdgcn_s_setprio(1);
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                const u32x4 bP = acc_to_operand<T>(sab[rb], hh);
                u32x4 bS = acc_to_operand<T>(pab[rb], hh);
                if constexpr (PK) bS = mul_f16x8(bP, bS);
#pragma unroll
                for (int db = 0; db < DB; ++db) {
                    dva[db] = T::mma(ld_tr<true>(dOb, QP, 32 * rb + 16 * hh, db * 32, lane), bP, dva[db]);
                    dka[db] = T::mma(ld_tr<true>(Qb, QP, 32 * rb + 16 * hh, db * 32, lane), bS, dka[db]);
                }
            }
            __builtin_amdgcn_s_setprio(0);
        }
        if (has1) store_tile(trn, buf ^ 1, i0_k1);
        __syncthreads();
        i0_k = i0_k1;
    }

    if (!p.grad_f32) {
        // 16-bit dK and dV leave through LDS as whole rows (the Q/dO tiles
        // are free after the loop's last barrier): in the accumulator layout
        // a store instruction covers 8 bytes of each of 32 rows.  Row r's
        // 16-byte chunk j sits at (j + r) mod D/8, spreading the staging
        // writes of a wavefront's 32 rows over the banks.
        constexpr int NC = D / 8;
        static_assert(2 * BC * D <= 2 * L::NBUF * TILE, "staging fits the tile buffers");
        static_assert((BC * NC) % k2Threads == 0, "whole chunks per thread");
        uint16_t* sk = Qs0;                 // [BC][D]
        uint16_t* sv = Qs0 + BC * D;        // [BC][D]
        const int r = 32 * kw + c;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int ch = (4 * db + q + r) % NC;
                u32x2 x;
                x[0] = T::pack(f32_round(dka[db][4 * q + 0] * p.scale), f32_round(dka[db][4 * q + 1] * p.scale));
                x[1] = T::pack(f32_round(dka[db][4 * q + 2] * p.scale), f32_round(dka[db][4 * q + 3] * p.scale));
                st8(&sk[r * D + ch * 8 + 4 * g], x);
                x[0] = T::pack(dva[db][4 * q + 0], dva[db][4 * q + 1]);
                x[1] = T::pack(dva[db][4 * q + 2], dva[db][4 * q + 3]);
                st8(&sv[r * D + ch * 8 + 4 * g], x);
            }
        __syncthreads();
        const int nrow = min(BC, lk - j0);
        uint16_t* dkp = p.dk.p + b * p.dk.sb + hk * p.dk.sh + (int64_t)(k0 + j0) * p.dk.ss;
        uint16_t* dvp = p.dv.p + b * p.dv.sb + hk * p.dv.sh + (int64_t)(k0 + j0) * p.dv.ss;
#pragma unroll
        for (int x = 0; x < BC * NC / k2Threads; ++x) {
            const int e = tid + k2Threads * x, row = e / NC, ch = e % NC, pos = (ch + row) % NC;
            if (row < nrow) {
                st16(dkp + (int64_t)row * p.dk.ss + ch * 8, ld16(&sk[row * D + pos * 8]));
                st16(dvp + (int64_t)row * p.dv.ss + ch * 8, ld16(&sv[row * D + pos * 8]));
            }
        }
        return;
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

// Query-tile items of the two-wavefront form: the wide body with two
// wavefronts, 64 rows against 64-key tiles.
template <class T, int D, bool CAUSAL>
__device__ __forceinline__ void fused2_dq(const BwdParams& p, unsigned char* arena, int bx, int by) {
    bwd_dqw_body<T, D, CAUSAL, 2>(p, arena, bx, by);
}

// The two-wavefront launch: key-tile items and 64-row query-tile items in one
// grid, ordered as the four-wavefront kernel orders its 64-row form.
template <class T, int D, bool CAUSAL>
__global__ __launch_bounds__(k2Threads, 2) void bwd_fused2_kernel(BwdParams p, Fused8Map m) {
    constexpr int A = Key2Lds<D>::BYTES > DqwLds<D>::BYTES ? Key2Lds<D>::BYTES : DqwLds<D>::BYTES;
    __shared__ __align__(16) unsigned char arena[A];
    const int id = blockIdx.x;
    if (m.alternate) {
        const int seg = id / m.main_x, within = id % m.main_x;
        if (!(seg & 1)) bwd_key2_body<T, D, CAUSAL>(p, arena, within, seg >> 1);
        else fused2_dq<T, D, CAUSAL>(p, arena, m.dq_x - 1 - (seg >> 1), within);
        return;
    }
    const int n_main = m.main_x * m.main_y;
    if (id < n_main) {
        bwd_key2_body<T, D, CAUSAL>(p, arena, id % m.main_x, id / m.main_x);
    } else {
        const int r = id - n_main;
        fused2_dq<T, D, CAUSAL>(p, arena, m.dq_x - 1 - r / m.dq_y, r % m.dq_y);
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
    static_assert(D == 64, "the D=64 launch");
    if (!L.deterministic) return launch_bwd_d64_atomic(p, L, st);   // dQ mode 2: fp32 atomics
    if (CAUSAL) {
        // Two-wavefront form for causal problems of at most 2048 keys with at
        // least one item per workgroup slot (four per CU).  Measured against
        // the four-wavefront form (D=64, fp16, same box): B4 H12 S1024
        // 43.8 -> 40.6 us, B2 H16 S2048 84.0 -> 80.9, B4 H12 S2048
        // 124.3 -> 121.8, B8 H8 S512 23.6 -> 22.8; B1 H16 S4096 even (+1 %);
        // with fewer items it loses (B2 H12 S1024 +17 %, B1 H12 S1024 +30 %,
        // B2 H8 S512 +23 %, B1 H2 S8192 +50 %): an item runs on two SIMDs
        // instead of four, so the longest items set the time.
        const int mx = L.n_seq * p.Hkv, my = L.max_kv_tiles64;
        const int qy = L.n_seq * p.Hq;
        const int slots2 = 2 * fused8_slots();
        const long n2 = (long)mx * my + (long)L.max_q_tiles64 * qy;
        if (slots2 > 0 && my <= 32 && n2 >= slots2) {
            if (L.phase & BwdLaunch::kFirst) launch_pre<T, D>(p, 0, st);
            Fused8Map m{mx, my, L.max_q_tiles64, qy, 0};
            m.alternate = (mx == qy && my == m.dq_x) ? 1 : 0;
            PROF_LAUNCH(KID_BWD_FUSED2, st, (bwd_fused2_kernel<T, D, CAUSAL>), dim3((unsigned)n2), dim3(k2Threads), 0,
                        st, p, m);
            return hipGetLastError();
        }
    }
    {
        // The row pass, then one launch of both bodies; dQ is computed without
        // atomics, so the result is deterministic (dQ modes 0 and 1).
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
    if (L.D == 192) return launch_bwd_d192(p, L, st);
    if (L.D != 64) return launch_bwd_d128(p, L, st);
    return L.dtype == 0 ? launch_bwd_d<F16, 64>(p, L, st) : launch_bwd_d<BF16, 64>(p, L, st);
}

}  // namespace sdpa
