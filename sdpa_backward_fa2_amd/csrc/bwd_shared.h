// Device helpers shared by the D=64 and D=128 backward kernels: statistics
// row locations, the softmax gradient of one 32x32 tile, the workgroup shape
// of the four-wavefront bodies and the 64-row query-tile dQ body.
#pragma once
#include "common.h"

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

// The row pass (Delta = sum_d dO*O, the statistics as log2-domain LSE and,
// in the atomic dQ mode, the fp32 accumulator row cleared) over the rows of
// workgroup (bx, by) of NT threads, LPR lanes per row (a power of two; 16
// elements per lane at D=64 and 128, 24 at D=192): dense, bx = chunks of rows
// of one (batch, head) = by; packed, bx = chunks of the (token, head) rows in
// memory order (the heads of a token are adjacent in the packed layout).
template <int D>
constexpr int pre_lanes() { return D == 64 ? 4 : 8; }

template <class T, int D, int NT>
__device__ __forceinline__ void row_pass_rows(const BwdParams& p, int zero_dq, int bx, int by) {
    constexpr int LPR = pre_lanes<D>();
    constexpr int EPL = D / LPR;                 // elements per lane
    constexpr int NC = EPL / 8;                  // 16-byte chunks per lane
    static_assert(EPL % 8 == 0 && (LPR & (LPR - 1)) == 0, "row split");
    constexpr int RPB = NT / LPR;                // rows per workgroup
    const int part = threadIdx.x % LPR;
    int64_t R;
    bool ok;
    RowLoc L;
    if (p.varlen) {
        R = (int64_t)bx * RPB + threadIdx.x / LPR;
        ok = R < p.rows;
        const int64_t Rc = ok ? R : p.rows - 1;           // rows past the end re-read the last
        L = RowLoc{0, Rc % p.Hq, Rc / p.Hq};
    } else {
        const int i = bx * RPB + threadIdx.x / LPR;
        const int y = by;
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

// The same softmax step leaving pa = dP - Delta: the caller forms dS = P o
// (dP - Delta) from the two 16-bit operands with packed fp16 products (two
// per instruction, rounded to nearest like the operands).
template <bool MASKED>
__device__ __forceinline__ void softmax_p_tile_nd(f32x16& sa, const float* lse_row, float scale_log2, int g, int t) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const f32x4 Lr = *reinterpret_cast<const f32x4*>(&lse_row[8 * q + 4 * g]);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int rg = 4 * q + r;
            float pv = fast_exp2(__builtin_fmaf(sa[rg], scale_log2, -Lr[r]));
            if (MASKED) pv = (8 * q + r >= t) ? pv : 0.f;
            sa[rg] = pv;
        }
    }
}

// (Each element is copied to a scalar before its bit_cast: a bit_cast of the
// indexed vector element itself compiled to four copies of element 0.)
__device__ __forceinline__ u32x4 mul_f16x8(u32x4 a, u32x4 b) {
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    u32x4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t x = a[i], y = b[i];
        r[i] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(h2, x) * __builtin_bit_cast(h2, y));
    }
    return r;
}

// Wavefronts per workgroup of the D=64 kernel and the dQ body: two row halves
// of kKeySlices key slices.  Four wavefronts let two workgroups share a CU (two
// wavefronts per SIMD), so one workgroup's memory waits and barriers overlap
// the other's arithmetic.
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kKeySlices = kWaves / 2;

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

// D: head dim of Q and K (and of dQ); DV: of V and dO.  At D = DV = 128 the
// key tiles go from global memory straight to LDS (global_load_lds_dwordx4,
// no staging registers) into unpadded rows whose 16-byte chunk j of row r
// sits at j ^ swz128(r): the MFMA operand reads of the dS and dQ products
// then meet distinct banks (the padded rows of the register-staged form left
// 26 M bank-conflict cycles against 23 M LDS instructions at S=4096, and its
// 255 registers had no room for the swizzle's address arithmetic).
template <int D, int DV>
constexpr bool dq8_direct() { return D == 128 && DV == 128; }

template <int D, int DV = D>
struct Dq8Lds {
    static constexpr int BK = 32 * kKeySlices, DB = D / 32;
    static constexpr int KP = dq8_direct<D, DV>() ? D : D + 8, KPV = dq8_direct<D, DV>() ? DV : DV + 8;
    static constexpr int TILE_B = BK * KP * 2, TILE_VB = BK * KPV * 2;
    static constexpr int LOOP_B = 2 * TILE_B + 2 * TILE_VB;
    static constexpr int RED_B = (kKeySlices - 1) * 2 * 64 * (DB * 16) * 4;
    static constexpr int BYTES = LOOP_B > RED_B ? LOOP_B : RED_B;
};

template <class T, int D, bool CAUSAL, int DV = D>
__device__ __forceinline__ void bwd_dq8_body(const BwdParams& p, unsigned char* arena, int bx, int by) {
    constexpr int BQ = 64;           // query rows per workgroup
    constexpr int BK = 32 * kKeySlices;   // keys per step
    constexpr int KS = D / 16;       // k-steps of S over D (32x32x16)
    constexpr int KSV = DV / 16;     // k-steps of dP over DV
    constexpr int KSM = KS > KSV ? KS : KSV;
    constexpr int DB = D / 32;       // 32-row blocks of dQ^T
    constexpr bool DIRECT = dq8_direct<D, DV>();   // direct-to-LDS, swizzled tiles
    constexpr int KP = Dq8Lds<D, DV>::KP;          // row stride of Ks  [key][d]
    constexpr int KPV = Dq8Lds<D, DV>::KPV;        // row stride of Vs  [key][dv]
    constexpr int CH = BK * D / 8 / kThreads;     // 16-byte chunks per thread per K tile
    constexpr int CHV = BK * DV / 8 / kThreads;   // and per V tile
    constexpr int TILE_B = BK * KP * 2, TILE_VB = BK * KPV * 2;
    constexpr int OFF_K = 0, OFF_V = 2 * TILE_B;
    constexpr int LOOP_B = 2 * TILE_B + 2 * TILE_VB;
    constexpr int RED_B = (kKeySlices - 1) * 2 * 64 * (DB * 16) * 4;   // key slices 1.. of both row halves
    static_assert(Dq8Lds<D, DV>::BYTES >= (LOOP_B > RED_B ? LOOP_B : RED_B), "arena size");
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
    uint32_t koff[CH], voff[CHV];
    int crow[CH], ccol[CH];
#pragma unroll
    for (int x = 0; x < CH; ++x) {
        const int e = tid + kThreads * x;
        const int r = e / (D / 8), cc = (e % (D / 8)) * 8;
        crow[x] = r;
        ccol[x] = cc;
        koff[x] = r * kss + 2 * cc;
    }
    // chunk x of a V tile (the K tile's when DV == D)
    auto vrow = [&](int x) { return (tid + kThreads * x) / (DV / 8); };
    auto vcol = [&](int x) { return ((tid + kThreads * x) % (DV / 8)) * 8; };
#pragma unroll
    for (int x = 0; x < CHV; ++x) voff[x] = vrow(x) * vss + 2 * vcol(x);
    // Unconditional loads: keys past the end of the sequence re-read its last
    // key and are masked out (P = 0), so nothing is waited for before the tile
    // is stored after the step's products.
    u32x4 pk[CH], pv[CHV];
    const uint16_t* kb = kbase;          // key tile being loaded, advanced per step
    const uint16_t* vb = vbase;
    const int64_t k_step = BK * p.k.ss, v_step = BK * p.v.ss;
    auto load_tile = [&](int st) {
        const int j0 = st * BK;
        uint32_t ok_[CH], ov_[CHV];
        if (j0 + BK <= lk) {
#pragma unroll
            for (int x = 0; x < CH; ++x) ok_[x] = koff[x];
#pragma unroll
            for (int x = 0; x < CHV; ++x) ov_[x] = voff[x];
        } else {
            const int last = lk - 1 - j0;
#pragma unroll
            for (int x = 0; x < CH; ++x) ok_[x] = (uint32_t)min(crow[x], last) * kss + 2 * ccol[x];
#pragma unroll
            for (int x = 0; x < CHV; ++x) ov_[x] = (uint32_t)min(vrow(x), last) * vss + 2 * vcol(x);
        }
#pragma unroll
        for (int x = 0; x < CH; ++x) pk[x] = ld16_at(kb, ok_[x]);
#pragma unroll
        for (int x = 0; x < CHV; ++x) pv[x] = ld16_at(vb, ov_[x]);
        kb += k_step;
        vb += v_step;
    };
    auto store_tile = [&](int buf) {
        uint16_t* Kd = Ks0 + buf * (BK * KP);
        uint16_t* Vd = Vs0 + buf * (BK * KPV);
#pragma unroll
        for (int x = 0; x < CH; ++x) st16(&Kd[crow[x] * KP + ccol[x]], pk[x]);
#pragma unroll
        for (int x = 0; x < CHV; ++x) st16(&Vd[vrow(x) * KPV + vcol(x)], pv[x]);
    };
    // Direct form: wavefront w fills 1 KiB blocks w*CH .. w*CH + CH-1 of
    // each tile; lane l of block m writes tile chunk position 64m + l (row
    // (64m + l) / 16, position (64m + l) % 16), which holds the row's
    // global chunk position ^ swz128(row).  Keys past the end re-read the
    // last key (masked out, P = 0).
    static_assert(!DIRECT || (CH == CHV && D / 8 == 16), "direct tiles: 16 chunks per row");
    auto dma_tile = [&](int st, int buf) {
        if constexpr (DIRECT) {
            const int j0 = st * BK, last = lk - 1 - j0;
            const unsigned char* kt = reinterpret_cast<const unsigned char*>(kbase + (int64_t)j0 * p.k.ss);
            const unsigned char* vt = reinterpret_cast<const unsigned char*>(vbase + (int64_t)j0 * p.v.ss);
#pragma unroll
            for (int x = 0; x < CH; ++x) {
                const int m = w * CH + x, q = 64 * m + lane, r = q >> 4;
                const uint32_t col = (uint32_t)(((q & 15) ^ swz128(r)) * 16);
                const uint32_t rr = (uint32_t)min(r, last);
                __builtin_amdgcn_global_load_lds(kt + rr * kss + col,
                                                 (__attribute__((address_space(3))) void*)(Ks0 + buf * (BK * KP) + 512 * m),
                                                 16, 0, 0);
                __builtin_amdgcn_global_load_lds(vt + rr * vss + col,
                                                 (__attribute__((address_space(3))) void*)(Vs0 + buf * (BK * KPV) + 512 * m),
                                                 16, 0, 0);
            }
        }
    };

    // Prologue: the first key tile and this lane's query row are requested
    // before anything waits for memory.
    if (n_steps > 0) {
        if constexpr (DIRECT) dma_tile(0, 0);
        else load_tile(0);
    }
    const int my_i = i0 + 32 * rh + c;
    const bool row_ok = my_i < lq;
    // a row past the end of the sequence re-reads its last row; its LSE is
    // +inf (P = 0) and its dQ is not stored
    const int my_ic = min(my_i, lq - 1);
    u32x4 qreg[KS], doreg[KSV];
#pragma unroll
    for (int s = 0; s < KSM; ++s) {
        if (s < KS) qreg[s] = ld16(qbase + (int64_t)my_ic * p.q.ss + 16 * s + 8 * g);
        if (s < KSV) doreg[s] = ld16(dobase + (int64_t)my_ic * p.dout.ss + 16 * s + 8 * g);
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

    if constexpr (!DIRECT) {
        if (n_steps > 0) store_tile(0);
    }
    wait_all_memory();
    __syncthreads();

    // last key this lane's row keeps, relative to the 8q+4g part of a tile row
    const int t_row = min(lk - 1, CAUSAL ? my_i : INT_MAX) - 32 * kw - 4 * g;

    for (int st = 0; st < n_steps; ++st) {
        const int buf = st & 1;
        const int j0 = st * BK;
        const bool has_next = st + 1 < n_steps;
        if (has_next) {
            // the other buffer's tile was last read before the previous step's barrier
            if constexpr (DIRECT) dma_tile(st + 1, buf ^ 1);
            else load_tile(st + 1);
        }
        const uint16_t* Kb = Ks0 + buf * (BK * KP);
        const uint16_t* Vb = Vs0 + buf * (BK * KPV);

        f32x16 s = zero16(), dp = ndl16;   // dP^T accumulates onto -Delta
        const int kr = 32 * kw + c;
#pragma unroll
        for (int ks = 0; ks < KSM; ++ks) {
            const int col = 16 * ks + 8 * g;
            if (ks < KS) s = T::mma(ld16(&Kb[kr * KP + (DIRECT ? swz128_col(kr, col) : col)]), qreg[ks], s);
            if (ks < KSV) dp = T::mma(ld16(&Vb[kr * KPV + (DIRECT ? swz128_col(kr, col) : col)]), doreg[ks], dp);
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
        if constexpr (!DIRECT) {
            if (has_next) store_tile(buf ^ 1);
        }
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            const u32x4 bS = acc_to_operand<T>(dp, hh);
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                u32x4 a;
                if constexpr (DIRECT) a = ld_tr_swz128<true>(Kb, 32 * kw + 16 * hh, db * 32, lane);
                else a = ld_tr<true>(Kb, KP, 32 * kw + 16 * hh, db * 32, lane);
                dq[db] = T::mma(a, bS, dq[db]);
            }
        }
        __builtin_amdgcn_s_setprio(0);
        // direct form: the next tile's loads land in LDS before the barrier
        if constexpr (DIRECT) wait_all_memory();
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

}  // namespace sdpa
