// Shared device helpers for the gfx950 SDPA kernels: 16-bit element types,
// MFMA wrappers, conversions and the kernel parameter blocks.
//
// MFMA register layouts used throughout (v_mfma_f32_32x32x16_{f16,bf16}, one
// wavefront of 64 lanes, lane = 32*g + c with g in {0,1}, c in 0..31):
//   A (32 x 16): lane (c, g) holds row c, eight k-slots (g, t), t = 0..7;
//   B (16 x 32): lane (c, g) holds column c, the same eight k-slots (g, t);
//   C (32 x 32): lane (c, g) holds column c, rows 8*q + 4*g + r in register 4*q + r.
// A and B pair slot (g, t) with slot (g, t), so any one-to-one assignment of the
// 16 k indices to the 16 slots gives the same product as long as A and B use
// the same assignment.  Two assignments occur:
//   "row slots":  k = 8*g + t             (operands read as 16 contiguous bytes);
//   "acc slots":  k = 4*g + t (t < 4), 8 + 4*g + (t-4) (t >= 4), relative to a
//                 16-row half of a C tile: this is how the rows of a C tile sit
//                 in registers 8*h .. 8*h+7, so a C tile (rows = the contracted
//                 index) feeds straight into the B operand of the next product.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sdpa {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kWave = 64;

struct F16 {
    static __device__ __forceinline__ f32x16 mma(u32x4 a, u32x4 b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    }
    static __device__ __forceinline__ f32x4 mma16(u32x4 a, u32x4 b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    }
    static __device__ __forceinline__ uint16_t cvt(float x) {
        return __builtin_bit_cast(uint16_t, (_Float16)x);
    }
    static __device__ __forceinline__ uint32_t pack(float lo, float hi) {
        return (uint32_t)cvt(lo) | ((uint32_t)cvt(hi) << 16);
    }
    static __device__ __forceinline__ float to_f32(uint16_t x) {
        return (float)__builtin_bit_cast(_Float16, x);
    }
    // MFMA operands built from fp32 intermediates (P, dS): one instruction per
    // pair (gfx950's v_cvt_pk_f16_f32), rounding to nearest even like the
    // outputs, so the 16-bit operands carry no rounding bias.
    static __device__ __forceinline__ uint32_t pack_op(float lo, float hi) {
        typedef _Float16 h2 __attribute__((ext_vector_type(2)));
        const h2 v = {(_Float16)lo, (_Float16)hi};
        return __builtin_bit_cast(uint32_t, v);
    }
    // c + a.lo*b.lo + a.hi*b.hi in fp32 (one v_dot2 instruction)
    static __device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
        typedef _Float16 h2 __attribute__((ext_vector_type(2)));
        return __builtin_amdgcn_fdot2(__builtin_bit_cast(h2, a), __builtin_bit_cast(h2, b), c, false);
    }
};

struct BF16 {
    static __device__ __forceinline__ f32x16 mma(u32x4 a, u32x4 b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    }
    static __device__ __forceinline__ f32x4 mma16(u32x4 a, u32x4 b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    }
    static __device__ __forceinline__ uint16_t cvt(float x) {
        return __builtin_bit_cast(uint16_t, (__bf16)x);
    }
    // a pair as one vector conversion, so that it is one gfx950 instruction
    // (round to nearest even, as the scalar conversion)
    static __device__ __forceinline__ uint32_t pack(float lo, float hi) {
        typedef float f2 __attribute__((ext_vector_type(2)));
        typedef __bf16 b2 __attribute__((ext_vector_type(2)));
        const f2 v = {lo, hi};
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, b2));
    }
    static __device__ __forceinline__ float to_f32(uint16_t x) {
        return __builtin_bit_cast(float, (uint32_t)x << 16);
    }
    static __device__ __forceinline__ uint32_t pack_op(float lo, float hi) { return pack(lo, hi); }
    static __device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
        typedef __bf16 b2 __attribute__((ext_vector_type(2)));
        return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(b2, a), __builtin_bit_cast(b2, b), c, false);
    }
};

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// The value as an fp32 result: keeps the compiler from fusing the product that
// made it into a later conversion to 16 bits (v_fma_mix*, one rounding), so a
// 16-bit output equals the fp32 output of the same call rounded to 16 bits.
__device__ __forceinline__ float f32_round(float x) {
    asm volatile("" : "+v"(x));
    return x;
}

// lane exchange inside a row of 16 lanes (DPP control word CTRL)
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}

// Sum over aligned groups of N (8 or 16) consecutive lanes; every lane of the
// group receives the sum.  Quad swaps, then the half-row and row mirrors.
template <int N>
__device__ __forceinline__ float lane_group_sum(float x) {
    static_assert(N == 8 || N == 16, "group size");
    x += dpp_f32<0xB1>(x);    // quad_perm 1,0,3,2
    x += dpp_f32<0x4E>(x);    // quad_perm 2,3,0,1
    x += dpp_f32<0x141>(x);   // row_half_mirror
    if (N == 16) x += dpp_f32<0x140>(x);   // row_mirror
    return x;
}

// Wait for every outstanding memory operation of the wavefront.
__device__ __forceinline__ void wait_all_memory() { __builtin_amdgcn_s_waitcnt(0); }

__device__ __forceinline__ u32x4 ld16(const uint16_t* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void st16(uint16_t* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }
__device__ __forceinline__ u32x2 ld8(const uint16_t* p) { return *reinterpret_cast<const u32x2*>(p); }
// Loads at an unsigned 32-bit byte offset from a base every lane shares: they
// take the scalar-base + vector-offset addressing form, with no 64-bit
// address arithmetic per lane.
__device__ __forceinline__ u32x4 ld16_at(const void* base, uint32_t off) {
    return *reinterpret_cast<const u32x4*>(static_cast<const unsigned char*>(base) + off);
}
__device__ __forceinline__ float ldf_at(const float* base, uint32_t off) {
    return *reinterpret_cast<const float*>(reinterpret_cast<const unsigned char*>(base) + off);
}
__device__ __forceinline__ void st8(uint16_t* p, u32x2 v) { *reinterpret_cast<u32x2*>(p) = v; }

// Gradient outputs hold either the input dtype T (f32 == 0) or fp32; `off`
// counts elements from `base`, so both forms use the caller's element strides.
template <class T>
__device__ __forceinline__ void st_grad4(uint16_t* base, int64_t off, int f32, float a, float b, float c, float d) {
    if (f32) {
        const f32x4 v = {a, b, c, d};
        *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(base) + off) = v;
    } else {
        u32x2 v;
        v[0] = T::pack(a, b);
        v[1] = T::pack(c, d);
        st8(base + off, v);
    }
}
template <class T>
__device__ __forceinline__ void st_grad8(uint16_t* base, int64_t off, int f32, const float* x) {
    if (f32) {
        const f32x4 lo = {x[0], x[1], x[2], x[3]}, hi = {x[4], x[5], x[6], x[7]};
        f32x4* d = reinterpret_cast<f32x4*>(reinterpret_cast<float*>(base) + off);
        d[0] = lo;
        d[1] = hi;
    } else {
        u32x4 v;
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = T::pack(x[2 * i], x[2 * i + 1]);
        st16(base + off, v);
    }
}

__device__ __forceinline__ uint16_t elem16(u32x4 v, int t) {
    uint32_t w = v[t >> 1];
    return (uint16_t)((t & 1) ? (w >> 16) : (w & 0xffffu));
}

// Eight consecutive fp32 registers of a C tile (rows 16*h .. 16*h+15 of the
// tile in "acc slot" order) rounded to a 16-bit B operand.
template <class T>
__device__ __forceinline__ u32x4 acc_to_operand(const f32x16& a, int h) {
    u32x4 r;
    r[0] = T::pack_op(a[8 * h + 0], a[8 * h + 1]);
    r[1] = T::pack_op(a[8 * h + 2], a[8 * h + 3]);
    r[2] = T::pack_op(a[8 * h + 4], a[8 * h + 5]);
    r[3] = T::pack_op(a[8 * h + 6], a[8 * h + 7]);
    return r;
}

// A operand in "acc slot" order from a row of a transposed LDS tile: the row
// holds the contracted index contiguously; `base` points at element 16*h of the
// 32-wide block, g is the lane half.
__device__ __forceinline__ u32x4 ld_acc_slots(const uint16_t* base, int g) {
    u32x2 lo = ld8(base + 4 * g);
    u32x2 hi = ld8(base + 8 + 4 * g);
    u32x4 r;
    r[0] = lo[0]; r[1] = lo[1]; r[2] = hi[0]; r[3] = hi[1];
    return r;
}

// Transposed operand from a row-major LDS tile X (row stride ld elements) whose
// rows are the contracted index k and whose columns are the MFMA's free index:
// this lane gets column n0 + (lane % 32) and the eight k values of its slots.
// ds_read_b64_tr_b16 works on 16-lane groups: lane p of a group supplies the
// address of four consecutive columns 4*(p%4).. of row p/4 and receives column
// p of the four rows, so two reads give the eight slots.
//   ACC = false: "row slots"  k = k0 + 8*g + t;
//   ACC = true:  "acc slots"  k = k0 + 4*g + t (t < 4), k0 + 8 + 4*g + t - 4.
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

template <bool ACC>
__device__ __forceinline__ u32x4 ld_tr(const uint16_t* X, int ld, int k0, int n0, int lane) {
    const int p = lane & 15, grp = lane >> 4;
    const int g = grp >> 1, cb = (grp & 1) * 16;
    const int kr0 = ACC ? (k0 + 4 * g) : (k0 + 8 * g);
    const int kr1 = ACC ? (k0 + 8 + 4 * g) : (k0 + 8 * g + 4);
    const int col = n0 + cb + 4 * (p & 3);
    const s16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(X + (kr0 + (p >> 2)) * ld + col));
    const s16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(X + (kr1 + (p >> 2)) * ld + col));
    const u32x2 a = __builtin_bit_cast(u32x2, v0), b = __builtin_bit_cast(u32x2, v1);
    u32x4 r;
    r[0] = a[0]; r[1] = a[1]; r[2] = b[0]; r[3] = b[1];
    return r;
}

// Tiles of 128 16-bit columns (256-byte rows, no padding) store 16-byte chunk
// j of row r at chunk j ^ swz128(r).  A 16-byte read of rows r0 .. r0+15 at
// one chunk (the MFMA A operand, one row per lane) then meets 16 distinct
// chunks, and a transposed read of 4 consecutive rows (from a multiple of 4)
// over 4 chunks of one aligned group meets 4 distinct groups: both fill the
// 64 banks without conflict, where a padded row pitch serves only one of them.
// In the D=128 key-tile kernel: 343 -> 306 us on B2 H16 S4096 bf16 causal,
// 390 -> 355 us on 8 packed sequences x 32 heads.  (A 160-column pitch with
// the swap confined to each group of four chunks, whose addresses stay
// immediate offsets, gave 330 us; in the dQ pass, at 252 of 256 registers,
// either form spills.)
__device__ __forceinline__ int swz128(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }
__device__ __forceinline__ int swz128_col(int r, int col) { return (((col >> 3) ^ swz128(r)) << 3) | (col & 7); }

// ld_tr on a swizzled 128-column tile.
template <bool ACC>
__device__ __forceinline__ u32x4 ld_tr_swz128(const uint16_t* X, int k0, int n0, int lane) {
    const int p = lane & 15, grp = lane >> 4;
    const int g = grp >> 1, cb = (grp & 1) * 16;
    const int kr0 = (ACC ? (k0 + 4 * g) : (k0 + 8 * g)) + (p >> 2);
    const int kr1 = (ACC ? (k0 + 8 + 4 * g) : (k0 + 8 * g + 4)) + (p >> 2);
    const int col = n0 + cb + 4 * (p & 3);
    const s16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(X + kr0 * 128 + swz128_col(kr0, col)));
    const s16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(X + kr1 * 128 + swz128_col(kr1, col)));
    const u32x2 a = __builtin_bit_cast(u32x2, v0), b = __builtin_bit_cast(u32x2, v1);
    u32x4 r;
    r[0] = a[0]; r[1] = a[1]; r[2] = b[0]; r[3] = b[1];
    return r;
}

// The same for v_mfma_f32_16x16x32 operands: 16-lane group G = lane / 16 holds
// k = k0 + 8*G + t (t = 0..7) of column n0 + lane % 16.  (16x16 C tiles: lane
// holds column lane % 16, rows 4*G + r in register r.)
__device__ __forceinline__ u32x4 ld_tr16x16(const uint16_t* X, int ld, int k0, int n0, int lane) {
    const int p = lane & 15, G = lane >> 4;
    const int col = n0 + 4 * (p & 3);
    const s16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(X + (k0 + 8 * G + (p >> 2)) * ld + col));
    const s16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(X + (k0 + 8 * G + 4 + (p >> 2)) * ld + col));
    const u32x2 a = __builtin_bit_cast(u32x2, v0), b = __builtin_bit_cast(u32x2, v1);
    u32x4 r;
    r[0] = a[0]; r[1] = a[1]; r[2] = b[0]; r[3] = b[1];
    return r;
}

// 16x16x32 operand in "acc slots" order: k = k0 + 4*G + t (t < 4) and
// k0 + 16 + 4*G + (t - 4) (t >= 4): the rows two 16x16 C tiles (k0.., k0+16..)
// hold in one lane, so their pair feeds the B operand of the next product.
__device__ __forceinline__ u32x4 ld_tr16x16_acc(const uint16_t* X, int ld, int k0, int n0, int lane) {
    const int p = lane & 15, G = lane >> 4;
    const int col = n0 + 4 * (p & 3);
    const s16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(X + (k0 + 4 * G + (p >> 2)) * ld + col));
    const s16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(X + (k0 + 16 + 4 * G + (p >> 2)) * ld + col));
    const u32x2 a = __builtin_bit_cast(u32x2, v0), b = __builtin_bit_cast(u32x2, v1);
    u32x4 r;
    r[0] = a[0]; r[1] = a[1]; r[2] = b[0]; r[3] = b[1];
    return r;
}

__device__ __forceinline__ f32x16 zero16() {
    f32x16 z;
#pragma unroll
    for (int i = 0; i < 16; ++i) z[i] = 0.f;
    return z;
}

__device__ __forceinline__ f32x4 zero4() {
    f32x4 z = {0.f, 0.f, 0.f, 0.f};
    return z;
}

// ---------------------------------------------------------------------------
// Parameter blocks (passed by value as kernel arguments)
// ---------------------------------------------------------------------------

constexpr int kMaxSeqArgs = 64;

// Strided 16-bit tensor; the innermost (D) stride is 1.
struct TensorArg {
    uint16_t* p;
    int64_t sb, sh, ss;   // dense: batch/head/row strides; packed: sb = 0, ss = token stride
};

// Sequence table.  Dense problems use n = B with q0 = k0 = 0 and the batch
// stride; packed problems use sb = 0 and the per-sequence first rows.
struct SeqTable {
    int32_t n;
    int32_t q0[kMaxSeqArgs], k0[kMaxSeqArgs], lq[kMaxSeqArgs], lk[kMaxSeqArgs];
    const int32_t* dev;   // when n > kMaxSeqArgs: device array of 4*n ints (q0, k0, lq, lk)
};

// The values are uniform across the workgroup; readfirstlane keeps them (and
// everything derived from them, such as loop bounds) in scalar registers.
__device__ __forceinline__ void seq_get(const SeqTable& t, int b, int& q0, int& k0, int& lq, int& lk) {
    if (t.dev) {
        q0 = t.dev[4 * b + 0]; k0 = t.dev[4 * b + 1]; lq = t.dev[4 * b + 2]; lk = t.dev[4 * b + 3];
    } else {
        q0 = t.q0[b]; k0 = t.k0[b]; lq = t.lq[b]; lk = t.lk[b];
    }
    q0 = __builtin_amdgcn_readfirstlane(q0);
    k0 = __builtin_amdgcn_readfirstlane(k0);
    lq = __builtin_amdgcn_readfirstlane(lq);
    lk = __builtin_amdgcn_readfirstlane(lk);
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

// The key-tile kernel's order.  Units (sequence, KV head) share Q and dO;
// items are a unit's key tiles, longest causal range first.  With n_unit a
// multiple of 8, unit u runs on XCD u % 8, and each XCD takes its units in
// groups of kXcdGroup: all items of a group, item-major across its units,
// before the next group, so that the workgroups an XCD runs at once read few
// units' rows from its L2.  Packed sequences come sorted by decreasing length
// (the host sorts them), so the longest units go first.  Plain order (units
// fastest) otherwise.  A bijection on [0, n_unit * n_item).  With four units
// per XCD (B2 H16 S4096) a group is the whole XCD share and the order is the
// plain one.  On 8 packed sequences x 32 heads (32 units per XCD) it cut the
// kernel's HBM reads from 1121 to 336 MB per launch (FETCH_SIZE); the time
// stayed 387-391 us, which the one-wavefront-per-SIMD kernel spends on
// latency, not bandwidth.  Groups of 2 were slower (401 us), of 8 the same.
constexpr int kXcdGroup = 4;
__device__ __forceinline__ void xcd_group_order(int n_unit, int n_item, int L, int& unit, int& item) {
    if (n_unit & 7) {
        unit = L % n_unit;
        item = L / n_unit;
        return;
    }
    const int xcd = L & 7, slot = L >> 3;
    const int per_xcd = n_unit >> 3;
    const int gi = slot / (kXcdGroup * n_item), s = slot % (kXcdGroup * n_item);
    const int gu = min(kXcdGroup, per_xcd - gi * kXcdGroup);   // units in this group
    item = s / gu;
    unit = (gi * kXcdGroup + s % gu) * 8 + xcd;
}

struct FwdParams {
    TensorArg q, k, v, o;
    float* lse; int64_t lse_sb, lse_sh, lse_ss;
    int B, Hq, Hkv, Sq, Sk;   // packed: B = sequences of this launch, Sq/Sk unused
    float scale_log2;
    int varlen;               // rows of sequence b: tokens seqs.q0[b] .. + seqs.lq[b]
    SeqTable seqs;
};

// Row statistics workspace layout: row index R of (b, h, i)
//   dense:  R = (b*Hq + h)*Sq + i        packed: R = (q0 + i)*Hq + h
// fp32 dQ accumulator rows (D floats each), head-major in both cases so that
// consecutive query rows of one head are adjacent:
//   dense:  A = (b*Hq + h)*Sq + i        packed: A = h*Tq + q0 + i
struct BwdParams {
    TensorArg q, k, v, o, dout, dq, dk, dv;
    // user statistics
    int32_t stats_kind;
    const float* st_a; const float* st_b; int64_t st_sb, st_sh, st_ss;
    // workspace
    float* lse2;      // [R] LSE * log2(e), +inf for rows without keys
    float* delta;     // [R] sum_d dO*O
    float* dqacc;     // [R][D] fp32 dQ accumulator (unscaled)
    int B, Hq, Hkv, Sq, Sk;   // Sq/Sk: dense lengths (packed: Tq/Tk totals)
    int64_t rows;             // number of statistics rows R
    int varlen;
    int grad_f32;             // dQ, dK, dV are fp32 (else the input dtype)
    SeqTable seqs;
    float scale, scale_log2;
};

}  // namespace sdpa
