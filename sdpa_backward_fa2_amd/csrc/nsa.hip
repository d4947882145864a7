// NSA selected-attention backward (aclnnNsaSelectedAttentionGrad) for gfx950.
//
// For query token t and KV head h2 the keys are the block_count blocks of
// block_size rows that topk[t, h2, :] names, gathered with repetition (the
// operator page's Gather over 0 <= i < selectedBlockCount, "Formula" section);
// the gradients are the page's dV = P^T dY, dQ = dS K / sqrt(d),
// dK = dS^T Q / sqrt(d) over those keys.  Q and K have head dim DK, V, O and
// dY head dim DV (the page: 192 or 128, unequal allowed); S, dQ and dK
// contract or produce DK columns, dP, dV and O DV columns.  Gradients are
// stored in the input type or fp32.
//
// Kernels, all on the caller's stream:
//   nsa_rank_kernel          per (token tile, KV head): each (token, slot)
//                            entry's rank within its tile and block, and the
//                            tile's per-block totals (LDS counters, no atomics);
//                            in the backward nsa_rank_pre_kernel, which also
//                            runs the row pass (Delta and log2-LSE per
//                            (token, head))
//   nsa_hist_scan_kernel     per (KV block, KV head): prefixes of those totals
//                            over the tiles, and the block's entry count
//   nsa_scan_kernel          CSR offsets of the lists and a table of work
//                            pieces (at most `chunk` entries of one block each)
//   nsa_scatter_kernel       stores each entry in its block's list, which so
//                            comes out in (token, slot) order; up to 4096
//                            buckets nsa_scan_scatter_kernel does the scan too
//   nsa_kv_kernel            per piece and 64-key half of its block: dK, dV
//                            over the piece's tokens (G heads per token form
//                            the query rows of a step); a block with one piece
//                            writes dK/dV, otherwise an fp32 partial
//   nsa_kv_reduce_kernel     sums the partials of multi-piece blocks in piece
//                            order (deterministic); zero-fills unselected blocks
//   nsa_dq_kernel            per (token, KV head, 16-head tile): dQ over the
//                            gathered keys, without atomics
//   nsa_dq_ds_kernel         16 query heads per KV head: dQ
//                            from the dS that nsa_kv_kernel stored (K gathered,
//                            S and dP not recomputed)
//   nsa_fwd_kernel           the forward: O and (max, sum) per (token, head)
//                            over the gathered keys, same tiling as nsa_dq
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <string>
#include <type_traits>
#include <vector>

#include "../../include/sdpa_bwd.h"
#include "bwd_shared.h"
#include "common.h"
#include "kernels.h"
#include "prof.h"

namespace sdpa {

typedef int i32x4 __attribute__((ext_vector_type(4)));

struct NsaParams {
    const int32_t* topk;
    int64_t tk_st, tk_sn, tk_sk;
    int count, bs, N2, NB, G, Hq;
    int g_mul;            // ceil(2^16 / G): r / G == (r * g_mul) >> 16 for 0 <= r < 256
    int chunk;            // entries per work piece
    int max_pieces;
    SeqTable seqs;        // per sequence: first query row, first key row, lengths
    int32_t* counts;      // [N2*NB]
    int32_t* offsets;     // [N2*NB + 1]
    int32_t* entries;     // [Tq*N2*count]
    int32_t* pstart;      // [N2*NB + 1] first piece of each bucket
    int32_t* pieces;      // [max_pieces][3]: bucket, first entry, end entry
    int tt, n_tiles;      // index build: tokens per tile, tiles (ceil(Tq / tt))
    int32_t* hist;        // [N2][NB][n_tiles] per-tile block totals, then their prefixes
    int32_t* rank;        // [N2][Tq * count] entry ranks within their tile and block; after the
                          // scatter, each entry's position in the entries array (-1: none)
    // backward
    TensorArg q, k, v, dout, dq, dk, dv;
    const float* lse2;
    const float* delta;
    float* partial;       // [max_pieces][halves][64][D] for dK then dV
    // stored dS (16 query heads per KV head, Dqk = Dv = 128; null: the dQ
    // kernel recomputes it): [entry position][key of the block][16 heads in
    // the order 0-3, 8-11, 4-7, 12-15], 16-bit
    uint16_t* ds;
    int halves;           // ceil(bs / 64)
    int sparse_mode;
    int t_base;           // forward: first token of this launch (grid x counts from it)
    // optional user mask over (sequence-local query, sequence-local key)
    // positions, nonzero = masked out; rows mask_ss bytes apart, 16-byte
    // aligned, shared by every sequence and head (null: none)
    const uint8_t* mask;
    int64_t mask_ss;
    int Tq;
    int grad_f32;         // dQ, dK, dV are fp32 (else the input dtype)
    float scale, scale_log2;
    // forward outputs
    TensorArg o;
    float* m_out;         // softmax max of the scaled scores, natural units
    float* l_out;         // sum of exp(score - max)
    int64_t st_ss, st_sh; // token and head strides of m_out / l_out
};

// Bit i of the result is set when byte i of the 16 is nonzero.
__device__ __forceinline__ uint32_t mask_bits16(u32x4 v) {
    uint32_t r = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        uint32_t t = v[i] | (v[i] >> 4);
        t |= t >> 2;
        t |= t >> 1;
        // bit 0 of each byte is now "byte != 0"; the multiply gathers the
        // four into bits 24..27 (no two partial products meet below 2^32)
        r |= (((t & 0x01010101u) * 0x01020408u) >> 24 & 0xFu) << (4 * i);
    }
    return r;
}

// Sequence table access.  Up to kMaxSeqArgs sequences travel in the kernel
// arguments; more live in the workspace as int4 (q0, k0, lq, lk) rows, filled
// by nsa_seqtab_kernel at the start of the call.
struct SeqRow {
    int q0, k0, lq, lk;
};

__device__ __forceinline__ SeqRow seq_row(const SeqTable& s, int i) {
    if (s.dev) {
        const i32x4 v = *reinterpret_cast<const i32x4*>(s.dev + 4 * i);
        return SeqRow{v[0], v[1], v[2], v[3]};
    }
    return SeqRow{s.q0[i], s.k0[i], s.lq[i], s.lk[i]};
}

// The sequence holding position x of the packed query (F = 0) or key (F = 1)
// rows, or -1.  Starts are non-decreasing and each sequence ends where the
// next starts, so it is the last sequence starting at or before x, provided x
// lies before its end.
template <int F>
__device__ __forceinline__ int seq_of(const SeqTable& s, int x) {
    if (s.dev) {
        int lo = 0, hi = s.n - 1, r = -1;
        while (lo <= hi) {
            const int mid = (lo + hi) >> 1;
            if (s.dev[4 * mid + F] <= x) { r = mid; lo = mid + 1; }
            else hi = mid - 1;
        }
        if (r >= 0 && x >= s.dev[4 * r + F] + s.dev[4 * r + 2 + F]) r = -1;
        return r;
    }
    int r = -1;
    for (int i = 0; i < s.n; ++i) {
        const int a = F ? s.k0[i] : s.q0[i], n = F ? s.lk[i] : s.lq[i];
        if (x >= a && x < a + n) r = i;
    }
    return r;
}

__device__ __forceinline__ int seq_of_block(const SeqTable& s, int key_row) { return seq_of<1>(s, key_row); }
__device__ __forceinline__ int seq_of_token(const SeqTable& s, int t) { return seq_of<0>(s, t); }

// Writes rows first .. first + chunk.n - 1 of the workspace sequence table.
#ifndef SDPA_NSA_KV_UNIT
__global__ __launch_bounds__(64) void nsa_seqtab_kernel(SeqTable chunk, int32_t* table, int first) {
    const int i = threadIdx.x;
    if (i >= chunk.n) return;
    i32x4 v;
    v[0] = chunk.q0[i]; v[1] = chunk.k0[i]; v[2] = chunk.lq[i]; v[3] = chunk.lk[i];
    *reinterpret_cast<i32x4*>(table + 4 * (first + i)) = v;
}
#endif


// ---------------------------------------------------------------------------
// Inverse index: a stable counting sort of the (token, slot) entries by block
// ---------------------------------------------------------------------------
//
// The entries e = t * count + slot of KV head h2 are cut into tiles of p.tt
// consecutive tokens.  nsa_rank_kernel (one wavefront per tile and head)
// walks its tile in entry order, 64 entries a step, with one LDS counter per
// block: each entry's rank among the tile's earlier entries naming the same
// block is the counter plus the number of lower lanes of its step that name
// it (a match mask built from one ballot per bit of the block number).  It
// writes the ranks and the tile's per-block totals hist[h2][g][tile].
// nsa_hist_scan_kernel turns each block's row of tile totals into exclusive
// prefixes and the block's count; nsa_scan_kernel makes the CSR offsets and
// the work pieces; nsa_scatter_kernel stores each entry at offset + tile
// prefix + rank.  Every list comes out in (token, slot) order
// without atomics, in work linear in the entries plus blocks x tiles.

constexpr int kIdxWin = 4096;   // block counters per pass of the rank kernel
constexpr int kIdxBatch = 4;    // tile steps whose top-k values are loaded together

// The top-k value of entry c + lane of a tile step (e_end: the tile's end;
// lanes past it read the tile's last entry).
__device__ __forceinline__ int step_choice(const NsaParams& p, const int32_t* tk, int c, int e_end, int lane) {
    const int e = min(c + lane, e_end - 1);
    const int t = (int)((uint32_t)e / (uint32_t)p.count);
    const int slot = e - t * p.count;
    return tk[(int64_t)t * p.tk_st + (int64_t)slot * p.tk_sk];
}

// The global block that value v of entry c + lane names, or -1 past the
// tile's end or when v is not a block of the token's sequence.  s_cur
// (uniform) is moved past the sequences that end at or before the step's
// first token; sequences partition the packed tokens.
__device__ __forceinline__ int step_block(const NsaParams& p, int v, int c, int e_end, int lane, int& s_cur) {
    const int e = min(c + lane, e_end - 1);
    const int t = (int)((uint32_t)e / (uint32_t)p.count);
    const int t_first = (int)((uint32_t)c / (uint32_t)p.count);
    const int t_last = (int)((uint32_t)min(c + 63, e_end - 1) / (uint32_t)p.count);
    while (s_cur + 1 < p.seqs.n) {
        const SeqRow r = seq_row(p.seqs, s_cur);
        if (r.q0 + r.lq > t_first) break;
        ++s_cur;
    }
    int g = -1;
    for (int s = s_cur; s < p.seqs.n; ++s) {
        const SeqRow r = seq_row(p.seqs, s);
        if (r.q0 > t_last) break;
        if (t >= r.q0 && t < r.q0 + r.lq && v >= 0 && v < r.lk / p.bs) g = r.k0 / p.bs + v;
    }
    return c + lane < e_end ? g : -1;
}

__device__ __forceinline__ void rank_body(const NsaParams& p, int tile, int h2) {
    __shared__ int cnt[kIdxWin];
    const int lane = threadIdx.x;
    const int t0 = tile * p.tt, t1 = min(p.Tq, t0 + p.tt);
    const int e_begin = t0 * p.count, e_end = t1 * p.count;
    const int sa = seq_of_token(p.seqs, t0), sb = seq_of_token(p.seqs, t1 - 1);
    // the blocks of the sequences the tile touches
    const int gA = seq_row(p.seqs, sa).k0 / p.bs;
    const SeqRow rb = seq_row(p.seqs, sb);
    const int gB = (rb.k0 + rb.lk) / p.bs;
    const int32_t* tk = p.topk + (int64_t)h2 * p.tk_sn;
    int32_t* rank = p.rank + (int64_t)h2 * p.Tq * p.count;
    int32_t* hist = p.hist + (int64_t)h2 * p.NB * p.n_tiles;
    const unsigned long long below = (1ull << lane) - 1ull;
    for (int w0 = gA; w0 < gB; w0 += kIdxWin) {
        const int nw = min(gB - w0, kIdxWin);
        int bits = 0;
        while ((1 << bits) < nw) ++bits;
        for (int i = lane; i < nw; i += 64) cnt[i] = 0;
        __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
        int s_cur = sa;
        for (int cb = e_begin; cb < e_end; cb += 64 * kIdxBatch) {
            int v[kIdxBatch];
#pragma unroll
            for (int u = 0; u < kIdxBatch; ++u) v[u] = step_choice(p, tk, min(cb + 64 * u, e_end - 1), e_end, lane);
#pragma unroll
            for (int u = 0; u < kIdxBatch; ++u) {
                const int c = cb + 64 * u;
                if (c >= e_end) break;
                const int g = step_block(p, v[u], c, e_end, lane, s_cur);
                const int key = g - w0;
                const bool mine = g >= w0 && key < nw;
                unsigned long long m = __ballot(mine);
                for (int b = 0; b < bits; ++b) {
                    const bool on = (key >> b) & 1;
                    const unsigned long long hb = __ballot(mine && on);
                    m &= on ? hb : ~hb;
                }
                // one wavefront: its LDS reads and writes take effect in program order
                if (mine) {
                    const int old = cnt[key];
                    const int before = __popcll(m & below);
                    if (before == 0) cnt[key] = old + __popcll(m);
                    rank[c + lane] = old + before;
                }
                __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
            }
        }
        for (int i = lane; i < nw; i += 64) hist[(int64_t)(w0 + i) * p.n_tiles + tile] = cnt[i];
        __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    }
}

#ifndef SDPA_NSA_KV_UNIT
__global__ __launch_bounds__(64) void nsa_rank_kernel(NsaParams p) {
    rank_body(p, blockIdx.x, blockIdx.y);
}
#endif


// The rank pass and the backward's row pass (Delta and log2-LSE of every
// (token, head) row, which the index does not need) in one launch: the rank
// items first, then row-pass items of 64 threads.
template <class T, int DV>
__global__ __launch_bounds__(64) void nsa_rank_pre_kernel(NsaParams p, BwdParams bp, int n_rank) {
    const int id = blockIdx.x;
    if (id < n_rank) rank_body(p, id % p.n_tiles, id / p.n_tiles);
    else row_pass_rows<T, DV, 64>(bp, 0, id - n_rank, 0);
}

// One wavefront, one (block, KV head) = bucket: exclusive prefixes over the
// tiles of the block's sequence, in place; returns the block's entry count
// (in every lane).
__device__ __forceinline__ int hist_scan_bucket(const NsaParams& p, int bucket, int lane) {
    const int g = bucket % p.NB;
    const int s = seq_of_block(p.seqs, g * p.bs);
    const SeqRow r = seq_row(p.seqs, s < 0 ? 0 : s);
    if (s < 0 || r.lq == 0) return 0;
    const int ta = r.q0 / p.tt, tb = (r.q0 + r.lq - 1) / p.tt + 1;
    int32_t* h = p.hist + (int64_t)bucket * p.n_tiles;
    // each lane takes a run of consecutive tiles
    const int per = (tb - ta + 63) / 64;
    const int a = min(tb, ta + lane * per), b = min(tb, a + per);
    int sum = 0;
    for (int i = a; i < b; ++i) sum += h[i];
    int x = sum;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(x, o);
        if (lane >= o) x += y;
    }
    int run = x - sum;
    for (int i = a; i < b; ++i) {
        const int v = h[i];
        h[i] = run;
        run += v;
    }
    return __shfl(x, 63);
}

#ifndef SDPA_NSA_KV_UNIT
__global__ __launch_bounds__(64) void nsa_hist_scan_kernel(NsaParams p) {
    const int bucket = blockIdx.y * p.NB + blockIdx.x;
    const int n = hist_scan_bucket(p, bucket, threadIdx.x);
    if (threadIdx.x == 0) p.counts[bucket] = n;
}
#endif


// One wavefront per (tile, KV head): entry e goes to offset + tile prefix +
// rank of its block's list (off: the KV head's CSR offsets).
__device__ __forceinline__ void scatter_body(const NsaParams& p, int tile, int h2, const int32_t* off) {
    const int lane = threadIdx.x;
    const int t0 = tile * p.tt, t1 = min(p.Tq, t0 + p.tt);
    const int e_begin = t0 * p.count, e_end = t1 * p.count;
    const int32_t* tk = p.topk + (int64_t)h2 * p.tk_sn;
    int32_t* rank = p.rank + (int64_t)h2 * p.Tq * p.count;
    const int32_t* hist = p.hist + (int64_t)h2 * p.NB * p.n_tiles;
    int s_cur = seq_of_token(p.seqs, t0);
    for (int cb = e_begin; cb < e_end; cb += 64 * kIdxBatch) {
        int v[kIdxBatch], rk[kIdxBatch], g[kIdxBatch], pos[kIdxBatch];
#pragma unroll
        for (int u = 0; u < kIdxBatch; ++u) {
            const int c = min(cb + 64 * u, e_end - 1);
            v[u] = step_choice(p, tk, c, e_end, lane);
            rk[u] = rank[min(c + lane, e_end - 1)];
        }
#pragma unroll
        for (int u = 0; u < kIdxBatch; ++u)
            g[u] = cb + 64 * u < e_end ? step_block(p, v[u], cb + 64 * u, e_end, lane, s_cur) : -1;
#pragma unroll
        for (int u = 0; u < kIdxBatch; ++u)
            pos[u] = g[u] >= 0 ? off[g[u]] + hist[(int64_t)g[u] * p.n_tiles + tile] + rk[u] : -1;
#pragma unroll
        for (int u = 0; u < kIdxBatch; ++u) {
            const int e = cb + 64 * u + lane;
            if (g[u] >= 0) p.entries[pos[u]] = e;
            // each entry's list position replaces its rank (read above by
            // this lane only): the stored-dS dQ kernel finds its dS by it
            if (e < e_end) rank[e] = pos[u];
        }
    }
}

#ifndef SDPA_NSA_KV_UNIT
__global__ __launch_bounds__(64) void nsa_scatter_kernel(NsaParams p) {
    scatter_body(p, blockIdx.x, blockIdx.y, p.offsets + blockIdx.y * p.NB);
}
#endif


// Index builds of at most kScanScatterMax buckets: the offsets scan rides in
// the scatter launch.  Every workgroup scans the buckets' entry counts itself
// (a run of consecutive buckets per lane) into LDS offsets, and workgroup
// (0, 0) also writes the CSR offsets, the pieces' starts and the work pieces,
// which the kernels after the index build read.
constexpr int kScanScatterMax = 4096;
#ifndef SDPA_NSA_KV_UNIT
__global__ __launch_bounds__(64) void nsa_scan_scatter_kernel(NsaParams p) {
    __shared__ int32_t off_s[kScanScatterMax];
    const int lane = threadIdx.x;
    const int nb = p.N2 * p.NB;
    const int per = (nb + 63) / 64;
    const int a = min(nb, lane * per), b = min(nb, a + per);
    int sum = 0, psum = 0;
    for (int i = a; i < b; ++i) {
        const int c = p.counts[i];
        sum += c;
        psum += (c + p.chunk - 1) / p.chunk;
    }
    int x = sum, y = psum;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int xs = __shfl_up(x, o), ys = __shfl_up(y, o);
        if (lane >= o) {
            x += xs;
            y += ys;
        }
    }
    int run = x - sum, prun = y - psum;
    const bool writer = blockIdx.x == 0 && blockIdx.y == 0;
    for (int i = a; i < b; ++i) {
        const int c = p.counts[i];
        off_s[i] = run;
        if (writer) {
            const int np = (c + p.chunk - 1) / p.chunk;
            p.offsets[i] = run;
            p.pstart[i] = prun;
            for (int k = 0; k < np; ++k) {
                p.pieces[(prun + k) * 3 + 0] = i;
                p.pieces[(prun + k) * 3 + 1] = run + k * p.chunk;
                p.pieces[(prun + k) * 3 + 2] = min(run + (k + 1) * p.chunk, run + c);
            }
            prun += np;
        }
        run += c;
    }
    const int total = __shfl(x, 63), ptotal = __shfl(y, 63);
    if (writer && lane == 0) {
        p.offsets[nb] = total;
        p.pstart[nb] = ptotal;
    }
    __syncthreads();
    scatter_body(p, blockIdx.x, blockIdx.y, off_s + blockIdx.y * p.NB);
}
#endif


// Block-wide exclusive scan of one value per thread (1024 threads); returns the
// exclusive prefix and writes the block total to *total.
__device__ __forceinline__ int block_exclusive_scan(int x, int* wsum, int* total) {
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    int v = x;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(v, o);
        if (lane >= o) v += y;
    }
    if (lane == 63) wsum[w] = v;
    __syncthreads();
    if (tid == 0) {
        int acc = 0;
        for (int i = 0; i < 16; ++i) {
            const int t = wsum[i];
            wsum[i] = acc;
            acc += t;
        }
        wsum[16] = acc;
    }
    __syncthreads();
    const int r = v - x + wsum[w];
    *total = wsum[16];
    __syncthreads();
    return r;
}

#ifndef SDPA_NSA_KV_UNIT
__global__ __launch_bounds__(1024) void nsa_scan_kernel(NsaParams p) {
    __shared__ int wsum[17];
    const int nb = p.N2 * p.NB;
    int carry_e = 0, carry_p = 0;
    for (int c0 = 0; c0 < nb; c0 += 1024) {
        const int i = c0 + threadIdx.x;
        const int cnt = i < nb ? p.counts[i] : 0;
        const int np = (cnt + p.chunk - 1) / p.chunk;
        int te, tp;
        const int oe = block_exclusive_scan(cnt, wsum, &te);
        const int op = block_exclusive_scan(np, wsum, &tp);
        if (i < nb) {
            const int off = carry_e + oe, ps = carry_p + op;
            p.offsets[i] = off;
            p.pstart[i] = ps;
            for (int k = 0; k < np; ++k) {
                p.pieces[(ps + k) * 3 + 0] = i;
                p.pieces[(ps + k) * 3 + 1] = off + k * p.chunk;
                p.pieces[(ps + k) * 3 + 2] = min(off + (k + 1) * p.chunk, off + cnt);
            }
        }
        carry_e += te;
        carry_p += tp;
    }
    if (threadIdx.x == 0) {
        p.offsets[nb] = carry_e;
        p.pstart[nb] = carry_p;
    }
}
#endif


// ---------------------------------------------------------------------------
// dK / dV: key-block outer over pieces of the inverse lists
// ---------------------------------------------------------------------------
//
// Workgroup of four wavefronts: wavefront w = kw + 2*rh owns keys 32*kw .. +31
// of the 64-key half and rows 32*rh .. +31 of each 64-row step.  A step packs
// E = 64 / G consecutive entries of the list; row r is head r % G of the token
// of entry r / G.  The rest mirrors the dense main kernel: S and dP on MFMA,
// P and dS on the vector ALU, dV^T += dO^T P and dK^T += Q^T dS with the
// transposed operands read by ds_read_b64_tr_b16.

// UM: with a user attention mask (a separate instance, so that the mask's
// staging registers do not weigh on the unmasked kernel).
template <class T, int DK, int DV, bool UM>
__global__ __launch_bounds__(256) void nsa_kv_kernel(NsaParams p) {
    // DK: head dim of Q and K; DV: of V, O and dO.  Rows per step: 128 at
    // DK = DV = 128 (each wavefront takes two 32-row blocks of its 64-row
    // half, so a step's barrier and loads cover twice the products), 64
    // otherwise (D=64: two workgroups per CU; DK=192: the tiles' LDS)
    constexpr int BR = (DK == 128 && DV == 128) ? 128 : 64;
    constexpr int NSB = BR / 64;               // 32-row blocks per wavefront and step
    constexpr int KSK = DK / 16, KSV = DV / 16;   // k-steps of S (over DK) and of dP (over DV)
    constexpr int KSM = KSK > KSV ? KSK : KSV;
    constexpr int DBK = DK / 32, DBV = DV / 32;   // 32-column blocks of dK and of dV
    constexpr int DBM = DBK > DBV ? DBK : DBV;
    constexpr int QPK = DK + 8, QPV = DV + 8;     // LDS row pitches of the Q and dO tiles
    constexpr int CHK = BR * DK / 8 / 256, CHV = BR * DV / 8 / 256;
    constexpr int TILES_B = 2 * BR * (QPK + QPV) * 2;       // Q and dO, double-buffered
    constexpr int RED_B = 2 * (DBK + DBV) * 16 * 64 * 4;   // dK/dV partials of two wavefronts
    constexpr int ARENA = TILES_B > RED_B ? TILES_B : RED_B;
    __shared__ __align__(16) unsigned char arena[ARENA];
    __shared__ __align__(16) float lse_s[2][BR];
    __shared__ __align__(16) float dlt_s[2][BR];
    __shared__ int tl_s[2][BR];          // sequence-local token position of each row
    __shared__ uint64_t mbits_s[UM ? 2 : 1][UM ? BR : 1];  // user mask: bit j = key j of this half masked
    __shared__ int tok_s[2048];          // token of each entry of the piece (<= 2048 / G entries)
    typedef uint16_t TileQ[BR * QPK];
    typedef uint16_t TileO[BR * QPV];
    TileQ* Qs = reinterpret_cast<TileQ*>(arena);
    TileO* dOs = reinterpret_cast<TileO*>(arena + 2 * BR * QPK * 2);

    const int piece = blockIdx.x;
    if (piece >= p.pstart[p.N2 * p.NB]) return;
    const int tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6;
    const int kw = w & 1, rh = w >> 1;
    const int g = lane >> 5, c = lane & 31;
    const int bucket = p.pieces[piece * 3 + 0];
    const int eb = p.pieces[piece * 3 + 1], ee = p.pieces[piece * 3 + 2];
    const int h2 = bucket / p.NB, blk = bucket % p.NB;
    const int half = blockIdx.y;
    const int kb0 = half * 64;                  // first key of this half inside the block
    if (kb0 >= p.bs) return;
    const int nkeys = min(64, p.bs - kb0);
    const int s_idx = seq_of_block(p.seqs, blk * p.bs);
    const SeqRow srow_info = seq_row(p.seqs, s_idx);
    const int blk_local = blk - srow_info.k0 / p.bs;
    const int key_row0 = blk * p.bs + kb0;      // packed KV row of key 0 of this half
    const int kpos0 = blk_local * p.bs + kb0;   // its sequence-local position

    const int myk = 32 * kw + c;
    const bool col_ok = myk < nkeys;
    u32x4 kreg[KSK], vreg[KSV];
    const uint16_t* kp = p.k.p + h2 * p.k.sh + (int64_t)(key_row0 + myk) * p.k.ss;
    const uint16_t* vp = p.v.p + h2 * p.v.sh + (int64_t)(key_row0 + myk) * p.v.ss;
#pragma unroll
    for (int s = 0; s < KSM; ++s) {
        u32x4 z = {0u, 0u, 0u, 0u};
        if (s < KSK) kreg[s] = col_ok ? ld16(kp + 16 * s + 8 * g) : z;
        if (s < KSV) vreg[s] = col_ok ? ld16(vp + 16 * s + 8 * g) : z;
    }
    f32x16 dva[DBV], dka[DBK];
#pragma unroll
    for (int db = 0; db < DBV; ++db) dva[db] = zero16();
#pragma unroll
    for (int db = 0; db < DBK; ++db) dka[db] = zero16();

    const int E = max(1, BR / p.G);             // entries per step
    const int n_steps = (ee - eb + E - 1) / E;
    const int q0s = srow_info.q0;

    // The tokens of the piece's entries go to LDS once, so that a step's
    // row addresses need no dependent global load.
    const int n_e = ee - eb;                    // >= 1: pieces are never empty
    for (int i = tid; i < n_e; i += 256) tok_s[i] = p.entries[eb + i] / p.count;
    __syncthreads();

    // Row r of step st is head r % G of entry st*E + r/G.  Loads are
    // unconditional: padding rows re-read the piece's last entry and are
    // given LSE = +inf when stored, so their P is exactly zero; nothing loaded
    // is used before store_tile.
    u32x4 pq[CHK], pdo[CHV];
    u32x4 pm[UM ? 4 : 1];                       // user mask bytes of the row's 64 keys
    float pl = INFINITY, pd = 0.f;
    int ptl = 0;
    bool pok = false;
    // row r of a tile: entry r / G, head r % G (r < 256, G <= 32: a multiply
    // and shift divide exactly)
    auto div_g = [&](int r) { return (r * p.g_mul) >> 16; };
    // token and head strides are below 2^23 elements: 32 x 32 -> 64-bit products
    const int qss = (int)p.q.ss, qsh = (int)p.q.sh, dss = (int)p.dout.ss, dsh = (int)p.dout.sh;
    auto load_tile = [&](int st) {
#pragma unroll
        for (int x = 0; x < CHK; ++x) {
            const int e = tid + 256 * x;
            const int r = e / (DK / 8), cc = (e % (DK / 8)) * 8;
            const int rq = div_g(r);
            const int t = tok_s[min(st * E + rq, n_e - 1)];
            const int h = h2 * p.G + r - rq * p.G;
            pq[x] = ld16(p.q.p + ((int64_t)t * qss + (int64_t)h * qsh + cc));
            if constexpr (DK == DV) pdo[x] = ld16(p.dout.p + ((int64_t)t * dss + (int64_t)h * dsh + cc));
        }
        if constexpr (DK != DV) {
#pragma unroll
            for (int x = 0; x < CHV; ++x) {
                const int e = tid + 256 * x;
                const int r = e / (DV / 8), cc = (e % (DV / 8)) * 8;
                const int rq = div_g(r);
                const int t = tok_s[min(st * E + rq, n_e - 1)];
                const int h = h2 * p.G + r - rq * p.G;
                pdo[x] = ld16(p.dout.p + ((int64_t)t * dss + (int64_t)h * dsh + cc));
            }
        }
        {
            const int r = tid & (BR - 1);
            const int rq = div_g(r);
            const int li = st * E + rq;
            const int t = tok_s[min(li, n_e - 1)];
            const int h = h2 * p.G + r - rq * p.G;
            pl = p.lse2[(int64_t)t * p.Hq + h];
            pd = p.delta[(int64_t)t * p.Hq + h];
            ptl = t - q0s;
            pok = r < E * p.G && li < n_e;
            if constexpr (UM) {
              if (tid < BR) {
                // 16-byte pieces of the row's mask bytes for this half's keys
                // (kpos0 and the row stride are multiples of 16; nkeys is too)
                const u32x4* mp = reinterpret_cast<const u32x4*>(p.mask + (int64_t)ptl * p.mask_ss + kpos0);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const u32x4 z = {0u, 0u, 0u, 0u};
                    pm[j] = 16 * j < nkeys ? mp[j] : z;
                }
              }
            }
        }
    };
    auto store_tile = [&](int buf) {
#pragma unroll
        for (int x = 0; x < CHK; ++x) {
            const int e = tid + 256 * x;
            const int r = e / (DK / 8), cc = (e % (DK / 8)) * 8;
            st16(&Qs[buf][r * QPK + cc], pq[x]);
        }
#pragma unroll
        for (int x = 0; x < CHV; ++x) {
            const int e = tid + 256 * x;
            const int r = e / (DV / 8), cc = (e % (DV / 8)) * 8;
            st16(&dOs[buf][r * QPV + cc], pdo[x]);
        }
        if (tid < BR) {
            lse_s[buf][tid] = pok ? pl : INFINITY;
            dlt_s[buf][tid] = pok ? -pd : 0.f;      // stored negated: it seeds dP - Delta
            tl_s[buf][tid] = ptl;
            if constexpr (UM)
                mbits_s[buf][tid] = (uint64_t)(mask_bits16(pm[0]) | (mask_bits16(pm[1]) << 16)) |
                                    ((uint64_t)(mask_bits16(pm[2]) | (mask_bits16(pm[3]) << 16)) << 32);
        }
    };

    if (n_steps > 0) {
        load_tile(0);
        store_tile(0);
    }
    wait_all_memory();
    __syncthreads();
    const int my_kpos = kpos0 + myk;
    const int last_kpos = kpos0 + nkeys - 1;   // the half block's last key position
    for (int st = 0; st < n_steps; ++st) {
        const int buf = st & 1;
        const bool has_next = st + 1 < n_steps;
        if (has_next) load_tile(st + 1);
        const uint16_t* Qb = Qs[buf];
        const uint16_t* dOb = dOs[buf];
        // a bucket's entries are sorted by token, so row 0 holds the step's
        // first token: when it sees the whole half block, no element is masked
        const bool masked = nkeys < 64 || (p.sparse_mode == 2 && last_kpos > tl_s[buf][0]);
        // S^T and dP^T of every 32-row block of the step first, then each
        // block's softmax gradient and dV/dK products, so that (one wavefront
        // per SIMD) the matrix cores work through the next block's products
        // while the vector ALUs run this block's softmax.  dP^T accumulates
        // onto the rows' -Delta: pa ends as dP - Delta.
        f32x16 sab[NSB], pab[NSB];
#pragma unroll
        for (int sb = 0; sb < NSB; ++sb) {
            const int r0 = (BR / 2) * rh + 32 * sb;     // first row of this 32-row block
            sab[sb] = zero16();
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const f32x4 nd = *reinterpret_cast<const f32x4*>(&dlt_s[buf][r0 + 8 * q + 4 * g]);
#pragma unroll
                for (int r = 0; r < 4; ++r) pab[sb][4 * q + r] = nd[r];
            }
#pragma unroll
            for (int s = 0; s < KSM; ++s) {
                if (s < KSK) sab[sb] = T::mma(ld16(&Qb[(r0 + c) * QPK + 16 * s + 8 * g]), kreg[s], sab[sb]);
                if (s < KSV) pab[sb] = T::mma(ld16(&dOb[(r0 + c) * QPV + 16 * s + 8 * g]), vreg[s], pab[sb]);
            }
        }
#pragma unroll
        for (int sb = 0; sb < NSB; ++sb) {
            const int r0 = (BR / 2) * rh + 32 * sb;
            f32x16& sa = sab[sb];
            f32x16& pa = pab[sb];
            auto grad = [&](auto masked_tag, auto user_tag) {
                constexpr bool MK = decltype(masked_tag)::value;
                constexpr bool UMK = decltype(user_tag)::value;   // user mask: MK as well
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int rb = r0 + 8 * q + 4 * g;
                    const f32x4 Lr = *reinterpret_cast<const f32x4*>(&lse_s[buf][rb]);
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int rg = 4 * q + r;
                        float pv = fast_exp2(__builtin_fmaf(sa[rg], p.scale_log2, -Lr[r]));
                        if (MK) {
                            bool off = !col_ok || (p.sparse_mode == 2 && my_kpos > tl_s[buf][rb + r]);
                            if constexpr (UMK) off = off || ((mbits_s[buf][rb + r] >> myk) & 1);
                            pv = off ? 0.f : pv;
                        }
                        sa[rg] = pv;
                        pa[rg] = pv * pa[rg];
                    }
                }
            };
            if constexpr (UM) grad(std::true_type{}, std::true_type{});
            else if (masked) grad(std::true_type{}, std::false_type{});
            else grad(std::false_type{}, std::false_type{});
            if (sb == NSB - 1 && has_next) store_tile(buf ^ 1);
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                const u32x4 bP = acc_to_operand<T>(sa, hh);
                const u32x4 bS = acc_to_operand<T>(pa, hh);
                {
                    // 16 heads per entry: rows r0 + 16hh .. +15 are one
                    // entry; this lane holds 8 of its heads for key myk
                    if (p.ds && col_ok) {
                        const int li = st * E + (r0 + 16 * hh) / 16;
                        if (li < n_e)
                            st16(p.ds + ((int64_t)(eb + li) * p.bs + kb0 + myk) * 16 + 8 * g, bS);
                    }
                }
#pragma unroll
                for (int db = 0; db < DBM; ++db) {
                    if (db < DBV) dva[db] = T::mma(ld_tr<true>(dOb, QPV, r0 + 16 * hh, db * 32, lane), bP, dva[db]);
                    if (db < DBK) dka[db] = T::mma(ld_tr<true>(Qb, QPK, r0 + 16 * hh, db * 32, lane), bS, dka[db]);
                }
            }
        }
        __syncthreads();
    }

    // row halves -> one sum (through LDS, reusing the Q/dO tiles)
    float* red = reinterpret_cast<float*>(arena);
    constexpr int NA = DBV + DBK;            // dV blocks, then dK blocks
    if (rh == 1) {
#pragma unroll
        for (int a = 0; a < NA; ++a) {
            const f32x16& v = a < DBV ? dva[a] : dka[a - DBV];
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                f32x4 x = {v[4 * r4 + 0], v[4 * r4 + 1], v[4 * r4 + 2], v[4 * r4 + 3]};
                *reinterpret_cast<f32x4*>(&red[(((kw * NA + a) * 4 + r4) * 64 + lane) * 4]) = x;
            }
        }
    }
    __syncthreads();
    if (rh == 1 || !col_ok) return;
#pragma unroll
    for (int a = 0; a < NA; ++a) {
        f32x16& v = a < DBV ? dva[a] : dka[a - DBV];
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
            const f32x4 x = *reinterpret_cast<const f32x4*>(&red[(((kw * NA + a) * 4 + r4) * 64 + lane) * 4]);
            v[4 * r4 + 0] += x[0]; v[4 * r4 + 1] += x[1]; v[4 * r4 + 2] += x[2]; v[4 * r4 + 3] += x[3];
        }
    }
    const int npieces = p.pstart[bucket + 1] - p.pstart[bucket];
    if (npieces == 1) {
        const int64_t dko = h2 * p.dk.sh + (int64_t)(key_row0 + myk) * p.dk.ss;
        const int64_t dvo = h2 * p.dv.sh + (int64_t)(key_row0 + myk) * p.dv.ss;
#pragma unroll
        for (int db = 0; db < DBM; ++db)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int e = db * 32 + 8 * q + 4 * g;
                if (db < DBK)
                    st_grad4<T>(p.dk.p, dko + e, p.grad_f32, dka[db][4 * q + 0] * p.scale,
                                dka[db][4 * q + 1] * p.scale, dka[db][4 * q + 2] * p.scale,
                                dka[db][4 * q + 3] * p.scale);
                if (db < DBV)
                    st_grad4<T>(p.dv.p, dvo + e, p.grad_f32, dva[db][4 * q + 0], dva[db][4 * q + 1],
                                dva[db][4 * q + 2], dva[db][4 * q + 3]);
            }
    } else {
        // fp32 partials of a (piece, half): dK [64][DK], then dV [64][DV]
        float* const base = p.partial + ((int64_t)piece * p.halves + half) * 64 * (DK + DV);
        float* pk = base + myk * DK;
        float* pv = base + 64 * DK + myk * DV;
#pragma unroll
        for (int db = 0; db < DBM; ++db)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                if (db < DBK) {
                    f32x4 a = {dka[db][4 * q + 0], dka[db][4 * q + 1], dka[db][4 * q + 2], dka[db][4 * q + 3]};
                    *reinterpret_cast<f32x4*>(pk + db * 32 + 8 * q + 4 * g) = a;
                }
                if (db < DBV) {
                    f32x4 v = {dva[db][4 * q + 0], dva[db][4 * q + 1], dva[db][4 * q + 2], dva[db][4 * q + 3]};
                    *reinterpret_cast<f32x4*>(pv + db * 32 + 8 * q + 4 * g) = v;
                }
            }
    }
}

#ifdef SDPA_NSA_KV_UNIT
// The dK/dV kernel's launch, compiled in its own translation unit (nsa_kv.hip)
// so that the build can give the kernel scheduler options of its own.
template <class T, int DK, int DV>
hipError_t launch_nsa_kv(const NsaParams& p, hipStream_t st) {
    if (p.mask)
        PROF_LAUNCH(KID_NSA_KV, st, (nsa_kv_kernel<T, DK, DV, true>), dim3(p.max_pieces, p.halves), dim3(256), 0,
                    st, p);
    else
        PROF_LAUNCH(KID_NSA_KV, st, (nsa_kv_kernel<T, DK, DV, false>), dim3(p.max_pieces, p.halves), dim3(256), 0,
                    st, p);
    return hipGetLastError();
}
#define SDPA_NSA_KV_INST(T)                                                      \
    template hipError_t launch_nsa_kv<T, 64, 64>(const NsaParams&, hipStream_t);   \
    template hipError_t launch_nsa_kv<T, 128, 128>(const NsaParams&, hipStream_t); \
    template hipError_t launch_nsa_kv<T, 192, 192>(const NsaParams&, hipStream_t); \
    template hipError_t launch_nsa_kv<T, 192, 128>(const NsaParams&, hipStream_t);
SDPA_NSA_KV_INST(F16)
SDPA_NSA_KV_INST(BF16)
#undef SDPA_NSA_KV_INST

}  // namespace sdpa
#else   // the rest of the selected-attention kernels and the entry points

// Defined in nsa_kv.hip.
template <class T, int DK, int DV>
hipError_t launch_nsa_kv(const NsaParams& p, hipStream_t st);

// Sum the partials of blocks split into several pieces, in piece order; a
// block no token chose (no piece) gets zeros, and a block with one piece was
// written by the dK/dV kernel itself.  Grid:
// (bucket, 64-key half, key group); one (key, 8 columns) item per thread: the
// item's dK columns when they exist (d0 < DK) and its dV columns when those
// do (d0 < DV); LPR threads per key, LPR the power of two that covers the
// wider head.  The pieces' partials are read four at a time so that their
// loads are in flight together.
template <int DK, int DV>
constexpr int reduce_lanes() {
    constexpr int w = (DK > DV ? DK : DV) / 8;
    return w <= 8 ? 8 : w <= 16 ? 16 : 32;
}
template <int DK, int DV>
constexpr int reduce_key_groups() { return 64 / (256 / reduce_lanes<DK, DV>()); }

template <class T, int DK, int DV>
__device__ __forceinline__ void kv_reduce_body(const NsaParams& p, int bucket, int half, int group) {
    constexpr int LPR = reduce_lanes<DK, DV>();   // threads per key row, 8 columns each
    const int h2 = bucket / p.NB, blk = bucket % p.NB;
    const int kb0 = half * 64;
    if (kb0 >= p.bs) return;
    const int ps = p.pstart[bucket], np = p.pstart[bucket + 1] - ps;
    if (np == 1) return;
    const int nkeys = min(64, p.bs - kb0);
    const int key = group * (256 / LPR) + threadIdx.x / LPR, d0 = (threadIdx.x % LPR) * 8;
    const bool has_k = d0 < DK, has_v = d0 < DV;
    if (key >= nkeys || !(has_k || has_v)) return;
    float ak[8], av[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) { ak[i] = 0.f; av[i] = 0.f; }
    // partials of a (piece, half): dK [64][DK], then dV [64][DV]
    const float* base = p.partial + ((int64_t)ps * p.halves + half) * 64 * (DK + DV);
    const int kofs = key * DK + d0, vofs = 64 * DK + key * DV + d0;
    const int64_t pstride = (int64_t)p.halves * 64 * (DK + DV);   // between consecutive pieces
    auto add = [&](const float* pp) {
        if (has_k) {
            const f32x4 k0 = *reinterpret_cast<const f32x4*>(pp + kofs);
            const f32x4 k1 = *reinterpret_cast<const f32x4*>(pp + kofs + 4);
#pragma unroll
            for (int i = 0; i < 4; ++i) { ak[i] += k0[i]; ak[4 + i] += k1[i]; }
        }
        if (has_v) {
            const f32x4 v0 = *reinterpret_cast<const f32x4*>(pp + vofs);
            const f32x4 v1 = *reinterpret_cast<const f32x4*>(pp + vofs + 4);
#pragma unroll
            for (int i = 0; i < 4; ++i) { av[i] += v0[i]; av[4 + i] += v1[i]; }
        }
    };
    int x = 0;
    for (; x + 4 <= np; x += 4) {
#pragma unroll
        for (int u = 0; u < 4; ++u) add(base + (x + u) * pstride);
    }
    for (; x < np; ++x) add(base + x * pstride);
#pragma unroll
    for (int i = 0; i < 8; ++i) ak[i] *= p.scale;
    const int64_t row = (int64_t)blk * p.bs + kb0 + key;
    if (has_k) st_grad8<T>(p.dk.p, h2 * p.dk.sh + row * p.dk.ss + d0, p.grad_f32, ak);
    if (has_v) st_grad8<T>(p.dv.p, h2 * p.dv.sh + row * p.dv.ss + d0, p.grad_f32, av);
}

template <class T, int DK, int DV>
__global__ __launch_bounds__(256) void nsa_kv_reduce_kernel(NsaParams p) {
    kv_reduce_body<T, DK, DV>(p, blockIdx.x, blockIdx.y, blockIdx.z);
}

// ---------------------------------------------------------------------------
// dQ: token outer over the gathered keys
// ---------------------------------------------------------------------------
//
// Workgroup (four wavefronts) per (token, KV head, tile of 16 query heads).
// Keys stream through LDS 128 at a time (gathered rows of K and V); wavefront
// w takes keys 32*w .. +31 of each chunk.  Scores are computed transposed on
// v_mfma_f32_16x16x32 (S^T = K Q^T, 16 keys x 16 heads per tile) so the heads
// are the MFMA columns and each lane's LSE and Delta are one value; dQ^T +=
// K^T dS^T uses the two 16-key tiles of a wavefront as one 32-deep operand.
// The four wavefronts' partial dQ^T are summed through LDS at the end.

template <class T, int DK, int DV>
__global__ __launch_bounds__(256) void nsa_dq_kernel(NsaParams p) {
    constexpr int BK = 128;
    constexpr int KPK = DK + 8, KPV = DV + 8;     // LDS row pitches of the K and V chunks
    constexpr int KSK = DK / 32, KSV = DV / 32;   // k-steps of 16x16x32: S over DK, dP over DV
    constexpr int KSM = KSK > KSV ? KSK : KSV;
    constexpr int DB = DK / 16;                   // 16-row blocks of dQ^T
    constexpr int CHK = BK * DK / 8 / 256, CHV = BK * DV / 8 / 256;
    __shared__ __align__(16) uint16_t Ks[BK * KPK];
    __shared__ __align__(16) uint16_t Vs[BK * KPV];
    __shared__ int kpos_s[BK];
    __shared__ int blk_s[128];          // the token's chosen blocks (block_count <= 128)

    const int t = blockIdx.x;
    const int h2 = blockIdx.y / ((p.G + 15) / 16);
    const int ht = blockIdx.y % ((p.G + 15) / 16);
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int col = lane & 15, G16 = lane >> 4;
    const int s_idx = seq_of_token(p.seqs, t);
    if (s_idx < 0) return;
    const SeqRow sq = seq_row(p.seqs, s_idx);
    const int t_local = t - sq.q0;
    const int krow0 = sq.k0;
    const int nblk = sq.lk / p.bs;              // blocks of this sequence
    const int gh = ht * 16 + col;               // head within the group
    const bool head_ok = gh < p.G;
    const int h = h2 * p.G + (head_ok ? gh : 0);

    u32x4 qreg[KSK], doreg[KSV];
    const uint16_t* qp = p.q.p + (int64_t)t * p.q.ss + (int64_t)h * p.q.sh;
    const uint16_t* dop = p.dout.p + (int64_t)t * p.dout.ss + (int64_t)h * p.dout.sh;
#pragma unroll
    for (int s = 0; s < KSM; ++s) {
        u32x4 z = {0u, 0u, 0u, 0u};
        if (s < KSK) qreg[s] = head_ok ? ld16(qp + 32 * s + 8 * G16) : z;
        if (s < KSV) doreg[s] = head_ok ? ld16(dop + 32 * s + 8 * G16) : z;
    }
    const float l2 = head_ok ? p.lse2[(int64_t)t * p.Hq + h] : INFINITY;
    const float dl = head_ok ? p.delta[(int64_t)t * p.Hq + h] : 0.f;

    f32x4 dq[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) dq[db] = zero4();

    // The token's chosen blocks go to LDS once (as first packed key rows, or
    // -1 for a choice outside the sequence), so chunk addresses need no
    // dependent global load.  Each chunk's K/V rows are loaded into registers
    // while the previous chunk is being used; loads are unconditional (rows of
    // an ignored choice or past the gathered keys re-read key row krow0 and
    // are masked through kpos).
    const int nk = p.count * p.bs;
    const int32_t* tk = p.topk + (int64_t)t * p.tk_st + (int64_t)h2 * p.tk_sn;
    for (int i = tid; i < p.count; i += 256) {
        const int blk = tk[(int64_t)i * p.tk_sk];
        blk_s[i] = (blk >= 0 && blk < nblk) ? blk : -1;
    }
    __syncthreads();
    u32x4 kv[CHK], vv[CHV];
    int kpos_r = 0x7fffffff;
    // slot and row-in-block of gathered key n: when block_size divides the
    // chunk, chunk c0 starts at slot c0 / block_size and a row's part of that
    // is fixed, so the divisions are done once
    const bool bs_divides = BK % p.bs == 0;
    int rq[CHK], rr[CHK], rqv[CHV], rrv[CHV];
#pragma unroll
    for (int x = 0; x < CHK; ++x) {
        const int r = (tid + 256 * x) / (DK / 8);
        rq[x] = r / p.bs;
        rr[x] = r % p.bs;
    }
#pragma unroll
    for (int x = 0; x < CHV; ++x) {
        if constexpr (DK == DV) {
            rqv[x] = rq[x];
            rrv[x] = rr[x];
        } else {
            const int r = (tid + 256 * x) / (DV / 8);
            rqv[x] = r / p.bs;
            rrv[x] = r % p.bs;
        }
    }
    const int rq_k = (tid & (BK - 1)) / p.bs, rr_k = (tid & (BK - 1)) % p.bs;
    // the user mask's row of this token (a masked key is treated as absent)
    const uint8_t* mrow = p.mask ? p.mask + (int64_t)t_local * p.mask_ss : nullptr;
    uint32_t mbyte = 0;
    // row strides are below 2^23 elements: 32 x 32 -> 64-bit row offsets
    const int kss = (int)p.k.ss, vss = (int)p.v.ss;
    const uint16_t* const kh = p.k.p + (int64_t)h2 * p.k.sh;
    const uint16_t* const vh = p.v.p + (int64_t)h2 * p.v.sh;
    // packed key row of gathered key c0 + r (row krow0, masked, for an
    // ignored choice or past the gathered keys)
    auto key_row = [&](int c0, int cs, int r, int q, int rm) {
        int slot, rb;
        if (bs_divides) { slot = cs + q; rb = rm; }
        else { const int n = c0 + r; slot = n / p.bs; rb = n % p.bs; }
        const int blk = blk_s[min(slot, p.count - 1)];
        const bool ok = c0 + r < nk && blk >= 0;
        return krow0 + (ok ? blk * p.bs + rb : 0);
    };
    auto load_chunk = [&](int c0) {
        const int cs = bs_divides ? c0 / p.bs : 0;
#pragma unroll
        for (int x = 0; x < CHK; ++x) {
            const int e = tid + 256 * x;
            const int r = e / (DK / 8), cc = (e % (DK / 8)) * 8;
            const int row = key_row(c0, cs, r, rq[x], rr[x]);
            kv[x] = ld16(kh + (int64_t)row * kss + cc);
            if constexpr (DK == DV) vv[x] = ld16(vh + (int64_t)row * vss + cc);
        }
        if constexpr (DK != DV) {
#pragma unroll
            for (int x = 0; x < CHV; ++x) {
                const int e = tid + 256 * x;
                const int r = e / (DV / 8), cc = (e % (DV / 8)) * 8;
                const int row = key_row(c0, cs, r, rqv[x], rrv[x]);
                vv[x] = ld16(vh + (int64_t)row * vss + cc);
            }
        }
        const int n = c0 + (tid & (BK - 1));
        int slot, rb;
        if (bs_divides) { slot = cs + rq_k; rb = rr_k; }
        else { slot = n / p.bs; rb = n % p.bs; }
        const int blk = blk_s[min(slot, p.count - 1)];
        kpos_r = (n < nk && blk >= 0) ? blk * p.bs + rb : 0x7fffffff;   // masked: no key there
        if (mrow && kpos_r != 0x7fffffff) mbyte = mrow[kpos_r];
    };
    load_chunk(0);
    for (int c0 = 0; c0 < nk; c0 += BK) {
        if (mrow && mbyte) kpos_r = 0x7fffffff;
        mbyte = 0;
        __syncthreads();
#pragma unroll
        for (int x = 0; x < CHK; ++x) {
            const int e = tid + 256 * x;
            const int r = e / (DK / 8), cc = (e % (DK / 8)) * 8;
            st16(&Ks[r * KPK + cc], kv[x]);
        }
#pragma unroll
        for (int x = 0; x < CHV; ++x) {
            const int e = tid + 256 * x;
            const int r = e / (DV / 8), cc = (e % (DV / 8)) * 8;
            st16(&Vs[r * KPV + cc], vv[x]);
        }
        if (tid < BK) kpos_s[tid] = kpos_r;
        // whether any key of the chunk is masked for this token
        const bool masked = __syncthreads_or(tid < BK && (kpos_r == 0x7fffffff ||
                                                          (p.sparse_mode == 2 && kpos_r > t_local)));
        if (c0 + BK < nk) load_chunk(c0 + BK);
        f32x4 s[2], dp[2];
#pragma unroll
        for (int x = 0; x < 2; ++x) {
            s[x] = zero4();
            dp[x][0] = dp[x][1] = dp[x][2] = dp[x][3] = -dl;   // dP^T accumulates onto -Delta
            const int kr = 32 * w + 16 * x + col;       // A rows: keys
#pragma unroll
            for (int ks = 0; ks < KSM; ++ks) {
                if (ks < KSK) s[x] = T::mma16(ld16(&Ks[kr * KPK + 32 * ks + 8 * G16]), qreg[ks], s[x]);
                if (ks < KSV) dp[x] = T::mma16(ld16(&Vs[kr * KPV + 32 * ks + 8 * G16]), doreg[ks], dp[x]);
            }
            if (masked) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int kl = 32 * w + 16 * x + 4 * G16 + r;   // chunk-local key of this element
                    const int kpos = kpos_s[kl];
                    const bool off = kpos == 0x7fffffff || (p.sparse_mode == 2 && kpos > t_local);
                    const float pv = fast_exp2(__builtin_fmaf(s[x][r], p.scale_log2, -l2));
                    dp[x][r] = off ? 0.f : pv * dp[x][r];
                }
            } else {
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    dp[x][r] = fast_exp2(__builtin_fmaf(s[x][r], p.scale_log2, -l2)) * dp[x][r];
            }
        }
        u32x4 bS;
        bS[0] = T::pack_op(dp[0][0], dp[0][1]);
        bS[1] = T::pack_op(dp[0][2], dp[0][3]);
        bS[2] = T::pack_op(dp[1][0], dp[1][1]);
        bS[3] = T::pack_op(dp[1][2], dp[1][3]);
#pragma unroll
        for (int db = 0; db < DB; ++db)
            dq[db] = T::mma16(ld_tr16x16_acc(Ks, KPK, 32 * w, 16 * db, lane), bS, dq[db]);
    }

    // sum the four wavefronts' partials (through LDS, reusing Ks)
    __syncthreads();
    float* red = reinterpret_cast<float*>(Ks);
    static_assert(sizeof(Ks) >= 3 * DB * 64 * 4 * 4, "reduction space");
    if (w != 0) {
#pragma unroll
        for (int db = 0; db < DB; ++db)
            *reinterpret_cast<f32x4*>(&red[((((w - 1) * DB) + db) * 64 + lane) * 4]) = dq[db];
    }
    __syncthreads();
    if (w != 0 || !head_ok) return;
#pragma unroll
    for (int x = 0; x < 3; ++x)
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            const f32x4 v = *reinterpret_cast<const f32x4*>(&red[(((x * DB) + db) * 64 + lane) * 4]);
            dq[db][0] += v[0]; dq[db][1] += v[1]; dq[db][2] += v[2]; dq[db][3] += v[3];
        }
    // dQ^T tile: lane holds head `col`, head dims 16*db + 4*G16 + r
    const int64_t dqo = (int64_t)t * p.dq.ss + (int64_t)h * p.dq.sh;
#pragma unroll
    for (int db = 0; db < DB; ++db)
        st_grad4<T>(p.dq.p, dqo + 16 * db + 4 * G16, p.grad_f32, dq[db][0] * p.scale, dq[db][1] * p.scale,
                    dq[db][2] * p.scale, dq[db][3] * p.scale);
}

// ---------------------------------------------------------------------------
// dQ from the stored dS (16 query heads per KV head)
// ---------------------------------------------------------------------------
//
// dQ_t = scale * sum over the token's gathered keys j of dS_tj K_j, with dS
// as the dK/dV kernel stored it (one 16-head x block_size tile per entry),
// so this pass gathers K only and recomputes neither S nor dP.  Workgroup
// (four wavefronts) per (token, KV head); the gathered keys go 64 at a time:
// the chunk's K rows and dS^T rows are loaded into registers during the
// previous chunk and staged in LDS; wavefront w forms
// dQ^T for head dims D/4 * w .. + D/4 - 1 as K^T dS^T (v_mfma_f32_16x16x32,
// both operands by transposing LDS reads), so no partials are reduced.  A
// choice outside the sequence has no entry and contributes zero.  The pass
// is bound by the latency of its gathered loads, so it is sized for
// occupancy: 64-key chunks (20 KB of LDS at D = 128) and 72 registers at
// D = 128, six workgroups per CU: NSA workload 95 -> 86 us at Dqk = 128
// and 185 -> 140 us at 192 against 128-key chunks at four (two-buffer
// 128-key chunks at two workgroups per CU: 136 us).
template <class T, int D>
__device__ __forceinline__ void dq_ds_body(const NsaParams& p, int t, int h2) {
    static_assert(D == 64 || D == 128 || D == 192, "stored-dS dQ: Dqk 64, 128 or 192");
    constexpr int BK = 64;
    constexpr int NJ = D / 64;                   // 16-column dQ^T tiles per wavefront
    constexpr int KP = D + 8;                    // K rows in LDS, padded
    constexpr int DP = 16;                       // dS^T rows: 16 heads
    constexpr int CHK = BK * D / 8 / 256;        // 16-byte K chunks per thread
    __shared__ __align__(16) uint16_t Ks[BK * KP];
    __shared__ __align__(16) uint16_t Ds[BK * DP];
    __shared__ int blk_s[128];                   // the token's chosen blocks (-1: none)
    __shared__ int pos_s[128];                   // their entries' list positions

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int col = lane & 15, G16 = lane >> 4;
    const int s_idx = seq_of_token(p.seqs, t);
    if (s_idx < 0) return;
    const SeqRow sq = seq_row(p.seqs, s_idx);
    const int krow0 = sq.k0;
    const int nblk = sq.lk / p.bs;
    const int nk = p.count * p.bs;
    const int32_t* tk = p.topk + (int64_t)t * p.tk_st + (int64_t)h2 * p.tk_sn;
    const int32_t* pos_of = p.rank + (int64_t)h2 * p.Tq * p.count + (int64_t)t * p.count;
    for (int i = tid; i < p.count; i += 256) {
        const int blk = tk[(int64_t)i * p.tk_sk];
        const bool ok = blk >= 0 && blk < nblk;
        blk_s[i] = ok ? blk : -1;
        pos_s[i] = ok ? pos_of[i] : -1;
    }
    __syncthreads();

    const int kss = (int)p.k.ss;
    const uint16_t* const kh = p.k.p + (int64_t)h2 * p.k.sh;
    u32x4 kv[CHK], dv;
    // Unconditional loads: a key of no block, or past the gathered keys,
    // re-reads key row krow0 and entry 0's dS, and its dS is zeroed.
    auto load_chunk = [&](int c0) {
#pragma unroll
        for (int x = 0; x < CHK; ++x) {
            const int e = tid + 256 * x;
            const int r = e / (D / 8), cc = (e % (D / 8)) * 8;
            const int n = c0 + r;
            const int slot = min(n / p.bs, p.count - 1);
            const int blk = blk_s[slot];
            const int row = krow0 + ((n < nk && blk >= 0) ? blk * p.bs + n % p.bs : 0);
            kv[x] = ld16(kh + (int64_t)row * kss + cc);
        }
        const int n = c0 + ((tid >> 1) & (BK - 1));
        const int slot = min(n / p.bs, p.count - 1);
        const int pos = n < nk ? pos_s[slot] : -1;
        dv = ld16(p.ds + ((int64_t)max(pos, 0) * p.bs + n % p.bs) * 16 + 8 * (tid & 1));
        if (pos < 0) dv = u32x4{0u, 0u, 0u, 0u};
    };
    f32x4 dq[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) dq[j] = zero4();
    load_chunk(0);
    for (int c0 = 0; c0 < nk; c0 += BK) {
        __syncthreads();
#pragma unroll
        for (int x = 0; x < CHK; ++x) {
            const int e = tid + 256 * x;
            st16(&Ks[(e / (D / 8)) * KP + (e % (D / 8)) * 8], kv[x]);
        }
        if (tid < 2 * BK) st16(&Ds[(tid >> 1) * DP + 8 * (tid & 1)], dv);
        __syncthreads();
        if (c0 + BK < nk) load_chunk(c0 + BK);
#pragma unroll
        for (int ks = 0; ks < BK / 32; ++ks) {
            const u32x4 b = ld_tr16x16(Ds, DP, 32 * ks, 0, lane);
#pragma unroll
            for (int j = 0; j < NJ; ++j)
                dq[j] = T::mma16(ld_tr16x16(Ks, KP, 32 * ks, 16 * (NJ * w + j), lane), b, dq[j]);
        }
    }
    // dQ^T tiles: lane holds stored head slot `col` (head 0-3, 8-11, 4-7,
    // 12-15 in slot order), head dims 16 (NJ w + j) + 4*G16 + r
    const int h = h2 * 16 + ((col & 4) ? (col >> 3) * 4 + 8 + (col & 3) : (col >> 3) * 4 + (col & 3));
    const int64_t dqo = (int64_t)t * p.dq.ss + (int64_t)h * p.dq.sh;
#pragma unroll
    for (int j = 0; j < NJ; ++j)
        st_grad4<T>(p.dq.p, dqo + 16 * (NJ * w + j) + 4 * G16, p.grad_f32, dq[j][0] * p.scale, dq[j][1] * p.scale,
                    dq[j][2] * p.scale, dq[j][3] * p.scale);
}

// One launch for the stored-dS dQ pass and the partial-sum reduction of
// dK/dV (independent of each other; both follow the dK/dV kernel): the dQ
// items first, one per (token, KV head), then the reduction's items, which
// fill the CUs the dQ pass's last round leaves idle.
template <class T, int DK, int DV>
__global__ __launch_bounds__(256, 6) void nsa_dq_ds_kernel(NsaParams p, int n_dq) {
    const int id = blockIdx.x;
    if (id < n_dq) {
        dq_ds_body<T, DK>(p, id / p.N2, id % p.N2);
        return;
    }
    constexpr int NG = reduce_key_groups<DK, DV>();
    const int r = id - n_dq;
    kv_reduce_body<T, DK, DV>(p, r / (p.halves * NG), (r / NG) % p.halves, r % NG);
}

// ---------------------------------------------------------------------------
// dQ at Dqk = 192: wavefronts on their own
// ---------------------------------------------------------------------------
//
// Workgroup (four wavefronts) per (token, KV head, tile of 16 query heads).
// The token's gathered keys go in steps of 32; wavefront w takes steps w,
// w + 4, ... on its own: it loads the step's K and V rows from global memory
// straight into registers in the A-operand layout of v_mfma_f32_16x16x32
// (S^T = K Q^T and dP^T = V dO^T, 16 keys x 16 heads per tile, so the heads
// are the MFMA columns and each lane's LSE and Delta are one value), the next
// step's rows in flight meanwhile, and stages only K in an LDS tile of its
// own for the transposed operand of dQ^T += K^T dS^T (the two 16-key tiles of
// the step as one 32-deep operand).  No LDS is shared during the loop, so
// there is no barrier; the four partial dQ^T are summed through LDS at the
// end, in wavefront order.  (A 16-key group lies within one block: block
// sizes are multiples of 16.)  At Dqk = 192 the shared-chunk kernel above
// needs 86 KB of LDS and 320 registers, one workgroup per CU; this form fits
// two wavefronts per SIMD: 519 -> 300 us at (192, 128) and 467 -> 356 us at
// (192, 192) on the NSA workload shape.  At Dqk = 128, where both run two
// wavefronts per SIMD, the shared-chunk kernel is faster (190 against 241
// us): its loads read whole rows, four per instruction, where a wavefront's
// own MFMA-layout loads touch 16 rows each.

template <class T, int DK, int DV>
__global__ __launch_bounds__(256, 2) void nsa_dq_wave_kernel(NsaParams p) {
    constexpr int KPK = DK + 8;                   // LDS row pitch of a wavefront's K tile
    constexpr int KSK = DK / 32, KSV = DV / 32;   // k-steps of 16x16x32: S over DK, dP over DV
    constexpr int KSM = KSK > KSV ? KSK : KSV;
    constexpr int DB = DK / 16;                   // 16-row blocks of dQ^T
    constexpr bool PF = DK <= 128 && DV <= 128;   // two register sets of K/V rows fit
    constexpr int TILE = 32 * KPK;
    __shared__ __align__(16) uint16_t Kt[4 * TILE];
    __shared__ int blk_s[128];          // the token's chosen blocks (block_count <= 128)
    static_assert(sizeof(Kt) >= 3 * DB * 64 * 16, "reduction space");

    const int t = blockIdx.x;
    const int h2 = blockIdx.y / ((p.G + 15) / 16);
    const int ht = blockIdx.y % ((p.G + 15) / 16);
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: the step loop and its block lookups stay scalar
    const int col = lane & 15, G16 = lane >> 4;
    const int s_idx = seq_of_token(p.seqs, t);
    if (s_idx < 0) return;
    const SeqRow sq = seq_row(p.seqs, s_idx);
    const int t_local = t - sq.q0;
    const int krow0 = sq.k0;
    const int nblk = sq.lk / p.bs;              // blocks of this sequence
    const int gh = ht * 16 + col;               // head within the group
    const bool head_ok = gh < p.G;
    const int h = h2 * p.G + (head_ok ? gh : 0);

    u32x4 qreg[KSK], doreg[KSV];
    const uint16_t* qp = p.q.p + (int64_t)t * p.q.ss + (int64_t)h * p.q.sh;
    const uint16_t* dop = p.dout.p + (int64_t)t * p.dout.ss + (int64_t)h * p.dout.sh;
#pragma unroll
    for (int s = 0; s < KSM; ++s) {
        u32x4 z = {0u, 0u, 0u, 0u};
        if (s < KSK) qreg[s] = head_ok ? ld16(qp + 32 * s + 8 * G16) : z;
        if (s < KSV) doreg[s] = head_ok ? ld16(dop + 32 * s + 8 * G16) : z;
    }
    const float l2 = head_ok ? p.lse2[(int64_t)t * p.Hq + h] : INFINITY;
    const float dl = head_ok ? p.delta[(int64_t)t * p.Hq + h] : 0.f;

    f32x4 dq[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) dq[db] = zero4();

    // the token's chosen blocks (-1 for a choice outside the sequence)
    const int32_t* tk = p.topk + (int64_t)t * p.tk_st + (int64_t)h2 * p.tk_sn;
    for (int i = tid; i < p.count; i += 256) {
        const int blk = tk[(int64_t)i * p.tk_sk];
        blk_s[i] = (blk >= 0 && blk < nblk) ? blk : -1;
    }
    __syncthreads();

    const int nk = p.count * p.bs;              // gathered keys, a multiple of 16
    const int n_steps = (nk + 31) / 32;
    // row strides are below 2^23 elements: 32 x 32 -> 64-bit row offsets
    const int kss = (int)p.k.ss, vss = (int)p.v.ss;
    const uint16_t* const kh = p.k.p + (int64_t)h2 * p.k.sh;
    const uint16_t* const vh = p.v.p + (int64_t)h2 * p.v.sh;
    // the user mask's row of this token (a masked key is treated as absent)
    const uint8_t* mrow = p.mask ? p.mask + (int64_t)t_local * p.mask_ss : nullptr;
    uint16_t* const Kw = Kt + w * TILE;

    // Rows of one step: K and V of this lane's key in the two 16-key groups.
    // Loads are unconditional: a group past the gathered keys or of an
    // ignored choice re-reads key row krow0 and is masked.
    struct Rows {
        u32x4 k[2][KSK], v[2][KSV];
    };
    // group x of step st: its sequence-local key position base (-1: absent)
    auto group_pos = [&](int st, int x) {
        const int n16 = st * 32 + 16 * x;
        const int blk = blk_s[min(n16 / p.bs, p.count - 1)];
        return (n16 < nk && blk >= 0) ? blk * p.bs + n16 % p.bs : -1;
    };
    auto load = [&](Rows& r, int st) {
#pragma unroll
        for (int x = 0; x < 2; ++x) {
            const int pos = group_pos(st, x);
            const int row = krow0 + (pos >= 0 ? pos + col : 0);
#pragma unroll
            for (int ks = 0; ks < KSK; ++ks) r.k[x][ks] = ld16(kh + (int64_t)row * kss + 32 * ks + 8 * G16);
#pragma unroll
            for (int ks = 0; ks < KSV; ++ks) r.v[x][ks] = ld16(vh + (int64_t)row * vss + 32 * ks + 8 * G16);
        }
    };
    auto step = [&](const Rows& r, int st) {
        const int pos0 = group_pos(st, 0), pos1 = group_pos(st, 1);
        // user-mask bytes of the four keys of each group this lane's C
        // elements cover
        uint32_t mb[2] = {0u, 0u};
        if (mrow) {
            if (pos0 >= 0) mb[0] = *reinterpret_cast<const uint32_t*>(mrow + pos0 + 4 * G16);
            if (pos1 >= 0) mb[1] = *reinterpret_cast<const uint32_t*>(mrow + pos1 + 4 * G16);
        }
        // K rows into this wavefront's tile for the transposed dQ operand
#pragma unroll
        for (int x = 0; x < 2; ++x)
#pragma unroll
            for (int ks = 0; ks < KSK; ++ks) st16(&Kw[(16 * x + col) * KPK + 32 * ks + 8 * G16], r.k[x][ks]);
        f32x4 s[2], dp[2];
#pragma unroll
        for (int x = 0; x < 2; ++x) {
            s[x] = zero4();
            dp[x][0] = dp[x][1] = dp[x][2] = dp[x][3] = -dl;   // dP^T accumulates onto -Delta
#pragma unroll
            for (int ks = 0; ks < KSM; ++ks) {
                if (ks < KSK) s[x] = T::mma16(r.k[x][ks], qreg[ks], s[x]);
                if (ks < KSV) dp[x] = T::mma16(r.v[x][ks], doreg[ks], dp[x]);
            }
        }
        // element (x, e): key position pos_x + 4*G16 + e of the sequence
        const bool whole = pos0 >= 0 && pos1 >= 0 && !mrow &&
                           (p.sparse_mode != 2 || max(pos0, pos1) + 15 <= t_local);
        if (whole) {
#pragma unroll
            for (int x = 0; x < 2; ++x)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    dp[x][e] = fast_exp2(__builtin_fmaf(s[x][e], p.scale_log2, -l2)) * dp[x][e];
        } else {
#pragma unroll
            for (int x = 0; x < 2; ++x) {
                const int pos = x ? pos1 : pos0;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int kp = pos + 4 * G16 + e;
                    const bool off = pos < 0 || (p.sparse_mode == 2 && kp > t_local) || ((mb[x] >> (8 * e)) & 0xffu);
                    const float pv = fast_exp2(__builtin_fmaf(s[x][e], p.scale_log2, -l2));
                    dp[x][e] = off ? 0.f : pv * dp[x][e];
                }
            }
        }
        u32x4 bS;
        bS[0] = T::pack_op(dp[0][0], dp[0][1]);
        bS[1] = T::pack_op(dp[0][2], dp[0][3]);
        bS[2] = T::pack_op(dp[1][0], dp[1][1]);
        bS[3] = T::pack_op(dp[1][2], dp[1][3]);
        // one wavefront writes and reads its tile: LDS keeps the order
        __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
#pragma unroll
        for (int db = 0; db < DB; ++db)
            dq[db] = T::mma16(ld_tr16x16_acc(Kw, KPK, 0, 16 * db, lane), bS, dq[db]);
        __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    };

    if constexpr (PF) {
        Rows ra, rb;
        if (w < n_steps) load(ra, w);
        for (int st = w; st < n_steps; st += 8) {
            const bool b_ok = st + 4 < n_steps;
            if (b_ok) load(rb, st + 4);
            step(ra, st);
            if (!b_ok) break;
            if (st + 8 < n_steps) load(ra, st + 8);
            step(rb, st + 4);
        }
    } else {
        Rows ra;
        for (int st = w; st < n_steps; st += 4) {
            load(ra, st);
            step(ra, st);
        }
    }

    // sum the four wavefronts' partials (through LDS, reusing the K tiles)
    __syncthreads();
    float* red = reinterpret_cast<float*>(Kt);
    if (w != 0) {
#pragma unroll
        for (int db = 0; db < DB; ++db)
            *reinterpret_cast<f32x4*>(&red[((((w - 1) * DB) + db) * 64 + lane) * 4]) = dq[db];
    }
    __syncthreads();
    if (w != 0 || !head_ok) return;
#pragma unroll
    for (int x = 0; x < 3; ++x)
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            const f32x4 v = *reinterpret_cast<const f32x4*>(&red[(((x * DB) + db) * 64 + lane) * 4]);
            dq[db][0] += v[0]; dq[db][1] += v[1]; dq[db][2] += v[2]; dq[db][3] += v[3];
        }
    // dQ^T tile: lane holds head `col`, head dims 16*db + 4*G16 + r
    const int64_t dqo = (int64_t)t * p.dq.ss + (int64_t)h * p.dq.sh;
#pragma unroll
    for (int db = 0; db < DB; ++db)
        st_grad4<T>(p.dq.p, dqo + 16 * db + 4 * G16, p.grad_f32, dq[db][0] * p.scale, dq[db][1] * p.scale,
                    dq[db][2] * p.scale, dq[db][3] * p.scale);
}

// ---------------------------------------------------------------------------
// Forward: O and the (max, sum) statistics over each token's gathered keys
// ---------------------------------------------------------------------------
//
// The selected-attention forward in training mode (Ascend
// aclnnNsaSelectedAttentionGrad page, "Formula": P is the softmax of the scaled
// scores over the gathered blocks; its softmaxMax / softmaxSum parameters are
// this kernel's statistics).  One workgroup per (token, 16 query heads of a KV
// head), as the dQ kernel: the token's chosen blocks stream through LDS 128
// gathered keys at a time; wavefront w scores keys 32w .. +31 of a chunk
// against the 16 heads (S^T = K Q^T, so each lane holds one head column) and
// keeps a running max and sum per head and an O^T partial; the four partials
// are merged at the end.
template <class T, int DK, int DV>
__global__ __launch_bounds__(256) void nsa_fwd_kernel(NsaParams p) {
    constexpr int BK = 128;
    constexpr int KPK = DK + 8, KPV = DV + 8;     // LDS row pitches of the K and V chunks
    constexpr int KS = DK / 32;      // k-steps of 16x16x32 over the query/key head dimension
    constexpr int DB = DV / 16;      // 16-row blocks of O^T
    constexpr int CHK = BK * DK / 8 / 256, CHV = BK * DV / 8 / 256;
    __shared__ __align__(16) uint16_t Ks[BK * KPK];
    __shared__ __align__(16) uint16_t Vs[BK * KPV];
    __shared__ int kpos_s[BK];
    __shared__ int blk_s[128];          // the token's chosen blocks (block_count <= 128)

    const int t = p.t_base + blockIdx.x;
    const int h2 = blockIdx.y / ((p.G + 15) / 16);
    const int ht = blockIdx.y % ((p.G + 15) / 16);
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int col = lane & 15, G16 = lane >> 4;
    const int s_idx = seq_of_token(p.seqs, t);
    if (s_idx < 0) return;
    const SeqRow sq = seq_row(p.seqs, s_idx);
    const int t_local = t - sq.q0;
    const int krow0 = sq.k0;
    const int nblk = sq.lk / p.bs;
    const int gh = ht * 16 + col;
    const bool head_ok = gh < p.G;
    const int h = h2 * p.G + (head_ok ? gh : 0);

    u32x4 qreg[KS];
    const uint16_t* qp = p.q.p + (int64_t)t * p.q.ss + (int64_t)h * p.q.sh;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
        u32x4 z = {0u, 0u, 0u, 0u};
        qreg[s] = head_ok ? ld16(qp + 32 * s + 8 * G16) : z;
    }

    f32x4 o[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) o[db] = zero4();
    float m = -INFINITY, l = 0.f;       // this wavefront's running max (log2 domain) and sum

    const int nk = p.count * p.bs;
    const int32_t* tk = p.topk + (int64_t)t * p.tk_st + (int64_t)h2 * p.tk_sn;
    for (int i = tid; i < p.count; i += 256) {
        const int blk = tk[(int64_t)i * p.tk_sk];
        blk_s[i] = (blk >= 0 && blk < nblk) ? blk : -1;
    }
    __syncthreads();
    // chunk loads as in the dQ kernel: unconditional, an ignored choice or a
    // row past the gathered keys re-reads key row krow0 and is masked
    u32x4 kv[CHK], vv[CHV];
    int kpos_r = 0x7fffffff;
    // the user mask's row of this token (a masked key is treated as absent)
    const uint8_t* mrow = p.mask ? p.mask + (int64_t)t_local * p.mask_ss : nullptr;
    uint32_t mbyte = 0;
    // packed key row of gathered key n (row krow0, masked, if there is none)
    auto key_row = [&](int n) {
        const int blk = blk_s[min(n / p.bs, p.count - 1)];
        const bool ok = n < nk && blk >= 0;
        return (int64_t)krow0 + (ok ? (int64_t)blk * p.bs + n % p.bs : 0);
    };
    auto load_chunk = [&](int c0) {
#pragma unroll
        for (int x = 0; x < CHK; ++x) {
            const int e = tid + 256 * x;
            const int r = e / (DK / 8), cc = (e % (DK / 8)) * 8;
            const int64_t row = key_row(c0 + r);
            kv[x] = ld16(p.k.p + row * p.k.ss + (int64_t)h2 * p.k.sh + cc);
            if constexpr (DK == DV) vv[x] = ld16(p.v.p + row * p.v.ss + (int64_t)h2 * p.v.sh + cc);
        }
        if constexpr (DK != DV) {
#pragma unroll
            for (int x = 0; x < CHV; ++x) {
                const int e = tid + 256 * x;
                const int r = e / (DV / 8), cc = (e % (DV / 8)) * 8;
                const int64_t row = key_row(c0 + r);
                vv[x] = ld16(p.v.p + row * p.v.ss + (int64_t)h2 * p.v.sh + cc);
            }
        }
        const int n = c0 + (tid & (BK - 1));
        const int blk = blk_s[min(n / p.bs, p.count - 1)];
        kpos_r = (n < nk && blk >= 0) ? blk * p.bs + n % p.bs : 0x7fffffff;
        if (mrow && kpos_r != 0x7fffffff) mbyte = mrow[kpos_r];
    };
    load_chunk(0);
    for (int c0 = 0; c0 < nk; c0 += BK) {
        if (mrow && mbyte) kpos_r = 0x7fffffff;
        mbyte = 0;
        __syncthreads();
#pragma unroll
        for (int x = 0; x < CHK; ++x) {
            const int e = tid + 256 * x;
            const int r = e / (DK / 8), cc = (e % (DK / 8)) * 8;
            st16(&Ks[r * KPK + cc], kv[x]);
        }
#pragma unroll
        for (int x = 0; x < CHV; ++x) {
            const int e = tid + 256 * x;
            const int r = e / (DV / 8), cc = (e % (DV / 8)) * 8;
            st16(&Vs[r * KPV + cc], vv[x]);
        }
        if (tid < BK) kpos_s[tid] = kpos_r;
        __syncthreads();
        if (c0 + BK < nk) load_chunk(c0 + BK);
        // scores of keys 32w + 16x + 4*G16 + r against head `col`, log2 domain
        f32x4 sc[2];
        float tmax = -INFINITY;
#pragma unroll
        for (int x = 0; x < 2; ++x) {
            sc[x] = zero4();
            const int kr = 32 * w + 16 * x + col;       // A rows: keys
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                sc[x] = T::mma16(ld16(&Ks[kr * KPK + 32 * ks + 8 * G16]), qreg[ks], sc[x]);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int kpos = kpos_s[32 * w + 16 * x + 4 * G16 + r];
                const bool masked = kpos == 0x7fffffff || (p.sparse_mode == 2 && kpos > t_local);
                sc[x][r] = masked ? -INFINITY : sc[x][r] * p.scale_log2;
                tmax = fmaxf(tmax, sc[x][r]);
            }
        }
        // the head's keys of this wavefront sit in the four 16-lane groups
        tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
        tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
        const float m_new = fmaxf(m, tmax);
        const float msub = m_new == -INFINITY ? 0.f : m_new;
        const float alpha = m == -INFINITY ? 0.f : fast_exp2(m - m_new);
        float rs = 0.f;
#pragma unroll
        for (int x = 0; x < 2; ++x)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                sc[x][r] = fast_exp2(sc[x][r] - msub);
                rs += sc[x][r];
            }
        rs += __shfl_xor(rs, 16);
        rs += __shfl_xor(rs, 32);
        l = l * alpha + rs;
        m = m_new;
        // O^T += V^T P^T over this wavefront's 32 keys (acc-slot order)
        u32x4 bP;
        bP[0] = T::pack_op(sc[0][0], sc[0][1]);
        bP[1] = T::pack_op(sc[0][2], sc[0][3]);
        bP[2] = T::pack_op(sc[1][0], sc[1][1]);
        bP[3] = T::pack_op(sc[1][2], sc[1][3]);
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            o[db][0] *= alpha; o[db][1] *= alpha; o[db][2] *= alpha; o[db][3] *= alpha;
            o[db] = T::mma16(ld_tr16x16_acc(Vs, KPV, 32 * w, 16 * db, lane), bP, o[db]);
        }
    }

    // merge the four wavefronts: M = max m_w, L = sum l_w 2^(m_w - M),
    // O = sum O_w 2^(m_w - M) / L  (through LDS, reusing Ks and kpos_s)
    __syncthreads();
    float* red = reinterpret_cast<float*>(Ks);
    float* ml = reinterpret_cast<float*>(kpos_s);   // [4 waves][16 heads][m, l]
    static_assert(sizeof(Ks) >= 3 * DB * 64 * 4 * 4, "merge space");
    static_assert(sizeof(kpos_s) >= 4 * 16 * 2 * 4, "merge space");
    if (w != 0) {
#pragma unroll
        for (int db = 0; db < DB; ++db)
            *reinterpret_cast<f32x4*>(&red[((((w - 1) * DB) + db) * 64 + lane) * 4]) = o[db];
    }
    if (G16 == 0) { ml[(w * 16 + col) * 2] = m; ml[(w * 16 + col) * 2 + 1] = l; }
    __syncthreads();
    if (w != 0 || !head_ok) return;
    float M = m;
#pragma unroll
    for (int x = 1; x < 4; ++x) M = fmaxf(M, ml[(x * 16 + col) * 2]);
    const float f0 = m == -INFINITY ? 0.f : fast_exp2(m - M);
    float L = l * f0;
#pragma unroll
    for (int db = 0; db < DB; ++db) { o[db][0] *= f0; o[db][1] *= f0; o[db][2] *= f0; o[db][3] *= f0; }
#pragma unroll
    for (int x = 1; x < 4; ++x) {
        const float mx = ml[(x * 16 + col) * 2];
        const float fx = mx == -INFINITY ? 0.f : fast_exp2(mx - M);
        L += ml[(x * 16 + col) * 2 + 1] * fx;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            const f32x4 v = *reinterpret_cast<const f32x4*>(&red[((((x - 1) * DB) + db) * 64 + lane) * 4]);
            o[db][0] += v[0] * fx; o[db][1] += v[1] * fx; o[db][2] += v[2] * fx; o[db][3] += v[3] * fx;
        }
    }
    const float inv = L > 0.f ? 1.f / L : 0.f;
    // O^T tile: lane holds head `col`, head dims 16*db + 4*G16 + r
    uint16_t* op = p.o.p + (int64_t)t * p.o.ss + (int64_t)h * p.o.sh;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
        u32x2 v;
        v[0] = T::pack(o[db][0] * inv, o[db][1] * inv);
        v[1] = T::pack(o[db][2] * inv, o[db][3] * inv);
        st8(op + 16 * db + 4 * G16, v);
    }
    if (G16 == 0) {
        const int64_t so = (int64_t)t * p.st_ss + (int64_t)h * p.st_sh;
        p.m_out[so] = M == -INFINITY ? -INFINITY : M * kLn2;
        p.l_out[so] = L;
    }
}

// ---------------------------------------------------------------------------
// Launch
// ---------------------------------------------------------------------------

// The offsets scan and the scatter: one launch when the buckets fit the
// fused kernel's LDS and there are entries to scatter, else two.
static void launch_scan_scatter(const NsaParams& p, hipStream_t st) {
    if (p.n_tiles > 0 && (int64_t)p.N2 * p.NB <= kScanScatterMax) {
        PROF_LAUNCH(KID_NSA_INDEX, st, nsa_scan_scatter_kernel, dim3(p.n_tiles, p.N2), dim3(64), 0, st, p);
        return;
    }
    PROF_LAUNCH(KID_NSA_INDEX, st, nsa_scan_kernel, dim3(1), dim3(1024), 0, st, p);
    if (p.n_tiles > 0)
        PROF_LAUNCH(KID_NSA_INDEX, st, nsa_scatter_kernel, dim3(p.n_tiles, p.N2), dim3(64), 0, st, p);
}

static hipError_t launch_index(const NsaParams& p, hipStream_t st) {
    if (p.n_tiles > 0)
        PROF_LAUNCH(KID_NSA_INDEX, st, nsa_rank_kernel, dim3(p.n_tiles, p.N2), dim3(64), 0, st, p);
    PROF_LAUNCH(KID_NSA_INDEX, st, nsa_hist_scan_kernel, dim3(p.NB, p.N2), dim3(64), 0, st, p);
    launch_scan_scatter(p, st);
    return hipGetLastError();
}

template <class T, int DK, int DV>
static hipError_t launch_nsa_fwd_t(const NsaParams& p, hipStream_t st) {
    PROF_LAUNCH(KID_FWD, st, (nsa_fwd_kernel<T, DK, DV>), dim3(p.Tq, p.N2 * ((p.G + 15) / 16)), dim3(256), 0, st, p);
    return hipGetLastError();
}

template <class T>
static hipError_t launch_nsa_fwd_dims(const NsaParams& p, int D, int Dv, hipStream_t st) {
    if (D == 64) return launch_nsa_fwd_t<T, 64, 64>(p, st);
    if (D == 128) return launch_nsa_fwd_t<T, 128, 128>(p, st);
    if (Dv == 192) return launch_nsa_fwd_t<T, 192, 192>(p, st);
    return launch_nsa_fwd_t<T, 192, 128>(p, st);      // the other pair the host accepts
}

// DK: head dim of Q and K, DV: of V, O and dO (the row pass reduces dO o O)
template <class T, int DK, int DV>
static hipError_t launch_nsa_t(const NsaParams& p, const BwdParams& bp, hipStream_t st) {
    // the index build with the row pass in its first launch (the two are
    // independent): one launch fewer than index + row pass
    {
        const long n_rank = (long)p.n_tiles * p.N2;
        const long n_pre = (bp.rows + 64 / pre_lanes<DV>() - 1) / (64 / pre_lanes<DV>());
        if (n_rank + n_pre > 0)
            PROF_LAUNCH(KID_NSA_INDEX, st, (nsa_rank_pre_kernel<T, DV>), dim3((unsigned)(n_rank + n_pre)), dim3(64), 0,
                        st, p, bp, (int)n_rank);
        PROF_LAUNCH(KID_NSA_INDEX, st, nsa_hist_scan_kernel, dim3(p.NB, p.N2), dim3(64), 0, st, p);
        launch_scan_scatter(p, st);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    e = launch_nsa_kv<T, DK, DV>(p, st);
    if (e != hipSuccess) return e;
    {
        if (p.ds) {
            // the dQ pass and the reduction in one launch
            const long n_dq = (long)p.Tq * p.N2;
            const long n_red = (long)p.N2 * p.NB * p.halves * reduce_key_groups<DK, DV>();
            if (n_dq + n_red > 0)
                PROF_LAUNCH(KID_NSA_DQ, st, (nsa_dq_ds_kernel<T, DK, DV>), dim3((unsigned)(n_dq + n_red)), dim3(256), 0,
                            st, p, (int)n_dq);
            return hipGetLastError();
        }
    }
    PROF_LAUNCH(KID_NSA_KV_REDUCE, st, (nsa_kv_reduce_kernel<T, DK, DV>),
                dim3(p.N2 * p.NB, p.halves, reduce_key_groups<DK, DV>()), dim3(256), 0, st, p);
    // with no query token (every query length 0) dK and dV are the reduction's
    // zeros and there is no dQ row to write
    if (p.Tq > 0) {
        const dim3 grid(p.Tq, p.N2 * ((p.G + 15) / 16));
        if constexpr (DK > 128) {
            PROF_LAUNCH(KID_NSA_DQ, st, (nsa_dq_wave_kernel<T, DK, DV>), grid, dim3(256), 0, st, p);
        } else {
            PROF_LAUNCH(KID_NSA_DQ, st, (nsa_dq_kernel<T, DK, DV>), grid, dim3(256), 0, st, p);
        }
    }
    return hipGetLastError();
}

template <class T>
static hipError_t launch_nsa_dims(const NsaParams& p, const BwdParams& bp, int D, int Dv, hipStream_t st) {
    if (D == 64) return launch_nsa_t<T, 64, 64>(p, bp, st);
    if (D == 128) return launch_nsa_t<T, 128, 128>(p, bp, st);
    if (Dv == 192) return launch_nsa_t<T, 192, 192>(p, bp, st);
    return launch_nsa_t<T, 192, 128>(p, bp, st);      // the other pair the host accepts
}

}  // namespace sdpa

// ---------------------------------------------------------------------------
// C ABI
// ---------------------------------------------------------------------------

namespace {

constexpr size_t kAlignN = 256;
size_t up(size_t x) { return (x + kAlignN - 1) / kAlignN * kAlignN; }

struct NsaLayout {
    int64_t NB = 0, nbk = 0, E = 0, chunk = 1, max_pieces = 0, halves = 1, tt = 16, n_tiles = 0;
    size_t counts = 0, offsets = 0, entries = 0, pstart = 0, pieces = 0, hist = 0, rank = 0, lse2 = 0, delta = 0,
           partial = 0, seqtab = 0, ds = 0, total = 0;
    bool use_ds = false;      // the dK/dV kernel stores dS for the dQ pass
};

struct Seqs {
    std::vector<int64_t> q0, k0, lq, lk;
    int64_t Tq = 0, Tk = 0;
};

int read_seqs(int64_t batch, const int64_t* cuq, const int64_t* cuk, Seqs& S) {
    int64_t pq = 0, pk = 0;
    for (int64_t b = 0; b < batch; ++b) {
        if (cuq[b] < pq || cuk[b] < pk) return SDPA_ERR_INVALID;
        S.q0.push_back(pq); S.k0.push_back(pk);
        S.lq.push_back(cuq[b] - pq); S.lk.push_back(cuk[b] - pk);
        pq = cuq[b]; pk = cuk[b];
    }
    S.Tq = pq; S.Tk = pk;
    return SDPA_OK;
}

// Head dims (Q/K D, V Dv) with kernels: equal 64, 128 or 192, and D = 192
// with Dv = 128 (the Ascend page: D is 192 or 128, unequal for K and V allowed).
bool nsa_dims_ok(int64_t D, int64_t Dv) {
    return (D == Dv && (D == 64 || D == 128 || D == 192)) || (D == 192 && Dv == 128);
}

// Validation shared by the size query, the backward and the index build
// (Ascend page, "Constraints"): block_size <= 128 and a multiple of 16,
// 1 <= block_count <= 128, count * size < 8192, every KV length a multiple of
// block_size and >= count * size; sparse_mode 2 needs equal lengths.
int check_selected(int64_t batch, const int64_t* cuq, const int64_t* cuk, int64_t Hq, int64_t Hkv,
                   int64_t D, int64_t Dv, int64_t bs, int64_t count, int sparse_mode, Seqs& S,
                   const uint8_t* mask = nullptr, int64_t mask_stride = 0) {
    if (batch < 1 || Hq < 1 || Hkv < 1 || D < 1 || Dv < 1 || Hq % Hkv) return SDPA_ERR_INVALID;
    if (Hq / Hkv > 32) return SDPA_ERR_INVALID;
    if (bs < 16 || bs > 128 || bs % 16) return SDPA_ERR_INVALID;
    if (count < 1 || count > 128 || count * bs >= 8192) return SDPA_ERR_INVALID;
    if (sparse_mode != 0 && sparse_mode != 2) return SDPA_ERR_INVALID;
    if (int s = read_seqs(batch, cuq, cuk, S)) return s;
    int64_t max_lk = 0;
    for (size_t b = 0; b < S.lk.size(); ++b) {
        if (S.lk[b] % bs) return SDPA_ERR_INVALID;
        if (S.lk[b] < count * bs) return SDPA_ERR_INVALID;
        if (sparse_mode == 2 && S.lq[b] != S.lk[b]) return SDPA_ERR_INVALID;
        max_lk = std::max(max_lk, S.lk[b]);
    }
    // a user mask row covers every key position of the longest sequence
    if (mask && mask_stride < max_lk) return SDPA_ERR_INVALID;
    if (!nsa_dims_ok(D, Dv)) return SDPA_ERR_UNSUPPORTED;
    if (mask && ((reinterpret_cast<uintptr_t>(mask) & 15u) || (mask_stride % 16) || mask_stride >= ((int64_t)1 << 31)))
        return SDPA_ERR_UNSUPPORTED;
    if (S.Tq * Hkv * count >= ((int64_t)1 << 31) || S.Tk >= ((int64_t)1 << 31)) return SDPA_ERR_UNSUPPORTED;
    if (S.Tq > 2147483647 || Hkv * ((Hq / Hkv + 15) / 16) > 65535) return SDPA_ERR_UNSUPPORTED;
    return SDPA_OK;
}

// Compute units of the current device (256 if the query fails).
int device_cus() {
    constexpr int kMaxDev = 64;
    static int cached[kMaxDev] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev) return 256;
    if (cached[dev] == 0) {
        int cu = 0;
        if (hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cu <= 0) return 256;
        cached[dev] = cu;
    }
    return cached[dev];
}

NsaLayout nsa_layout(const Seqs& S, int64_t Hq, int64_t Hkv, int64_t D, int64_t Dv, int64_t bs, int64_t count) {
    NsaLayout L;
    L.NB = S.Tk / bs;
    L.nbk = Hkv * L.NB;
    L.E = S.Tq * Hkv * count;
    const int64_t G = Hq / Hkv;
    // Entries per work piece of the dK/dV kernel: k steps of BR rows (BR / G
    // entries each), k chosen to minimise an estimate of the kernel's span,
    // the rounds of pieces over the device's workgroup slots times k steps,
    // plus a small cost per piece for its partial sums (the pieces' count is
    // bounded by one partial piece per bucket).  On the NSA workload (65536
    // entries, 64 buckets, 256 slots) pieces of 16 steps took 199 us, of 12
    // steps 182 us, of 10 steps 197 us and of 8 steps 191 us: the rounds, not
    // the piece length, set the span.  At most 1.5x the pieces (and partial
    // workspace) of the longest pieces.
    const int64_t BR = (D == 128 && Dv == 128) ? 128 : 64;      // the kernel's rows per step
    const int64_t per_step = std::max<int64_t>(1, BR / G);
    const int64_t slots = (int64_t)device_cus() * (D == 64 ? 2 : 1);
    const int64_t kmax = 2048 / BR;                  // a piece's tokens fit the kernel's 2048 / G table
    const int64_t np_cap = 3 * (L.nbk + (L.E + kmax * per_step - 1) / (kmax * per_step)) / 2;
    double best = -1.0;
    for (int64_t k = kmax; k >= 4; --k) {
        const int64_t ch = k * per_step;
        const int64_t np = L.nbk + (L.E + ch - 1) / ch;
        if (k < kmax && np > np_cap) break;
        const double cost = (double)((np + slots - 1) / slots) * k * BR + 0.4 * np;
        if (best < 0.0 || cost < best) {
            best = cost;
            L.chunk = ch;
        }
    }
    L.max_pieces = L.nbk + (L.E + L.chunk - 1) / L.chunk;
    L.halves = (bs + 63) / 64;
    // index tiles: 16 tokens, doubled until blocks x tiles is at most 2^22
    // (the per-tile totals stay within 16 MiB per KV head)
    while (L.NB * ((S.Tq + L.tt - 1) / L.tt) > ((int64_t)1 << 22)) L.tt *= 2;
    L.n_tiles = (S.Tq + L.tt - 1) / L.tt;
    size_t o = 0;
    L.counts = o; o = up(o + L.nbk * 4);
    L.offsets = o; o = up(o + (L.nbk + 1) * 4);
    L.entries = o; o = up(o + std::max<int64_t>(L.E, 1) * 4);
    L.pstart = o; o = up(o + (L.nbk + 1) * 4);
    L.pieces = o; o = up(o + L.max_pieces * 3 * 4);
    L.hist = o; o = up(o + (size_t)Hkv * L.NB * L.n_tiles * 4);
    L.rank = o; o = up(o + std::max<int64_t>(L.E, 1) * 4);
    L.lse2 = o; o = up(o + S.Tq * Hq * 4);
    L.delta = o; o = up(o + S.Tq * Hq * 4);
    L.partial = o; o = up(o + (size_t)L.max_pieces * L.halves * 64 * (D + Dv) * 4);   // dK, dV partials
    // stored dS for a dQ pass without recomputation: 16 query heads per KV
    // head, block sizes that divide 128, up to 1 GiB
    const size_t ds_bytes = (size_t)std::max<int64_t>(L.E, 1) * bs * 16 * 2;
    L.use_ds = G == 16 && 128 % bs == 0 && ds_bytes <= ((size_t)1 << 30);
    L.ds = o; o = up(o + (L.use_ds ? ds_bytes : 0));
    // more sequences than the kernel arguments carry: a table in the workspace
    const int64_t n = (int64_t)S.q0.size();
    L.seqtab = o; o = up(o + (n > sdpa::kMaxSeqArgs ? (size_t)n * 16 : 0));
    L.total = o;
    return L;
}

// Sequences [first, first + n) of S into an argument table.
void fill_seq_chunk(sdpa::SeqTable& t, const Seqs& S, int64_t first, int n) {
    t.n = n;
    t.dev = nullptr;
    for (int i = 0; i < n; ++i) {
        t.q0[i] = (int32_t)S.q0[first + i]; t.k0[i] = (int32_t)S.k0[first + i];
        t.lq[i] = (int32_t)S.lq[first + i]; t.lk[i] = (int32_t)S.lk[first + i];
    }
}

// The kernels' sequence table: in the arguments for up to kMaxSeqArgs
// sequences, else the workspace table at `table` (filled by launch_seqtab).
void fill_seq_table(sdpa::SeqTable& t, const Seqs& S, int32_t* table) {
    const int64_t n = (int64_t)S.q0.size();
    if (n <= sdpa::kMaxSeqArgs) {
        fill_seq_chunk(t, S, 0, (int)n);
        return;
    }
    t.n = (int)n;
    t.dev = table;
}

// Fills the workspace sequence table, kMaxSeqArgs rows per launch (kernels,
// no copies, so the call stays capturable in a graph).
hipError_t launch_seqtab(const Seqs& S, int32_t* table, hipStream_t st) {
    const int64_t n = (int64_t)S.q0.size();
    if (n <= sdpa::kMaxSeqArgs) return hipSuccess;
    for (int64_t c = 0; c < n; c += sdpa::kMaxSeqArgs) {
        sdpa::SeqTable chunk{};
        fill_seq_chunk(chunk, S, c, (int)std::min<int64_t>(sdpa::kMaxSeqArgs, n - c));
        hipLaunchKernelGGL(sdpa::nsa_seqtab_kernel, dim3(1), dim3(64), 0, st, chunk, table, (int)c);
    }
    return hipGetLastError();
}

thread_local std::string g_nsa_err;

int hip_fail(hipError_t e, const char* where) {
    g_nsa_err = std::string(where) + ": " + hipGetErrorString(e);
    sdpa::set_last_error(g_nsa_err.c_str());
    return SDPA_ERR_HIP;
}

int device_ok() {
    int n = 0;
    hipError_t e = hipGetDeviceCount(&n);
    if (e != hipSuccess) return hip_fail(e, "hipGetDeviceCount");
    if (n <= 0) {
        sdpa::set_last_error("no HIP device");
        return SDPA_ERR_HIP;
    }
    return SDPA_OK;
}

// Checked mode (environment SDPA_BWD_CHECK set and not "0", read at every
// call): the selected calls copy the top-k values to the host, a copy that
// synchronises the caller's stream, and reject a value outside its token's
// sequence's blocks with SDPA_ERR_INVALID instead of ignoring that slot.
// (Negative strides are not checked.)
int check_topk(const Seqs& S, int64_t Hkv, const int32_t* topk, int64_t st, int64_t sn, int64_t sk, int64_t bs,
               int64_t count, void* stream) {
    const char* env = std::getenv("SDPA_BWD_CHECK");
    if (!env || !env[0] || env[0] == '0' || S.Tq == 0) return SDPA_OK;
    if (st < 0 || sn < 0 || sk < 0) return SDPA_OK;
    const size_t n = (size_t)((S.Tq - 1) * st + (Hkv - 1) * sn + (count - 1) * sk + 1);
    std::vector<int32_t> h(n);
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = hipMemcpyAsync(h.data(), topk, n * sizeof(int32_t), hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) return hip_fail(e, "top-k check copy");
    for (size_t b = 0; b < S.q0.size(); ++b) {
        const int64_t nblk = S.lk[b] / bs;
        for (int64_t t = S.q0[b]; t < S.q0[b] + S.lq[b]; ++t)
            for (int64_t h2 = 0; h2 < Hkv; ++h2)
                for (int64_t i = 0; i < count; ++i) {
                    const int32_t v = h[(size_t)(t * st + h2 * sn + i * sk)];
                    if (v < 0 || v >= nblk) {
                        g_nsa_err = "topk[" + std::to_string(t) + ", " + std::to_string(h2) + ", " + std::to_string(i) +
                                    "] = " + std::to_string(v) + " is outside the sequence's " + std::to_string(nblk) +
                                    " blocks";
                        sdpa::set_last_error(g_nsa_err.c_str());
                        return SDPA_ERR_INVALID;
                    }
                }
    }
    return SDPA_OK;
}

bool a16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int t3_ok(const sdpa_tensor3* t) {
    if (t->stride_d != 1 || !a16(t->data) || (t->stride_t % 8) || (t->stride_n % 8)) return SDPA_ERR_UNSUPPORTED;
    if (!sdpa::row_stride_ok(t->stride_t) || !sdpa::row_stride_ok(t->stride_n)) return SDPA_ERR_UNSUPPORTED;
    return SDPA_OK;
}

sdpa::TensorArg arg(const sdpa_tensor3* t) {
    return sdpa::TensorArg{static_cast<uint16_t*>(t->data), 0, t->stride_n, t->stride_t};
}

}  // namespace

extern "C" {

int sdpa_bwd_selected_workspace_size(int dtype, int64_t batch, const int64_t* cu_seqlens_q_host,
                                     const int64_t* cu_seqlens_kv_host, int64_t Hq, int64_t Hkv,
                                     int64_t D, int64_t Dv, int64_t block_size, int64_t block_count,
                                     int deterministic, size_t* bytes) {
    if (!bytes || !cu_seqlens_q_host || !cu_seqlens_kv_host) return SDPA_ERR_NULLPTR;
    if (dtype != SDPA_F16 && dtype != SDPA_BF16) return SDPA_ERR_INVALID;
    if (deterministic < 0 || deterministic > 2) return SDPA_ERR_INVALID;
    Seqs S;
    if (int s = check_selected(batch, cu_seqlens_q_host, cu_seqlens_kv_host, Hq, Hkv, D, Dv, block_size,
                               block_count, 0, S))
        return s;
    *bytes = nsa_layout(S, Hq, Hkv, D, Dv, block_size, block_count).total;
    return SDPA_OK;
}

static void fill_index_params(sdpa::NsaParams& p, const Seqs& S, const NsaLayout& L, char* ws, const int32_t* topk,
                              int64_t st, int64_t sn, int64_t sk, int64_t Hq, int64_t Hkv, int64_t bs, int64_t count) {
    p.topk = topk; p.tk_st = st; p.tk_sn = sn; p.tk_sk = sk;
    p.count = (int)count; p.bs = (int)bs; p.N2 = (int)Hkv; p.NB = (int)L.NB;
    p.G = (int)(Hq / Hkv); p.Hq = (int)Hq;
    p.g_mul = (65536 + p.G - 1) / p.G;
    p.chunk = (int)L.chunk; p.max_pieces = (int)L.max_pieces;
    fill_seq_table(p.seqs, S, reinterpret_cast<int32_t*>(ws + L.seqtab));
    p.counts = reinterpret_cast<int32_t*>(ws + L.counts);
    p.offsets = reinterpret_cast<int32_t*>(ws + L.offsets);
    p.entries = reinterpret_cast<int32_t*>(ws + L.entries);
    p.pstart = reinterpret_cast<int32_t*>(ws + L.pstart);
    p.pieces = reinterpret_cast<int32_t*>(ws + L.pieces);
    p.tt = (int)L.tt; p.n_tiles = (int)L.n_tiles;
    p.hist = reinterpret_cast<int32_t*>(ws + L.hist);
    p.rank = reinterpret_cast<int32_t*>(ws + L.rank);
    p.halves = (int)L.halves;
    p.Tq = (int)S.Tq;
}

int sdpa_fwd_selected(int dtype, int64_t batch, const int64_t* cu_seqlens_q_host,
                      const int64_t* cu_seqlens_kv_host, int64_t Hq, int64_t Hkv, int64_t D, int64_t Dv,
                      double scale, int sparse_mode, const uint8_t* atten_mask, int64_t atten_mask_stride,
                      const int32_t* topk, int64_t tk_st,
                      int64_t tk_sn, int64_t tk_sk, int64_t block_size, int64_t block_count,
                      const sdpa_tensor3* q, const sdpa_tensor3* k, const sdpa_tensor3* v,
                      const sdpa_tensor3* o_out, float* max_out, float* sum_out,
                      int64_t stats_stride_s, int64_t stats_stride_h, void* stream) {
    if (!cu_seqlens_q_host || !cu_seqlens_kv_host || !topk) return SDPA_ERR_NULLPTR;
    if (!q || !k || !v || !o_out || !max_out || !sum_out) return SDPA_ERR_NULLPTR;
    for (const sdpa_tensor3* t : {q, k, v, o_out})
        if (!t->data) return SDPA_ERR_NULLPTR;
    if (dtype != SDPA_F16 && dtype != SDPA_BF16) return SDPA_ERR_INVALID;
    if (!std::isfinite(scale)) return SDPA_ERR_INVALID;
    Seqs S;
    if (int s = check_selected(batch, cu_seqlens_q_host, cu_seqlens_kv_host, Hq, Hkv, D, Dv, block_size,
                               block_count, sparse_mode, S, atten_mask, atten_mask_stride))
        return s;
    for (const sdpa_tensor3* t : {q, k, v, o_out})
        if (int s = t3_ok(t)) return s;
    if (int s = device_ok()) return s;
    if (int s = check_topk(S, Hkv, topk, tk_st, tk_sn, tk_sk, block_size, block_count, stream)) return s;
    if (S.Tq == 0) return SDPA_OK;

    sdpa::NsaParams p{};
    p.topk = topk; p.tk_st = tk_st; p.tk_sn = tk_sn; p.tk_sk = tk_sk;
    p.count = (int)block_count; p.bs = (int)block_size; p.N2 = (int)Hkv;
    p.G = (int)(Hq / Hkv); p.Hq = (int)Hq;
    p.Tq = (int)S.Tq;
    p.q = arg(q); p.k = arg(k); p.v = arg(v); p.o = arg(o_out);
    p.m_out = max_out; p.l_out = sum_out;
    p.st_ss = stats_stride_s; p.st_sh = stats_stride_h;
    p.sparse_mode = sparse_mode;
    p.mask = atten_mask; p.mask_ss = atten_mask_stride;
    p.scale = (float)scale;
    p.scale_log2 = (float)(scale * 1.4426950408889634);
    hipStream_t st = static_cast<hipStream_t>(stream);
    // one launch per kMaxSeqArgs sequences (the forward has no workspace for
    // a sequence table), over those sequences' tokens
    const int64_t n = (int64_t)S.q0.size();
    for (int64_t c = 0; c < n; c += sdpa::kMaxSeqArgs) {
        const int m = (int)std::min<int64_t>(sdpa::kMaxSeqArgs, n - c);
        fill_seq_chunk(p.seqs, S, c, m);
        p.t_base = (int)S.q0[c];
        p.Tq = (int)(S.q0[c + m - 1] + S.lq[c + m - 1] - S.q0[c]);   // tokens of this launch
        if (p.Tq == 0) continue;
        hipError_t e;
        if (dtype == SDPA_F16)
            e = sdpa::launch_nsa_fwd_dims<sdpa::F16>(p, (int)D, (int)Dv, st);
        else
            e = sdpa::launch_nsa_fwd_dims<sdpa::BF16>(p, (int)D, (int)Dv, st);
        if (e != hipSuccess) return hip_fail(e, "selected forward launch");
    }
    return SDPA_OK;
}

int sdpa_bwd_selected(int dtype, int64_t batch, const int64_t* cu_seqlens_q_host,
                      const int64_t* cu_seqlens_kv_host, int64_t Hq, int64_t Hkv, int64_t D, int64_t Dv,
                      double scale, int sparse_mode, const uint8_t* atten_mask, int64_t atten_mask_stride,
                      const int32_t* topk, int64_t tk_st,
                      int64_t tk_sn, int64_t tk_sk, int64_t block_size, int64_t block_count,
                      int deterministic, int grad_dtype,
                      const sdpa_tensor3* q, const sdpa_tensor3* k, const sdpa_tensor3* v,
                      const sdpa_tensor3* o, const sdpa_tensor3* dout, const sdpa_stats* stats,
                      const sdpa_tensor3* dq, const sdpa_tensor3* dk, const sdpa_tensor3* dv,
                      void* workspace, size_t workspace_bytes, void* stream) {
    if (!cu_seqlens_q_host || !cu_seqlens_kv_host || !topk) return SDPA_ERR_NULLPTR;
    if (!q || !k || !v || !o || !dout || !stats || !dq || !dk || !dv) return SDPA_ERR_NULLPTR;
    for (const sdpa_tensor3* t : {q, k, v, o, dout, dq, dk, dv})
        if (!t->data) return SDPA_ERR_NULLPTR;
    if (!stats->lse_or_max || (stats->kind == SDPA_STATS_MAX_SUM && !stats->sum)) return SDPA_ERR_NULLPTR;
    if (!workspace) return SDPA_ERR_NULLPTR;
    if (dtype != SDPA_F16 && dtype != SDPA_BF16) return SDPA_ERR_INVALID;
    if (grad_dtype != dtype && grad_dtype != SDPA_F32) return SDPA_ERR_INVALID;
    if (!std::isfinite(scale)) return SDPA_ERR_INVALID;
    // every kernel of this path is deterministic, whatever dQ mode is asked for
    if (deterministic < 0 || deterministic > 2) return SDPA_ERR_INVALID;
    if (stats->kind != SDPA_STATS_LSE && stats->kind != SDPA_STATS_MAX_SUM) return SDPA_ERR_INVALID;
    Seqs S;
    if (int s = check_selected(batch, cu_seqlens_q_host, cu_seqlens_kv_host, Hq, Hkv, D, Dv, block_size,
                               block_count, sparse_mode, S, atten_mask, atten_mask_stride))
        return s;
    for (const sdpa_tensor3* t : {q, k, v, o, dout, dq, dk, dv})
        if (int s = t3_ok(t)) return s;
    if (!sdpa::row_stride_ok(stats->stride_s)) return SDPA_ERR_UNSUPPORTED;
    const NsaLayout L = nsa_layout(S, Hq, Hkv, D, Dv, block_size, block_count);
    if (workspace_bytes < L.total) return SDPA_ERR_WORKSPACE;
    if (int s = device_ok()) return s;
    if (int s = check_topk(S, Hkv, topk, tk_st, tk_sn, tk_sk, block_size, block_count, stream)) return s;
    if (S.Tk == 0) return SDPA_OK;

    char* ws = static_cast<char*>(workspace);
    sdpa::NsaParams p{};
    fill_index_params(p, S, L, ws, topk, tk_st, tk_sn, tk_sk, Hq, Hkv, block_size, block_count);
    p.q = arg(q); p.k = arg(k); p.v = arg(v); p.dout = arg(dout);
    p.dq = arg(dq); p.dk = arg(dk); p.dv = arg(dv);
    p.grad_f32 = grad_dtype == SDPA_F32;
    p.lse2 = reinterpret_cast<float*>(ws + L.lse2);
    p.delta = reinterpret_cast<float*>(ws + L.delta);
    p.partial = reinterpret_cast<float*>(ws + L.partial);
    p.ds = L.use_ds ? reinterpret_cast<uint16_t*>(ws + L.ds) : nullptr;
    p.sparse_mode = sparse_mode;
    p.mask = atten_mask; p.mask_ss = atten_mask_stride;
    p.scale = (float)scale;
    p.scale_log2 = (float)(scale * 1.4426950408889634);

    // row statistics in the packed layout (the dense preprocess kernel)
    sdpa::BwdParams bp{};
    bp.o = arg(o); bp.dout = arg(dout);
    bp.stats_kind = stats->kind; bp.st_a = stats->lse_or_max; bp.st_b = stats->sum;
    bp.st_sb = 0; bp.st_sh = stats->stride_h; bp.st_ss = stats->stride_s;
    bp.lse2 = const_cast<float*>(p.lse2);
    bp.delta = const_cast<float*>(p.delta);
    bp.dqacc = nullptr;
    bp.Hq = (int)Hq; bp.Hkv = (int)Hkv; bp.Sq = (int)S.Tq; bp.Sk = (int)S.Tk;
    bp.rows = S.Tq * Hq;
    bp.varlen = 1;
    hipStream_t st = static_cast<hipStream_t>(stream);
    hipError_t e = launch_seqtab(S, reinterpret_cast<int32_t*>(ws + L.seqtab), st);
    if (e != hipSuccess) return hip_fail(e, "sequence table launch");
    if (dtype == SDPA_F16)
        e = sdpa::launch_nsa_dims<sdpa::F16>(p, bp, (int)D, (int)Dv, st);
    else
        e = sdpa::launch_nsa_dims<sdpa::BF16>(p, bp, (int)D, (int)Dv, st);
    if (e != hipSuccess) return hip_fail(e, "selected launch");
    return SDPA_OK;
}

int sdpa_selected_build_index(int64_t batch, const int64_t* cu_seqlens_q_host,
                              const int64_t* cu_seqlens_kv_host, int64_t Hkv,
                              const int32_t* topk, int64_t tk_st, int64_t tk_sn, int64_t tk_sk,
                              int64_t block_size, int64_t block_count,
                              int32_t* offsets_out, int32_t* entries_out,
                              void* workspace, size_t workspace_bytes, void* stream) {
    if (!cu_seqlens_q_host || !cu_seqlens_kv_host || !topk || !offsets_out || !entries_out || !workspace)
        return SDPA_ERR_NULLPTR;
    Seqs S;
    if (int s = check_selected(batch, cu_seqlens_q_host, cu_seqlens_kv_host, Hkv, Hkv, 128, 128, block_size,
                               block_count, 0, S))
        return s;
    const NsaLayout L = nsa_layout(S, Hkv, Hkv, 128, 128, block_size, block_count);
    if (workspace_bytes < L.total) return SDPA_ERR_WORKSPACE;
    if (int s = device_ok()) return s;
    if (int s = check_topk(S, Hkv, topk, tk_st, tk_sn, tk_sk, block_size, block_count, stream)) return s;
    if (L.nbk == 0) return SDPA_OK;
    char* ws = static_cast<char*>(workspace);
    sdpa::NsaParams p{};
    fill_index_params(p, S, L, ws, topk, tk_st, tk_sn, tk_sk, Hkv, Hkv, block_size, block_count);
    p.offsets = offsets_out;
    p.entries = entries_out;
    hipError_t e = launch_seqtab(S, reinterpret_cast<int32_t*>(ws + L.seqtab), static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "sequence table launch");
    e = sdpa::launch_index(p, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "index launch");
    return SDPA_OK;
}

}  // extern "C"

#endif  // SDPA_NSA_KV_UNIT
