// C-ABI host side of libsdpa_bwd: argument validation, workspace carving and
// kernel launches on the caller's stream.  No device memory is allocated and
// nothing synchronises.  Status codes and the validation order are documented
// in include/sdpa_bwd.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/sdpa_bwd.h"
#include "common.h"
#include "kernels.h"

// Scratch of sdpa_bwd_noalloc (16 MiB per GPU; see scratch_address below).
constexpr size_t kScratchBytes = size_t(16) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

thread_local std::string g_last_error;

int fail_hip(hipError_t e, const char* where) {
    g_last_error = std::string(where) + ": " + hipGetErrorString(e);
    return SDPA_ERR_HIP;
}

int set_err(int code, const char* msg) {
    g_last_error = msg;
    return code;
}

bool log_enabled() {
    static int on = -1;
    if (on < 0) {
        const char* s = std::getenv("SDPA_BWD_LOG");
        on = (s && s[0] && s[0] != '0') ? 1 : 0;
    }
    return on == 1;
}

int check_device() {
    int n = 0;
    hipError_t e = hipGetDeviceCount(&n);
    if (e != hipSuccess) return fail_hip(e, "hipGetDeviceCount");
    if (n <= 0) return set_err(SDPA_ERR_HIP, "no HIP device");
    return SDPA_OK;
}

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// A strided 16-bit tensor is usable when d-stride is 1 and every row starts on
// a 16-byte boundary (base aligned, other strides multiples of 8 elements).
int tensor4_ok(const sdpa_tensor4* t) {
    if (t->stride_d != 1) return SDPA_ERR_UNSUPPORTED;
    if (!aligned16(t->data)) return SDPA_ERR_UNSUPPORTED;
    if ((t->stride_b % 8) || (t->stride_h % 8) || (t->stride_s % 8)) return SDPA_ERR_UNSUPPORTED;
    if (!sdpa::row_stride_ok(t->stride_s)) return SDPA_ERR_UNSUPPORTED;
    return SDPA_OK;
}

int tensor3_ok(const sdpa_tensor3* t) {
    if (t->stride_d != 1) return SDPA_ERR_UNSUPPORTED;
    if (!aligned16(t->data)) return SDPA_ERR_UNSUPPORTED;
    if ((t->stride_t % 8) || (t->stride_n % 8)) return SDPA_ERR_UNSUPPORTED;
    if (!sdpa::row_stride_ok(t->stride_t)) return SDPA_ERR_UNSUPPORTED;
    return SDPA_OK;
}

sdpa::TensorArg arg4(const sdpa_tensor4* t) {
    return sdpa::TensorArg{static_cast<uint16_t*>(t->data), t->stride_b, t->stride_h, t->stride_s};
}

sdpa::TensorArg arg3(const sdpa_tensor3* t) {
    return sdpa::TensorArg{static_cast<uint16_t*>(t->data), 0, t->stride_n, t->stride_t};
}

constexpr int64_t kMaxLen = (int64_t)1 << 30;
constexpr int64_t kMaxGridY = 65535;

struct Carve {
    size_t lse2 = 0, delta = 0, dqacc = 0, total = 0;
};

Carve carve_bwd(int64_t rows, int64_t D, bool deterministic) {
    Carve c;
    c.lse2 = 0;
    c.delta = align_up(c.lse2 + (size_t)rows * 4);
    c.dqacc = align_up(c.delta + (size_t)rows * 4);
    c.total = deterministic ? c.dqacc : align_up(c.dqacc + (size_t)rows * (size_t)D * 4);
    if (c.total == 0) c.total = kAlign;
    return c;
}

// dQ mode of the dense and packed entry points: 0 = the library's fastest
// method, 1 = bitwise reproducible, 2 = fp32 atomic accumulation (FA2's
// method).  The fastest method is the atomic-free one at every head size.
bool dq_mode_ok(int mode) { return mode >= 0 && mode <= 2; }
bool dq_atomic(int mode, int64_t D) { (void)D; return mode == 2; }

// Head dims of the dense and packed paths: D of Q and K, Dv of V, O and dO,
// equal (64, 128, 192) or (192, 128), the pair the Ascend page names.  At
// D = 192 the key-tile kernel's tiles take 102 KB of LDS, which leaves no
// room for the K and dS^T tiles of the atomic dQ form: dQ mode 2 is not
// offered there.
bool dense_dims_ok(int64_t D, int64_t Dv) {
    return (D == Dv && (D == 64 || D == 128 || D == 192)) || (D == 192 && Dv == 128);
}
bool dense_mode_ok(int mode, int64_t D, int64_t Dv) { return !(mode == 2 && (D == 192 || Dv != D)); }

int check_stats(const sdpa_stats* s) {
    if (!s->lse_or_max) return SDPA_ERR_NULLPTR;
    if (s->kind == SDPA_STATS_MAX_SUM && !s->sum) return SDPA_ERR_NULLPTR;
    return SDPA_OK;
}

int check_stats_kind(const sdpa_stats* s) {
    if (s->kind != SDPA_STATS_LSE && s->kind != SDPA_STATS_MAX_SUM) return SDPA_ERR_INVALID;
    return SDPA_OK;
}

int check_stats_stride(const sdpa_stats* s) {
    return sdpa::row_stride_ok(s->stride_s) ? SDPA_OK : SDPA_ERR_UNSUPPORTED;
}

void fill_stats(sdpa::BwdParams& p, const sdpa_stats* s) {
    p.stats_kind = s->kind;
    p.st_a = s->lse_or_max;
    p.st_b = s->sum;
    p.st_sb = s->stride_b;
    p.st_sh = s->stride_h;
    p.st_ss = s->stride_s;
}

// Packed-batch description checked from the host arrays.
struct Packed {
    std::vector<int64_t> q0, k0, lq, lk;
    int64_t Tq = 0, Tk = 0, max_lq = 0, max_lk = 0;
};

int read_packed(int64_t batch, const int64_t* cuq, const int64_t* cuk, Packed& P) {
    int64_t pq = 0, pk = 0;
    for (int64_t b = 0; b < batch; ++b) {
        const int64_t eq = cuq[b], ek = cuk[b];
        if (eq < pq || ek < pk) return SDPA_ERR_INVALID;
        const int64_t lq = eq - pq, lk = ek - pk;
        if (lq >= kMaxLen || lk >= kMaxLen) return SDPA_ERR_UNSUPPORTED;
        P.q0.push_back(pq); P.k0.push_back(pk); P.lq.push_back(lq); P.lk.push_back(lk);
        P.max_lq = std::max(P.max_lq, lq);
        P.max_lk = std::max(P.max_lk, lk);
        pq = eq; pk = ek;
    }
    P.Tq = pq; P.Tk = pk;
    if (P.Tq >= ((int64_t)1 << 31) || P.Tk >= ((int64_t)1 << 31)) return SDPA_ERR_UNSUPPORTED;
    return SDPA_OK;
}

// Scratch of sdpa_bwd_noalloc: the per-row log2-LSE and Delta (and, in dQ
// mode 2, the fp32 dQ accumulator) live in this fixed array instead of a
// caller workspace.  Each GPU the library runs on holds its own copy, at its
// own address, until the process ends.  In host code the name `scratch` only
// stands in for the symbol; kernels get the device address that
// hipGetSymbolAddress returns, fetched once per device.

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices] = {};

// Device address of the current device's scratch array.
int scratch_address(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail_hip(e, "hipGetDevice");
    if (dev < 0 || dev >= kMaxScratchDevices) return set_err(SDPA_ERR_UNSUPPORTED, "device ordinal above 63");
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return fail_hip(e, "hipGetSymbolAddress(scratch)");
        if (!p) return set_err(SDPA_ERR_HIP, "hipGetSymbolAddress(scratch) returned null");
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return SDPA_OK;
}

}  // namespace

namespace sdpa {
void set_last_error(const char* msg) { g_last_error = msg ? msg : ""; }
}  // namespace sdpa

extern "C" {

const char* sdpa_status_string(int status) {
    switch (status) {
        case SDPA_OK: return "ok";
        case SDPA_ERR_NULLPTR: return "null pointer argument";
        case SDPA_ERR_INVALID: return "invalid argument";
        case SDPA_ERR_UNSUPPORTED: return "unsupported argument (head dim, stride, alignment or size)";
        case SDPA_ERR_WORKSPACE: return "workspace too small";
        case SDPA_ERR_HIP: return g_last_error.empty() ? "HIP error" : g_last_error.c_str();
        default: return "unknown status";
    }
}

const char* sdpa_last_error(void) { return g_last_error.c_str(); }

// ---------------------------------------------------------------------------
// Forward statistics
// ---------------------------------------------------------------------------

int sdpa_fwd_stats(int dtype, int64_t B, int64_t Hq, int64_t Hkv, int64_t Sq, int64_t Sk,
                   int64_t D, int64_t Dv, double scale, int causal,
                   const sdpa_tensor4* q, const sdpa_tensor4* k, const sdpa_tensor4* v,
                   const sdpa_tensor4* o_out, const sdpa_stats_out* lse_out, void* stream) {
    if (!q || !k || !v || !o_out || !lse_out) return SDPA_ERR_NULLPTR;
    if (!q->data || !k->data || !v->data || !o_out->data || !lse_out->lse) return SDPA_ERR_NULLPTR;
    if (dtype != SDPA_F16 && dtype != SDPA_BF16) return SDPA_ERR_INVALID;
    if (B < 0 || Sq < 0 || Sk < 0 || Hq < 1 || Hkv < 1 || D < 1 || Dv < 1) return SDPA_ERR_INVALID;
    if (Hq % Hkv) return SDPA_ERR_INVALID;
    if (!std::isfinite(scale)) return SDPA_ERR_INVALID;
    if (!dense_dims_ok(D, Dv)) return SDPA_ERR_UNSUPPORTED;
    for (const sdpa_tensor4* t : {q, k, v, o_out})
        if (int s = tensor4_ok(t)) return s;
    if (Sq >= kMaxLen || Sk >= kMaxLen || B * Hq > kMaxGridY) return SDPA_ERR_UNSUPPORTED;
    if (int s = check_device()) return s;
    if (B == 0 || Sq == 0) return SDPA_OK;

    sdpa::FwdParams p{};
    p.q = arg4(q); p.k = arg4(k); p.v = arg4(v); p.o = arg4(o_out);
    p.lse = lse_out->lse;
    p.lse_sb = lse_out->stride_b; p.lse_sh = lse_out->stride_h; p.lse_ss = lse_out->stride_s;
    p.B = (int)B; p.Hq = (int)Hq; p.Hkv = (int)Hkv; p.Sq = (int)Sq; p.Sk = (int)Sk;
    p.scale_log2 = (float)(scale * 1.4426950408889634);
    hipError_t e = sdpa::launch_fwd(p, dtype, (int)D, (int)Dv, (int)Sq, causal != 0, static_cast<hipStream_t>(stream));
    if (log_enabled())
        std::fprintf(stderr, "[sdpa_bwd] fwd_stats dtype=%d B=%lld Hq=%lld Hkv=%lld Sq=%lld Sk=%lld D=%lld Dv=%lld causal=%d grid=(%lld,%lld)\n",
                     dtype, (long long)B, (long long)Hq, (long long)Hkv, (long long)Sq, (long long)Sk,
                     (long long)D, (long long)Dv, causal, (long long)((Sq + 127) / 128), (long long)(B * Hq));
    if (e != hipSuccess) return fail_hip(e, "fwd launch");
    return SDPA_OK;
}

int sdpa_fwd_stats_varlen(int dtype, int64_t batch, const int64_t* cu_seqlens_q_host,
                          const int64_t* cu_seqlens_kv_host, int64_t Hq, int64_t Hkv, int64_t D, int64_t Dv,
                          double scale, int causal, const sdpa_tensor3* q, const sdpa_tensor3* k,
                          const sdpa_tensor3* v, const sdpa_tensor3* o_out, const sdpa_stats_out* lse_out,
                          void* stream) {
    if (!cu_seqlens_q_host || !cu_seqlens_kv_host) return SDPA_ERR_NULLPTR;
    if (!q || !k || !v || !o_out || !lse_out) return SDPA_ERR_NULLPTR;
    if (!q->data || !k->data || !v->data || !o_out->data || !lse_out->lse) return SDPA_ERR_NULLPTR;
    if (dtype != SDPA_F16 && dtype != SDPA_BF16) return SDPA_ERR_INVALID;
    if (batch < 1 || Hq < 1 || Hkv < 1 || D < 1 || Dv < 1 || Hq % Hkv) return SDPA_ERR_INVALID;
    if (!std::isfinite(scale)) return SDPA_ERR_INVALID;
    Packed P;
    if (int s = read_packed(batch, cu_seqlens_q_host, cu_seqlens_kv_host, P)) return s;
    if (!dense_dims_ok(D, Dv)) return SDPA_ERR_UNSUPPORTED;
    for (const sdpa_tensor3* t : {q, k, v, o_out})
        if (int s = tensor3_ok(t)) return s;
    if (std::min<int64_t>(batch, sdpa::kMaxSeqArgs) * Hq > kMaxGridY) return SDPA_ERR_UNSUPPORTED;
    if (int s = check_device()) return s;
    if (P.Tq == 0) return SDPA_OK;

    sdpa::FwdParams p{};
    p.q = arg3(q); p.k = arg3(k); p.v = arg3(v); p.o = arg3(o_out);
    p.lse = lse_out->lse;
    p.lse_sb = 0; p.lse_sh = lse_out->stride_h; p.lse_ss = lse_out->stride_s;
    p.Hq = (int)Hq; p.Hkv = (int)Hkv; p.Sq = (int)P.Tq; p.Sk = (int)P.Tk;
    p.scale_log2 = (float)(scale * 1.4426950408889634);
    p.varlen = 1;
    // one launch per chunk of up to kMaxSeqArgs sequences
    const int64_t n = (int64_t)P.q0.size();
    for (int64_t c0 = 0; c0 < n; c0 += sdpa::kMaxSeqArgs) {
        const int64_t c1 = std::min<int64_t>(n, c0 + sdpa::kMaxSeqArgs);
        int64_t mlq = 0;
        p.seqs.n = (int)(c1 - c0);
        p.seqs.dev = nullptr;
        for (int64_t b = c0; b < c1; ++b) {
            p.seqs.q0[b - c0] = (int32_t)P.q0[b];
            p.seqs.k0[b - c0] = (int32_t)P.k0[b];
            p.seqs.lq[b - c0] = (int32_t)P.lq[b];
            p.seqs.lk[b - c0] = (int32_t)P.lk[b];
            mlq = std::max(mlq, P.lq[b]);
        }
        p.B = (int)(c1 - c0);
        if (mlq == 0) continue;
        hipError_t e = sdpa::launch_fwd(p, dtype, (int)D, (int)Dv, (int)mlq, causal != 0, static_cast<hipStream_t>(stream));
        if (e != hipSuccess) return fail_hip(e, "fwd varlen launch");
    }
    return SDPA_OK;
}

// ---------------------------------------------------------------------------
// Dense backward
// ---------------------------------------------------------------------------

int sdpa_bwd_workspace_size(int dtype, int64_t B, int64_t Hq, int64_t Hkv, int64_t Sq,
                            int64_t Sk, int64_t D, int64_t Dv, int deterministic, size_t* bytes) {
    if (!bytes) return SDPA_ERR_NULLPTR;
    if (dtype != SDPA_F16 && dtype != SDPA_BF16) return SDPA_ERR_INVALID;
    if (B < 0 || Sq < 0 || Sk < 0 || Hq < 1 || Hkv < 1 || D < 1 || Dv < 1 || Hq % Hkv) return SDPA_ERR_INVALID;
    if (!dq_mode_ok(deterministic)) return SDPA_ERR_INVALID;
    if (!dense_dims_ok(D, Dv) || !dense_mode_ok(deterministic, D, Dv)) return SDPA_ERR_UNSUPPORTED;
    *bytes = carve_bwd(B * Hq * Sq, D, !dq_atomic(deterministic, D)).total;
    return SDPA_OK;
}

static int run_bwd(int dtype, sdpa::BwdParams& p, int64_t D, int64_t Dv, bool causal, bool det,
                   const Packed* packed, int64_t B, int64_t Sq, int64_t Sk, hipStream_t st) {
    sdpa::BwdLaunch L{};
    L.dtype = dtype; L.D = (int)D; L.Dv = (int)Dv; L.causal = causal; L.deterministic = det;
    if (!packed) {
        p.varlen = 0;
        p.seqs.n = 0;
        p.seqs.dev = nullptr;
        L.n_seq = (int)B;
        L.max_kv_tiles = (int)((Sk + 127) / 128);
        L.max_kv_tiles64 = (int)((Sk + 63) / 64);
        L.max_q_tiles128 = (int)((Sq + 127) / 128);
        L.max_q_tiles64 = (int)((Sq + 63) / 64);
        hipError_t e = sdpa::launch_bwd(p, L, st);
        if (e != hipSuccess) return fail_hip(e, "bwd launch");
        return SDPA_OK;
    }
    // Packed: launch per chunk of up to kMaxSeqArgs sequences; the row-wise
    // kernels cover all rows on the first chunk only.  Sequences go longest
    // (most key rows, then query rows) first: every sequence carries its own
    // row offsets, so the order is free, and the kernels take their units in
    // table order.
    p.varlen = 1;
    const int64_t n = (int64_t)packed->q0.size();
    std::vector<int64_t> order((size_t)n);
    for (int64_t b = 0; b < n; ++b) order[(size_t)b] = b;
    std::stable_sort(order.begin(), order.end(), [&](int64_t a, int64_t c) {
        return packed->lk[a] != packed->lk[c] ? packed->lk[a] > packed->lk[c] : packed->lq[a] > packed->lq[c];
    });
    for (int64_t c0 = 0; c0 < n; c0 += sdpa::kMaxSeqArgs) {
        const int64_t c1 = std::min<int64_t>(n, c0 + sdpa::kMaxSeqArgs);
        int64_t mlq = 0, mlk = 0;
        p.seqs.n = (int)(c1 - c0);
        p.seqs.dev = nullptr;
        for (int64_t i = c0; i < c1; ++i) {
            const size_t b = (size_t)order[(size_t)i];
            p.seqs.q0[i - c0] = (int32_t)packed->q0[b];
            p.seqs.k0[i - c0] = (int32_t)packed->k0[b];
            p.seqs.lq[i - c0] = (int32_t)packed->lq[b];
            p.seqs.lk[i - c0] = (int32_t)packed->lk[b];
            mlq = std::max(mlq, packed->lq[b]);
            mlk = std::max(mlk, packed->lk[b]);
        }
        L.n_seq = (int)(c1 - c0);
        L.max_kv_tiles = (int)((mlk + 127) / 128);
        L.max_kv_tiles64 = (int)((mlk + 63) / 64);
        L.max_q_tiles128 = (int)((mlq + 127) / 128);
        L.max_q_tiles64 = (int)((mlq + 63) / 64);
        L.phase = (c0 == 0 ? sdpa::BwdLaunch::kFirst : 0) | (c1 == n ? sdpa::BwdLaunch::kLast : 0);
        hipError_t e = sdpa::launch_bwd(p, L, st);
        if (e != hipSuccess) return fail_hip(e, "bwd launch");
    }
    return SDPA_OK;
}

// The dense backward behind both entry points: `workspace` is the caller's
// buffer (sdpa_bwd), or null for the library's own scratch array
// (sdpa_bwd_noalloc), which is fetched only once the arguments are valid.
static int bwd_dense(int dtype, int64_t B, int64_t Hq, int64_t Hkv, int64_t Sq, int64_t Sk, int64_t D, int64_t Dv,
                     double scale, int causal, int deterministic, int grad_dtype,
                     const sdpa_tensor4* q, const sdpa_tensor4* k, const sdpa_tensor4* v,
                     const sdpa_tensor4* o, const sdpa_tensor4* dout, const sdpa_stats* stats,
                     const sdpa_tensor4* dq, const sdpa_tensor4* dk, const sdpa_tensor4* dv,
                     void* workspace, size_t workspace_bytes, bool scratch, void* stream) {
    if (!q || !k || !v || !o || !dout || !stats || !dq || !dk || !dv) return SDPA_ERR_NULLPTR;
    for (const sdpa_tensor4* t : {q, k, v, o, dout, dq, dk, dv})
        if (!t->data) return SDPA_ERR_NULLPTR;
    if (int s = check_stats(stats)) return s;
    if (!scratch && !workspace) return SDPA_ERR_NULLPTR;
    if (dtype != SDPA_F16 && dtype != SDPA_BF16) return SDPA_ERR_INVALID;
    if (grad_dtype != dtype && grad_dtype != SDPA_F32) return SDPA_ERR_INVALID;
    if (B < 0 || Sq < 0 || Sk < 0 || Hq < 1 || Hkv < 1 || D < 1 || Dv < 1) return SDPA_ERR_INVALID;
    if (Hq % Hkv) return SDPA_ERR_INVALID;
    if (!std::isfinite(scale)) return SDPA_ERR_INVALID;
    if (!dq_mode_ok(deterministic)) return SDPA_ERR_INVALID;
    if (int s = check_stats_kind(stats)) return s;
    if (!dense_dims_ok(D, Dv) || !dense_mode_ok(deterministic, D, Dv)) return SDPA_ERR_UNSUPPORTED;
    for (const sdpa_tensor4* t : {q, k, v, o, dout, dq, dk, dv})
        if (int s = tensor4_ok(t)) return s;
    if (int s = check_stats_stride(stats)) return s;
    if (Sq >= kMaxLen || Sk >= kMaxLen || (Sk + 127) / 128 > kMaxGridY || B * Hq > kMaxGridY)
        return SDPA_ERR_UNSUPPORTED;
    const bool det = !dq_atomic(deterministic, D);
    const int64_t rows = B * Hq * Sq;
    const Carve cv = carve_bwd(rows, D, det);
    if (scratch && cv.total > kScratchBytes) {
        g_last_error = "sdpa_bwd_noalloc: the problem needs " + std::to_string(cv.total) +
                       " bytes of scratch, above the library's fixed " + std::to_string(kScratchBytes) +
                       " bytes; call sdpa_bwd with a workspace";
        return SDPA_ERR_WORKSPACE;
    }
    if (!scratch && workspace_bytes < cv.total) return SDPA_ERR_WORKSPACE;
    if (int s = check_device()) return s;
    if (B == 0) return SDPA_OK;
    if (scratch) {
        if (int s = scratch_address(&workspace)) return s;
    }

    char* ws = static_cast<char*>(workspace);
    sdpa::BwdParams p{};
    p.q = arg4(q); p.k = arg4(k); p.v = arg4(v); p.o = arg4(o); p.dout = arg4(dout);
    p.dq = arg4(dq); p.dk = arg4(dk); p.dv = arg4(dv);
    p.grad_f32 = grad_dtype == SDPA_F32;
    fill_stats(p, stats);
    p.lse2 = reinterpret_cast<float*>(ws + cv.lse2);
    p.delta = reinterpret_cast<float*>(ws + cv.delta);
    p.dqacc = det ? nullptr : reinterpret_cast<float*>(ws + cv.dqacc);
    p.B = (int)B; p.Hq = (int)Hq; p.Hkv = (int)Hkv; p.Sq = (int)Sq; p.Sk = (int)Sk;
    p.rows = rows;
    p.scale = (float)scale;
    p.scale_log2 = (float)(scale * 1.4426950408889634);
    if (log_enabled())
        std::fprintf(stderr, "[sdpa_bwd] bwd%s dtype=%d B=%lld Hq=%lld Hkv=%lld Sq=%lld Sk=%lld D=%lld Dv=%lld causal=%d det=%d main_grid=(%lld,%lld)\n",
                     scratch ? "_noalloc" : "", dtype, (long long)B, (long long)Hq, (long long)Hkv, (long long)Sq,
                     (long long)Sk, (long long)D, (long long)Dv, causal, (int)det, (long long)(B * Hkv), (long long)((Sk + 127) / 128));
    return run_bwd(dtype, p, D, Dv, causal != 0, det, nullptr, B, Sq, Sk, static_cast<hipStream_t>(stream));
}

int sdpa_bwd(int dtype, int64_t B, int64_t Hq, int64_t Hkv, int64_t Sq, int64_t Sk, int64_t D, int64_t Dv,
             double scale, int causal, int deterministic, int grad_dtype,
             const sdpa_tensor4* q, const sdpa_tensor4* k, const sdpa_tensor4* v,
             const sdpa_tensor4* o, const sdpa_tensor4* dout, const sdpa_stats* stats,
             const sdpa_tensor4* dq, const sdpa_tensor4* dk, const sdpa_tensor4* dv,
             void* workspace, size_t workspace_bytes, void* stream) {
    return bwd_dense(dtype, B, Hq, Hkv, Sq, Sk, D, Dv, scale, causal, deterministic, grad_dtype, q, k, v, o, dout,
                     stats, dq, dk, dv, workspace, workspace_bytes, false, stream);
}

int sdpa_bwd_noalloc(int dtype, int64_t B, int64_t Hq, int64_t Hkv, int64_t Sq, int64_t Sk, int64_t D, int64_t Dv,
                     double scale, int causal, int deterministic, int grad_dtype,
                     const sdpa_tensor4* q, const sdpa_tensor4* k, const sdpa_tensor4* v,
                     const sdpa_tensor4* o, const sdpa_tensor4* dout, const sdpa_stats* stats,
                     const sdpa_tensor4* dq, const sdpa_tensor4* dk, const sdpa_tensor4* dv, void* stream) {
    return bwd_dense(dtype, B, Hq, Hkv, Sq, Sk, D, Dv, scale, causal, deterministic, grad_dtype, q, k, v, o, dout,
                     stats, dq, dk, dv, nullptr, 0, true, stream);
}

// ---------------------------------------------------------------------------
// Packed variable-length backward
// ---------------------------------------------------------------------------

int sdpa_bwd_varlen_workspace_size(int dtype, int64_t batch, const int64_t* cu_seqlens_q_host,
                                   const int64_t* cu_seqlens_kv_host, int64_t Hq, int64_t Hkv,
                                   int64_t D, int64_t Dv, int deterministic, size_t* bytes) {
    if (!bytes || !cu_seqlens_q_host || !cu_seqlens_kv_host) return SDPA_ERR_NULLPTR;
    if (dtype != SDPA_F16 && dtype != SDPA_BF16) return SDPA_ERR_INVALID;
    if (batch < 1 || Hq < 1 || Hkv < 1 || D < 1 || Dv < 1 || Hq % Hkv) return SDPA_ERR_INVALID;
    Packed P;
    if (int s = read_packed(batch, cu_seqlens_q_host, cu_seqlens_kv_host, P)) return s;
    if (!dq_mode_ok(deterministic)) return SDPA_ERR_INVALID;
    if (!dense_dims_ok(D, Dv) || !dense_mode_ok(deterministic, D, Dv)) return SDPA_ERR_UNSUPPORTED;
    *bytes = carve_bwd(P.Tq * Hq, D, !dq_atomic(deterministic, D)).total;
    return SDPA_OK;
}

int sdpa_bwd_varlen(int dtype, int64_t batch, const int64_t* cu_seqlens_q_host,
                    const int64_t* cu_seqlens_kv_host, int64_t Hq, int64_t Hkv, int64_t D, int64_t Dv,
                    double scale, int causal, int deterministic, int grad_dtype,
                    const sdpa_tensor3* q, const sdpa_tensor3* k, const sdpa_tensor3* v,
                    const sdpa_tensor3* o, const sdpa_tensor3* dout, const sdpa_stats* stats,
                    const sdpa_tensor3* dq, const sdpa_tensor3* dk, const sdpa_tensor3* dv,
                    void* workspace, size_t workspace_bytes, void* stream) {
    if (!cu_seqlens_q_host || !cu_seqlens_kv_host) return SDPA_ERR_NULLPTR;
    if (!q || !k || !v || !o || !dout || !stats || !dq || !dk || !dv) return SDPA_ERR_NULLPTR;
    for (const sdpa_tensor3* t : {q, k, v, o, dout, dq, dk, dv})
        if (!t->data) return SDPA_ERR_NULLPTR;
    if (int s = check_stats(stats)) return s;
    if (!workspace) return SDPA_ERR_NULLPTR;
    if (dtype != SDPA_F16 && dtype != SDPA_BF16) return SDPA_ERR_INVALID;
    if (grad_dtype != dtype && grad_dtype != SDPA_F32) return SDPA_ERR_INVALID;
    if (batch < 1 || Hq < 1 || Hkv < 1 || D < 1 || Dv < 1 || Hq % Hkv) return SDPA_ERR_INVALID;
    if (!std::isfinite(scale)) return SDPA_ERR_INVALID;
    if (!dq_mode_ok(deterministic)) return SDPA_ERR_INVALID;
    if (int s = check_stats_kind(stats)) return s;
    Packed P;
    if (int s = read_packed(batch, cu_seqlens_q_host, cu_seqlens_kv_host, P)) return s;
    if (!dense_dims_ok(D, Dv) || !dense_mode_ok(deterministic, D, Dv)) return SDPA_ERR_UNSUPPORTED;
    for (const sdpa_tensor3* t : {q, k, v, o, dout, dq, dk, dv})
        if (int s = tensor3_ok(t)) return s;
    if (int s = check_stats_stride(stats)) return s;
    // the D=128 dQ launch puts (sequence, query head) of a chunk of up to
    // kMaxSeqArgs sequences in grid y, the D=128 key-tile launch the key tiles
    if (P.max_lk / 128 + 1 > kMaxGridY || std::min<int64_t>(batch, sdpa::kMaxSeqArgs) * Hq > kMaxGridY)
        return SDPA_ERR_UNSUPPORTED;
    const bool det = !dq_atomic(deterministic, D);
    const int64_t rows = P.Tq * Hq;
    const Carve cv = carve_bwd(rows, D, det);
    if (workspace_bytes < cv.total) return SDPA_ERR_WORKSPACE;
    if (int s = check_device()) return s;

    char* ws = static_cast<char*>(workspace);
    sdpa::BwdParams p{};
    p.q = arg3(q); p.k = arg3(k); p.v = arg3(v); p.o = arg3(o); p.dout = arg3(dout);
    p.dq = arg3(dq); p.dk = arg3(dk); p.dv = arg3(dv);
    p.grad_f32 = grad_dtype == SDPA_F32;
    fill_stats(p, stats);
    p.st_sb = 0;
    p.lse2 = reinterpret_cast<float*>(ws + cv.lse2);
    p.delta = reinterpret_cast<float*>(ws + cv.delta);
    p.dqacc = det ? nullptr : reinterpret_cast<float*>(ws + cv.dqacc);
    p.B = (int)batch; p.Hq = (int)Hq; p.Hkv = (int)Hkv; p.Sq = (int)P.Tq; p.Sk = (int)P.Tk;
    p.rows = rows;
    p.scale = (float)scale;
    p.scale_log2 = (float)(scale * 1.4426950408889634);
    if (log_enabled())
        std::fprintf(stderr, "[sdpa_bwd] bwd_varlen dtype=%d batch=%lld Tq=%lld Tk=%lld Hq=%lld Hkv=%lld D=%lld Dv=%lld causal=%d det=%d\n",
                     dtype, (long long)batch, (long long)P.Tq, (long long)P.Tk, (long long)Hq,
                     (long long)Hkv, (long long)D, (long long)Dv, causal, (int)det);
    return run_bwd(dtype, p, D, Dv, causal != 0, det, &P, batch, 0, 0, static_cast<hipStream_t>(stream));
}

}  // extern "C"
