/*
 * libsdpa_bwd: backward pass of scaled dot-product attention on MI355X (gfx950).
 *
 * What the library computes, per sequence and head (Q: Sq x D, K, V: Sk x D,
 * multiplying scale s):
 *   S = s Q K^T restricted to the admissible keys (all, causal j <= i, or the
 *   gathered top-k blocks), P = exp(S - LSE) with LSE the row log-sum-exp,
 *   dV = P^T dO, dP = dO V^T, dS = P o (dP - Delta) with Delta_i = sum_d dO_id O_id,
 *   dQ = s dS K, dK = s dS^T Q.
 * The backward takes the forward's per-row statistics instead of recomputing
 * them (the cuDNN SDPA-backward sample notebook, introduction and stats
 * cells: the stats tensor is (B, H, S, 1) fp32 and passes from forward to
 * backward); the gradient formulas are those of the Ascend operator page
 * aclnnNsaSelectedAttentionGrad ("Formula" section), whose 1/sqrt(d) factor is
 * the case s = d^-1/2.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Element types: Q, K, V, O and dO are all fp16 or all bf16 (sdpa_dtype);
 *   the gradients dQ, dK, dV are that type or fp32 (grad_dtype of the
 *   backward entry points; the Ascend parameter table lists FLOAT16, BFLOAT16
 *   and FLOAT32 for dqOut, dkOut and dvOut); statistics are fp32.  Arithmetic
 *   is fp32 with 16-bit MFMA operands (the sample's io=HALF,
 *   intermediate=compute=FLOAT graph).
 * - Layout: every tensor is a strided view, strides counted in ELEMENTS.  Dense
 *   tensors are logical (B, H, S, D) with any strides, e.g. the sample's BSHD
 *   physical / BHSD logical strides (S*H*D, D, H*D, 1).  Packed tensors are
 *   (T, N, D) ("TND", the Ascend page's only layout).  The last (D) stride must
 *   be 1 and every base pointer 16-byte aligned; the S/T and H/N strides must
 *   keep every row 16-byte aligned.  The row stride (S or T) of every tensor
 *   and of the statistics must lie in [0, 2^23) elements.  Head dims: D of
 *   Q, K, dQ and dK, Dv of V, O, dO and dV; (D, Dv) is (64, 64), (128, 128),
 *   (192, 192) or (192, 128), the unequal pair that the Ascend page's head
 *   dim constraint allows ("Constraints": D is 192 or 128, K and V may
 *   differ).  Any other pair returns SDPA_ERR_UNSUPPORTED; D or Dv below 1
 *   is SDPA_ERR_INVALID.
 *   Any other layout returns SDPA_ERR_UNSUPPORTED.
 * - Ownership: the caller owns every buffer, including the workspace.  The
 *   library allocates no device memory, keeps no per-call state and never
 *   synchronises: kernels are enqueued on `stream` (a hipStream_t; NULL is the
 *   default stream) and the call returns once they are enqueued.  Host arrays
 *   (cumulative lengths) are read during the call only.  Outputs are
 *   overwritten, never accumulated into.  Outputs must not alias inputs.
 * - Errors: every function returns an sdpa_status and never aborts.  Argument
 *   errors are detected before any HIP call, in this order: NULL pointers
 *   (SDPA_ERR_NULLPTR), invalid values (SDPA_ERR_INVALID), valid but not
 *   implemented cases (SDPA_ERR_UNSUPPORTED), a workspace smaller than the size
 *   query returned (SDPA_ERR_WORKSPACE).  HIP failures, including "no device",
 *   return SDPA_ERR_HIP; sdpa_last_error() then gives the HIP error text of the
 *   calling thread.  This mirrors the Ascend page's split of return codes into
 *   a null-pointer error and an invalid-parameter error ("Return Value").
 * - Thread safety: calls are independent; concurrent calls on different
 *   streams must use different workspaces.
 */
#ifndef SDPA_BWD_H
#define SDPA_BWD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum sdpa_status {
    SDPA_OK = 0,
    SDPA_ERR_NULLPTR = 1,
    SDPA_ERR_INVALID = 2,
    SDPA_ERR_UNSUPPORTED = 3,
    SDPA_ERR_WORKSPACE = 4,
    SDPA_ERR_HIP = 5
} sdpa_status;

/* Element types (Ascend parameter table): Q, K, V, O and dO are BFLOAT16 or
 * FLOAT16; the gradients are that type or, as grad_dtype = SDPA_F32, FLOAT32
 * (the fp32 accumulators written without rounding to 16 bits). */
typedef enum sdpa_dtype { SDPA_F16 = 0, SDPA_BF16 = 1, SDPA_F32 = 2 } sdpa_dtype;

/* Form of the per-row softmax statistics.
 * SDPA_STATS_LSE:     one value per row, LSE_i = ln sum_j exp(S_ij) over the
 *                     admissible keys (the cuDNN sample's "stats"; -inf for a
 *                     row with no admissible key).
 * SDPA_STATS_MAX_SUM: two values per row, m_i = max_j S_ij and
 *                     l_i = sum_j exp(S_ij - m_i) (the Ascend softmaxMax and
 *                     softmaxSum; l_i = 0 for a row with no admissible key).
 * S is the scaled, masked score in both cases. */
typedef enum sdpa_stats_kind { SDPA_STATS_LSE = 0, SDPA_STATS_MAX_SUM = 1 } sdpa_stats_kind;

/* Dense 16-bit tensor, logical (B, H, S, D); strides in elements. */
typedef struct sdpa_tensor4 {
    void* data;
    int64_t stride_b, stride_h, stride_s, stride_d;
} sdpa_tensor4;

/* Packed 16-bit tensor, logical (T, N, D); strides in elements. */
typedef struct sdpa_tensor3 {
    void* data;
    int64_t stride_t, stride_n, stride_d;
} sdpa_tensor3;

/* fp32 per-row statistics.  Dense: element (b, h, i) at b*stride_b +
 * h*stride_h + i*stride_s.  Packed: element (t, n) at t*stride_s + n*stride_h
 * (stride_b unused).  The Ascend page's [T, N, 8] statistics (constraints
 * section) are read as stride_s = 8N, stride_h = 8: element 0 of the 8. */
typedef struct sdpa_stats {
    int32_t kind;          /* sdpa_stats_kind */
    const float* lse_or_max;
    const float* sum;      /* SDPA_STATS_MAX_SUM only; NULL otherwise */
    int64_t stride_b, stride_h, stride_s;
} sdpa_stats;

/* Per-row statistics output of the forward (dense layout as sdpa_stats). */
typedef struct sdpa_stats_out {
    float* lse;
    int64_t stride_b, stride_h, stride_s;
} sdpa_stats_out;

/* Text for a status; for SDPA_ERR_HIP the last HIP error message of this thread. */
const char* sdpa_status_string(int status);
const char* sdpa_last_error(void);

/*
 * sdpa_fwd_stats: attention forward in training mode, producing O and the LSE
 * statistics that the backward consumes (the cuDNN sample's forward graph with
 * is_inference=False: outputs o and stats; forward-graph cell).
 *   q: (B, Hq, Sq, D); k: (B, Hkv, Sk, D); v: (B, Hkv, Sk, Dv);
 *   o_out: (B, Hq, Sq, Dv) written;
 *   lse_out: (B, Hq, Sq) written, natural-log LSE of the scaled scores.
 *   Hq must be a multiple of Hkv; query head h reads KV head h / (Hq/Hkv).
 *   causal: key j visible to query i iff j <= i, for any Sq and Sk (aligned
 *   at the top left, as the PyTorch is_causal reference that the cuDNN sample
 *   checks against, last code cell): queries i >= Sk see every key.
 * Needs no workspace.
 */
int sdpa_fwd_stats(int dtype, int64_t B, int64_t Hq, int64_t Hkv, int64_t Sq, int64_t Sk,
                   int64_t D, int64_t Dv, double scale, int causal,
                   const sdpa_tensor4* q, const sdpa_tensor4* k, const sdpa_tensor4* v,
                   const sdpa_tensor4* o_out, const sdpa_stats_out* lse_out, void* stream);

/*
 * sdpa_fwd_stats_varlen: the same forward for a packed (TND) batch, one call
 * for all sequences (the Ascend page's packed layout and host cumulative
 * lengths, "Parameters" table; its softmaxMax/softmaxSum are given here as
 * the equivalent LSE = max + ln(sum)).
 *   cu_seqlens_q_host, cu_seqlens_kv_host: host arrays of `batch` inclusive
 *   end offsets (no leading zero), non-decreasing; read during the call only.
 *   q: (Tq, Hq, D); k: (Tk, Hkv, D); v: (Tk, Hkv, Dv); o_out: (Tq, Hq, Dv)
 *   written.
 *   lse_out: natural-log LSE of token t, head n at t*stride_s + n*stride_h
 *   (stride_b unused), written for every query token.
 *   causal: per sequence, key j visible to query i iff j <= i in local
 *   positions (top-left aligned; the lengths may differ).  A query with no
 *   visible key (empty key sequence) gets O = 0 and LSE = -inf.
 * Needs no workspace; errors as sdpa_fwd_stats.
 */
int sdpa_fwd_stats_varlen(int dtype, int64_t batch, const int64_t* cu_seqlens_q_host,
                          const int64_t* cu_seqlens_kv_host, int64_t Hq, int64_t Hkv, int64_t D, int64_t Dv,
                          double scale, int causal, const sdpa_tensor3* q, const sdpa_tensor3* k,
                          const sdpa_tensor3* v, const sdpa_tensor3* o_out, const sdpa_stats_out* lse_out,
                          void* stream);

/*
 * sdpa_bwd_workspace_size / sdpa_bwd: dense SDPA backward (the cuDNN sample's
 * sdpa_backward node: inputs q, k, v, o, dO, stats, attn_scale,
 * use_causal_mask; outputs dQ, dK, dV; backward-graph cell).
 *   Shapes as sdpa_fwd_stats; dq like q, dk like k; dout like o, dv like v.
 *   deterministic selects how dQ is formed (the Ascend page's deterministic
 *     option, "Constraints", extended):
 *     0: the library's fastest method; today that is the atomic-free query-
 *        outer pass for every head size, so results are reproducible;
 *     1: guaranteed bitwise reproducible: the atomic-free query-outer pass;
 *     2: fp32 atomic accumulation inside the key-outer kernel and a final
 *        conversion (FlashAttention-2's method; run-to-run rounding
 *        differences possible), at (D, Dv) = (64, 64) and (128, 128); at
 *        D=192 the key-outer kernel's tiles leave no LDS for it and the
 *        value returns SDPA_ERR_UNSUPPORTED.
 *     Any other value: SDPA_ERR_INVALID.  The workspace size depends on it.
 *   grad_dtype: element type of dq, dk and dv: `dtype`, or SDPA_F32 for fp32
 *     gradients (same layout rules, strides in fp32 elements); anything else
 *     is SDPA_ERR_INVALID.  It does not change the workspace size.
 *   workspace: device memory of at least *bytes from the size query, any
 *     contents on entry, 256-byte aligned.
 */
int sdpa_bwd_workspace_size(int dtype, int64_t B, int64_t Hq, int64_t Hkv, int64_t Sq,
                            int64_t Sk, int64_t D, int64_t Dv, int deterministic, size_t* bytes);
int sdpa_bwd(int dtype, int64_t B, int64_t Hq, int64_t Hkv, int64_t Sq, int64_t Sk, int64_t D, int64_t Dv,
             double scale, int causal, int deterministic, int grad_dtype,
             const sdpa_tensor4* q, const sdpa_tensor4* k, const sdpa_tensor4* v,
             const sdpa_tensor4* o, const sdpa_tensor4* dout, const sdpa_stats* stats,
             const sdpa_tensor4* dq, const sdpa_tensor4* dk, const sdpa_tensor4* dv,
             void* workspace, size_t workspace_bytes, void* stream);

/*
 * sdpa_bwd_noalloc: sdpa_bwd without a workspace argument, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc).  Arguments, results and error codes
 * are those of sdpa_bwd, and it runs the same kernels.  The per-row scratch
 * (log2-LSE and Delta, plus the fp32 dQ accumulator in dQ mode 2) lives in a
 * fixed 16 MiB array inside the library, one per GPU, kept until the process
 * ends; a problem whose sdpa_bwd_workspace_size exceeds 16 MiB
 * (16777216 bytes) returns SDPA_ERR_WORKSPACE, with the needed size in
 * sdpa_last_error(), before any HIP call.  Modes 0 and 1 need 8 bytes per
 * query row and head (about 2 million rows); mode 2 adds 4*D bytes per row.
 * The call allocates nothing (no hipMalloc, no library allocation); the first
 * call on a GPU looks up that GPU's array address once.  Every call on one
 * GPU shares that GPU's array and leaves its contents behind: the kernels
 * rewrite (and in mode 2 clear) what they read, but calls that overlap in
 * time on one GPU (different streams or threads) race on it and must be
 * serialised by the caller.
 */
int sdpa_bwd_noalloc(int dtype, int64_t B, int64_t Hq, int64_t Hkv, int64_t Sq, int64_t Sk, int64_t D, int64_t Dv,
                     double scale, int causal, int deterministic, int grad_dtype,
                     const sdpa_tensor4* q, const sdpa_tensor4* k, const sdpa_tensor4* v,
                     const sdpa_tensor4* o, const sdpa_tensor4* dout, const sdpa_stats* stats,
                     const sdpa_tensor4* dq, const sdpa_tensor4* dk, const sdpa_tensor4* dv, void* stream);

/*
 * sdpa_bwd_varlen_workspace_size / sdpa_bwd_varlen: packed variable-length
 * backward (TND).  `batch` sequences; cu_seqlens_q_host / cu_seqlens_kv_host
 * are HOST arrays of `batch` int64 inclusive end offsets with no leading zero
 * (the Ascend page's actualSeqQLen / actualSeqKvLen, "cumulative sum length
 * of S for each batch", passed as host integer arrays; its example passes {1}
 * and {1024} for one sequence).  Sequence b owns rows [cu[b-1], cu[b]) with
 * cu[-1] = 0.  Causal masking uses positions local to each sequence (j <= i,
 * top-left aligned when the query and key lengths differ).
 *   q, dq: (Tq, Hq, D); o, dout: (Tq, Hq, Dv); k, dk: (Tk, Hkv, D);
 *   v, dv: (Tk, Hkv, Dv); stats per (t, h).
 *   deterministic, grad_dtype: as for sdpa_bwd.
 */
int sdpa_bwd_varlen_workspace_size(int dtype, int64_t batch, const int64_t* cu_seqlens_q_host,
                                   const int64_t* cu_seqlens_kv_host, int64_t Hq, int64_t Hkv,
                                   int64_t D, int64_t Dv, int deterministic, size_t* bytes);
int sdpa_bwd_varlen(int dtype, int64_t batch, const int64_t* cu_seqlens_q_host,
                    const int64_t* cu_seqlens_kv_host, int64_t Hq, int64_t Hkv, int64_t D, int64_t Dv,
                    double scale, int causal, int deterministic, int grad_dtype,
                    const sdpa_tensor3* q, const sdpa_tensor3* k, const sdpa_tensor3* v,
                    const sdpa_tensor3* o, const sdpa_tensor3* dout, const sdpa_stats* stats,
                    const sdpa_tensor3* dq, const sdpa_tensor3* dk, const sdpa_tensor3* dv,
                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * sdpa_bwd_selected_workspace_size / sdpa_bwd_selected: NSA selected-attention
 * backward (aclnnNsaSelectedAttentionGrad).  For every query token t and KV
 * head h2 the keys are the block_count blocks of block_size rows named by
 * topk[t, h2, i] (0 <= i < block_count), gathered with repetition (a block
 * named twice counts twice; "Formula" section).  topk: DEVICE int32 tensor
 * (T, Hkv, block_count) with element strides (tk_st, tk_sn, tk_sk); block
 * indices are relative to the token's sequence start in K/V.
 *   sparse_mode 0: no mask; 2: causal, key position <= query position within
 *   the sequence (the page supports "0 or 2" without defining them).
 *   atten_mask: optional DEVICE byte array (the page's attenMaskOptional,
 *   BOOL/UINT8, two dimensions, "Parameters" table), or NULL for none.  Byte
 *   atten_mask[i * atten_mask_stride + j] nonzero masks out key position j
 *   for query position i, both counted from the start of their sequence; the
 *   same mask applies to every sequence and head, on top of sparse_mode's
 *   causal rule (the page gives no formula for it; this is the usual
 *   keep-out reading).  It needs a row for every query position of the
 *   longest query sequence and atten_mask_stride >= the longest KV sequence
 *   (else SDPA_ERR_INVALID); base and stride must be 16-byte multiples, with
 *   the stride below 2^31 (else SDPA_ERR_UNSUPPORTED).  A query left with no
 *   admissible key gets P = 0 (forward: O = 0, max = -inf, sum = 0).
 *   Constraints (Ascend page, "Constraints"): block_size <= 128 and a multiple
 *   of 16; 1 <= block_count <= 128; block_count * block_size < 8192; every KV
 *   sequence length a multiple of block_size and >= block_count * block_size;
 *   Hq a multiple of Hkv with Hq / Hkv <= 32; any number of sequences (more
 *   than 64 take a table of 16 bytes per sequence in the workspace); token
 *   and head strides of every tensor below 2^23 elements.  Topk
 *   values outside the sequence's blocks select nothing (those slots are
 *   ignored); the statistics must then describe the same reduced key set.
 *   Checked mode: with the environment variable SDPA_BWD_CHECK set (not
 *   "0"), the selected calls copy topk to the host, which synchronises
 *   `stream`, and return SDPA_ERR_INVALID for such a value instead.
 *   Every kernel of this path is deterministic; the flag (0, 1 or 2, else
 *   SDPA_ERR_INVALID) is accepted for symmetry with the other entry points.
 *   grad_dtype: `dtype` or SDPA_F32, as for sdpa_bwd.
 *   D: head dim of q, k, dq, dk; Dv: of v, o, dout, dv (the page: D is 192
 *   or 128, and K and V may differ).  Kernels exist for (D, Dv) = (64, 64),
 *   (128, 128), (192, 192) and (192, 128); other valid pairs return
 *   SDPA_ERR_UNSUPPORTED.
 */
int sdpa_bwd_selected_workspace_size(int dtype, int64_t batch, const int64_t* cu_seqlens_q_host,
                                     const int64_t* cu_seqlens_kv_host, int64_t Hq, int64_t Hkv,
                                     int64_t D, int64_t Dv, int64_t block_size, int64_t block_count,
                                     int deterministic, size_t* bytes);
int sdpa_bwd_selected(int dtype, int64_t batch, const int64_t* cu_seqlens_q_host,
                      const int64_t* cu_seqlens_kv_host, int64_t Hq, int64_t Hkv, int64_t D, int64_t Dv,
                      double scale, int sparse_mode, const uint8_t* atten_mask, int64_t atten_mask_stride,
                      const int32_t* topk, int64_t tk_st,
                      int64_t tk_sn, int64_t tk_sk, int64_t block_size, int64_t block_count,
                      int deterministic, int grad_dtype,
                      const sdpa_tensor3* q, const sdpa_tensor3* k, const sdpa_tensor3* v,
                      const sdpa_tensor3* o, const sdpa_tensor3* dout, const sdpa_stats* stats,
                      const sdpa_tensor3* dq, const sdpa_tensor3* dk, const sdpa_tensor3* dv,
                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * sdpa_fwd_selected: the NSA selected-attention forward in training mode,
 * producing O and the softmaxMax / softmaxSum statistics that
 * sdpa_bwd_selected consumes (Ascend page, "Formula": P is the softmax of the
 * scaled scores over the gathered blocks; "Parameters": softmaxMax,
 * softmaxSum).  Arguments, topk, sparse_mode, atten_mask, head dims (D, Dv)
 * and constraints as sdpa_bwd_selected; o_out: (Tq, Hq, Dv) written.
 *   max_out[t*stats_stride_s + h*stats_stride_h]: max over the admissible
 *   gathered keys of the scaled score (natural units); sum_out at the same
 *   offset: sum of exp(score - max).  A token with no admissible key gets
 *   O = 0, max = -inf, sum = 0.  Both arrays are caller-owned device fp32.
 * Needs no workspace; errors as sdpa_bwd_selected.
 */
int sdpa_fwd_selected(int dtype, int64_t batch, const int64_t* cu_seqlens_q_host,
                      const int64_t* cu_seqlens_kv_host, int64_t Hq, int64_t Hkv, int64_t D, int64_t Dv,
                      double scale, int sparse_mode, const uint8_t* atten_mask,
                      int64_t atten_mask_stride, const int32_t* topk, int64_t tk_st,
                      int64_t tk_sn, int64_t tk_sk, int64_t block_size, int64_t block_count,
                      const sdpa_tensor3* q, const sdpa_tensor3* k, const sdpa_tensor3* v,
                      const sdpa_tensor3* o_out, float* max_out, float* sum_out,
                      int64_t stats_stride_s, int64_t stats_stride_h, void* stream);

/*
 * sdpa_selected_build_index: the inverse of the top-k choice, as used by
 * sdpa_bwd_selected.  KV blocks are numbered over the packed KV rows (block g
 * covers rows [g*block_size, (g+1)*block_size)); for bucket = h2 * NB + g,
 * NB = Tk / block_size, the entries e = t * block_count + slot with
 * topk[t, h2, slot] naming block g, sorted increasingly.
 *   offsets_out: DEVICE int32 array of Hkv*NB + 1 CSR offsets (written);
 *   entries_out: DEVICE int32 array of Tq*Hkv*block_count entries (written).
 * workspace: at least the bytes returned by the selected workspace query.
 */
int sdpa_selected_build_index(int64_t batch, const int64_t* cu_seqlens_q_host,
                              const int64_t* cu_seqlens_kv_host, int64_t Hkv,
                              const int32_t* topk, int64_t tk_st, int64_t tk_sn, int64_t tk_sk,
                              int64_t block_size, int64_t block_count,
                              int32_t* offsets_out, int32_t* entries_out,
                              void* workspace, size_t workspace_bytes, void* stream);

/*
 * Kernel timing for measurement tools (not needed for computing anything).
 * Between sdpa_profile_begin() and sdpa_profile_end() every kernel launch of
 * this library carries a pair of HIP events that the runtime fills with the
 * kernel's own begin and end timestamps (hipExtLaunchKernelGGL), so the
 * elapsed time is the kernel's execution alone, without launch gaps.
 * sdpa_profile_end() waits for the last event, writes for
 * each kernel id k < n_kernels the summed elapsed milliseconds total_ms[k]
 * and the number of launches launches[k], and disables timing.  Kernel ids:
 * 0 forward, 1 backward preprocess, 2 backward key-tile kernel (D=128; D=64
 * in dQ mode 2), 3 dQ convert,
 * 4 deterministic dQ (D=128), 5 NSA index build (four launches; in the
 * selected backward the first also carries the row pass), 6 NSA dK/dV,
 * 7 NSA dQ (with the dK/dV partial reduction where the dQ pass reads stored
 * dS), 8 fused dK/dV and dQ (D=64), 9 NSA dK/dV partial reduction,
 * 10 fused dK/dV and dQ, two-wavefront form (D=64);
 * sdpa_kernel_name(id) gives the kernel's symbol name stem.  Not thread-safe
 * with respect to concurrent begin/end calls from several threads.
 */
int sdpa_profile_begin(void);
int sdpa_profile_end(int n_kernels, double* total_ms, int64_t* launches);
const char* sdpa_kernel_name(int kernel_id);

#ifdef __cplusplus
}
#endif

#endif /* SDPA_BWD_H */
