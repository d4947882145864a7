"""fp64 CPU oracle: SDPA forward statistics and the exact SDPA gradients.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Parity status of every
function: pinned by the CPU tests in ``tests/test_oracle_*.py`` against finite
differences, closed forms, invariants, torch fp64 autograd and brute force.

Notation (per sequence and head): Q in R^{Sq x D}, K in R^{Sk x D},
V in R^{Sk x Dv}, multiplying scale s.

* S = s * Q K^T, entries outside the admissible set set to -inf.
* m_i = max_j S_ij, l_i = sum_j exp(S_ij - m_i), LSE_i = m_i + ln l_i,
  P_ij = exp(S_ij - LSE_i) (0 outside the admissible set, and 0 on a row with
  no admissible key), O = P V.

  The forward's pattern is the unfused matmul -> scale -> softmax -> matmul
  chain (pytorch PR #94729, the attention pattern in its description) with the
  scale applied as a multiplier, as the cuDNN sample's ``attn_scale`` is
  (cudnn-frontend notebook, forward-graph cell).  The natural-log LSE of the
  scaled, masked scores is the "stats" tensor that the cuDNN sample passes from
  forward to backward (notebook, stats markdown cell); the max m and the sum l
  are the Ascend operator's softmaxMax / softmaxSum (aclnnNsaSelectedAttentionGrad,
  parameter table).

* Backward, for a loss whose gradient with respect to O is dO
  (aclnnNsaSelectedAttentionGrad, "Formula" section):
  dV = P^T dO, dP = dO V^T, dS_i = J(P_i) dP_i with J the row-softmax
  Jacobian diag(p) - p p^T, dQ = s * dS K, dK = s * dS^T Q.  The Ascend page
  writes the last two with a 1/sqrt(d) factor; that is the case s = d^-1/2.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "head_forward", "head_backward", "causal_mask", "dense_forward", "dense_backward",
    "varlen_forward", "varlen_backward", "selected_key_positions", "selected_block_lists",
    "selected_forward", "selected_backward", "rowsum_do_o",
]


# ----------------------------------------------------------------------------
# One head
# ----------------------------------------------------------------------------

def causal_mask(sq: int, sk: int) -> np.ndarray:
    """Admissible set of the causal mask: key j is visible to query i iff j <= i
    (the cuDNN sample's ``use_causal_mask``).  For Sq != Sk this is the top-left
    alignment of the PyTorch ``is_causal`` reference that the sample checks
    against (cudnn-frontend notebook, last code cell): queries i >= Sk see
    every key, keys j >= Sq are seen by no query."""
    return np.arange(sk)[None, :] <= np.arange(sq)[:, None]


def head_forward(q, k, v, scale: float, allowed=None) -> dict:
    """Scores, probabilities, output and row statistics for one head.

    q: (Sq, D), k: (Sk, D), v: (Sk, Dv) fp64; ``allowed`` is a boolean (Sq, Sk)
    admissible set (None = all keys)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    S = scale * (q @ k.T)
    if allowed is not None:
        S = np.where(allowed, S, -np.inf)
    m = S.max(axis=1) if S.shape[1] else np.full(S.shape[0], -np.inf)
    live = np.isfinite(m)
    m_safe = np.where(live, m, 0.0)
    E = np.exp(S - m_safe[:, None])          # exp(-inf) = 0 on masked entries
    l = E.sum(axis=1)
    P = np.where(live[:, None], E / np.where(live, l, 1.0)[:, None], 0.0)
    with np.errstate(divide="ignore"):
        lse = np.where(live, m_safe + np.log(np.where(live, l, 1.0)), -np.inf)
    O = P @ v
    return {"S": S, "P": P, "O": O, "m": m, "l": np.where(live, l, 0.0), "lse": lse}


def head_backward(q, k, v, do, scale: float, allowed=None) -> dict:
    """Exact gradients of O(Q, K, V) against dO for one head.

    Returns dq, dk, dv and the intermediates P, dP, dS."""
    f = head_forward(q, k, v, scale, allowed)
    P = f["P"]
    do = np.asarray(do, dtype=np.float64)
    dv = P.T @ do
    dP = do @ np.asarray(v, dtype=np.float64).T
    # Row softmax Jacobian applied to dP_i:  (diag(p) - p p^T) dp = p*dp - p (p.dp)
    dS = P * dP - P * np.sum(P * dP, axis=1, keepdims=True)
    dq = scale * (dS @ np.asarray(k, dtype=np.float64))
    dk = scale * (dS.T @ np.asarray(q, dtype=np.float64))
    return {"dq": dq, "dk": dk, "dv": dv, "P": P, "dP": dP, "dS": dS, "O": f["O"],
            "lse": f["lse"]}


def rowsum_do_o(do, o) -> np.ndarray:
    """Delta_i = sum_d dO_id O_id (the per-row term the FlashAttention-2 backward
    precomputes; used only by the oracle's self-tests to check that identity)."""
    return np.sum(np.asarray(do, np.float64) * np.asarray(o, np.float64), axis=-1)


def _kv_head(h: int, hq: int, hkv: int) -> int:
    """Query head h reads KV head floor(h / G), G = Hq / Hkv: contiguous groups
    (the Ascend page requires N1 to be a multiple of N2 and gives no mapping;
    contiguous groups is the plain reading)."""
    return h // (hq // hkv)


# ----------------------------------------------------------------------------
# Dense (B, H, S, D)
# ----------------------------------------------------------------------------

def dense_forward(q, k, v, scale: float, causal: bool) -> dict:
    """q: (B, Hq, Sq, D); k, v: (B, Hkv, Sk, D).  Returns O (B, Hq, Sq, Dv) and
    lse, m, l (B, Hq, Sq), all fp64."""
    B, Hq, Sq, _ = q.shape
    _, Hkv, Sk, Dv = v.shape
    allowed = causal_mask(Sq, Sk) if causal else None
    O = np.zeros((B, Hq, Sq, Dv))
    lse = np.zeros((B, Hq, Sq))
    m = np.zeros((B, Hq, Sq))
    l = np.zeros((B, Hq, Sq))
    for b in range(B):
        for h in range(Hq):
            hk = _kv_head(h, Hq, Hkv)
            f = head_forward(q[b, h], k[b, hk], v[b, hk], scale, allowed)
            O[b, h], lse[b, h], m[b, h], l[b, h] = f["O"], f["lse"], f["m"], f["l"]
    return {"O": O, "lse": lse, "m": m, "l": l}


def dense_backward(q, k, v, do, scale: float, causal: bool, heads=None) -> dict:
    """Exact dQ, dK, dV for dense attention.  dK and dV of a KV head sum the
    contributions of every query head in its group.

    ``heads``: optional list of (b, h_kv) pairs to compute (others left 0); the
    query heads of each listed group are all included, so the listed dK/dV and
    the dQ of those query heads are exact."""
    B, Hq, Sq, _ = q.shape
    _, Hkv, Sk, Dv = v.shape
    allowed = causal_mask(Sq, Sk) if causal else None
    dq = np.zeros(q.shape)
    dk = np.zeros(k.shape)
    dv = np.zeros(v.shape)
    G = Hq // Hkv
    todo = sorted(set(heads)) if heads is not None else [(b, hk) for b in range(B) for hk in range(Hkv)]
    for b, hk in todo:
        for h in range(hk * G, (hk + 1) * G):
            g = head_backward(q[b, h], k[b, hk], v[b, hk], do[b, h], scale, allowed)
            dq[b, h] = g["dq"]
            dk[b, hk] += g["dk"]
            dv[b, hk] += g["dv"]
    return {"dq": dq, "dk": dk, "dv": dv}


# ----------------------------------------------------------------------------
# Packed variable length (T, N, D)
# ----------------------------------------------------------------------------

def _starts(cu) -> np.ndarray:
    """Sequence start offsets from the inclusive cumulative lengths (B values,
    no leading zero: the Ascend example passes {1} / {1024} for one batch)."""
    cu = np.asarray(cu, dtype=np.int64)
    return np.concatenate([[0], cu[:-1]])


def varlen_forward(q, k, v, cu_q, cu_kv, scale: float, causal: bool) -> dict:
    """Per-sequence dense forward on a packed batch.  q: (Tq, Hq, D),
    k, v: (Tk, Hkv, D).  Returns O (Tq, Hq, Dv), lse, m, l (Tq, Hq)."""
    Tq, Hq, _ = q.shape
    _, Hkv, Dv = v.shape
    O = np.zeros((Tq, Hq, Dv))
    lse, m, l = (np.zeros((Tq, Hq)) for _ in range(3))
    for sq0, sq1, sk0, sk1 in zip(_starts(cu_q), cu_q, _starts(cu_kv), cu_kv):
        allowed = causal_mask(sq1 - sq0, sk1 - sk0) if causal else None
        for h in range(Hq):
            hk = _kv_head(h, Hq, Hkv)
            f = head_forward(q[sq0:sq1, h], k[sk0:sk1, hk], v[sk0:sk1, hk], scale, allowed)
            O[sq0:sq1, h] = f["O"]
            lse[sq0:sq1, h], m[sq0:sq1, h], l[sq0:sq1, h] = f["lse"], f["m"], f["l"]
    return {"O": O, "lse": lse, "m": m, "l": l}


def varlen_backward(q, k, v, do, cu_q, cu_kv, scale: float, causal: bool, seqs=None) -> dict:
    """Per-sequence exact gradients on a packed batch (causal in local indices).
    ``seqs``: optional list of sequence indices to compute (others left 0)."""
    Tq, Hq, _ = q.shape
    _, Hkv, _ = v.shape
    dq, dk, dv = np.zeros(q.shape), np.zeros(k.shape), np.zeros(v.shape)
    bounds = list(zip(_starts(cu_q), cu_q, _starts(cu_kv), cu_kv))
    todo = range(len(bounds)) if seqs is None else sorted(set(seqs))
    for i in todo:
        sq0, sq1, sk0, sk1 = bounds[i]
        allowed = causal_mask(sq1 - sq0, sk1 - sk0) if causal else None
        for h in range(Hq):
            hk = _kv_head(h, Hq, Hkv)
            g = head_backward(q[sq0:sq1, h], k[sk0:sk1, hk], v[sk0:sk1, hk],
                              do[sq0:sq1, h], scale, allowed)
            dq[sq0:sq1, h] = g["dq"]
            dk[sk0:sk1, hk] += g["dk"]
            dv[sk0:sk1, hk] += g["dv"]
    return {"dq": dq, "dk": dk, "dv": dv}


# ----------------------------------------------------------------------------
# NSA selected attention (aclnnNsaSelectedAttentionGrad)
# ----------------------------------------------------------------------------

def selected_key_positions(topk, block_size: int) -> np.ndarray:
    """Gathered key positions, sequence-local: for token t and KV head h2 the
    count*bs positions topk[t,h2,i]*bs + r, i-major (the page's Gather over
    0 <= i < selectedBlockCount, "Formula" section).  Duplicated blocks stay."""
    topk = np.asarray(topk, dtype=np.int64)
    r = np.arange(block_size, dtype=np.int64)
    pos = topk[..., None] * block_size + r
    return pos.reshape(topk.shape[0], topk.shape[1], -1)


def selected_block_lists(topk, cu_q, cu_kv, block_size: int):
    """Inverse of the top-k choice: for every (KV head h2, KV block), the list
    of entries e = t * count + slot (t a global token index) whose choice
    topk[t, h2, slot] names that block.  Lists are sorted by e.

    KV blocks are numbered globally: block g covers packed KV rows
    [g*bs, (g+1)*bs), so the block a token of sequence b selects is
    start_kv(b)/bs + topk.  Returns (offsets[N2*NB + 1], entries) in CSR form,
    bucket = h2 * NB + g, with NB = T_kv / bs.  Built by plain enumeration."""
    topk = np.asarray(topk, dtype=np.int64)
    T, N2, count = topk.shape
    cu_kv = np.asarray(cu_kv, dtype=np.int64)
    NB = int(cu_kv[-1]) // block_size
    buckets = [[] for _ in range(N2 * NB)]
    seq_of_token = np.zeros(T, dtype=np.int64)
    for b, (s0, s1) in enumerate(zip(_starts(cu_q), cu_q)):
        seq_of_token[s0:s1] = b
    kv_start = _starts(cu_kv)
    for t in range(T):
        blk0 = int(kv_start[seq_of_token[t]]) // block_size
        for h2 in range(N2):
            for slot in range(count):
                g = blk0 + int(topk[t, h2, slot])
                buckets[h2 * NB + g].append(t * count + slot)
    offsets = np.zeros(N2 * NB + 1, dtype=np.int64)
    for i, lst in enumerate(buckets):
        offsets[i + 1] = offsets[i] + len(lst)
    entries = np.array([e for lst in buckets for e in lst], dtype=np.int64)
    return offsets, entries


def _selected_token_rows(q, k, v, topk, cu_q, cu_kv, block_size, scale, sparse_mode, atten_mask=None):
    """Yields, per token t and KV head h2: the token, its query-head range, the
    absolute gathered positions and the admissible set over them.

    atten_mask: optional 2-D boolean array indexed by (sequence-local query
    position, sequence-local key position), True where the score is masked
    out, the same for every sequence and head (the Ascend page's
    attenMaskOptional, "Parameters" table: BOOL/UINT8, two dimensions; the page
    does not say more, so this reads it as the usual keep-out mask over the
    score matrix, combined with sparse_mode's causal rule)."""
    Tq, Hq, _ = q.shape
    _, Hkv, _ = k.shape
    G = Hq // Hkv
    pos_local = selected_key_positions(topk, block_size)
    mask = None if atten_mask is None else np.asarray(atten_mask).astype(bool)
    for s0, s1, k0 in zip(_starts(cu_q), cu_q, _starts(cu_kv)):
        for t in range(int(s0), int(s1)):
            t_local = t - int(s0)
            for h2 in range(Hkv):
                p = pos_local[t, h2]
                allowed = (p <= t_local) if sparse_mode == 2 else np.ones(p.shape, bool)
                if mask is not None:
                    allowed = allowed & ~mask[t_local, p]
                yield t, slice(h2 * G, (h2 + 1) * G), h2, int(k0) + p, allowed


def selected_forward(q, k, v, topk, cu_q, cu_kv, block_size: int, scale: float,
                     sparse_mode: int, atten_mask=None) -> dict:
    """Attention of every query token over its gathered keys.  sparse_mode 0: no
    mask; 2: causal, key position <= query position within the sequence (the
    page allows "0 or 2" without defining them; this is the plain reading).
    atten_mask: see _selected_token_rows.  A row left with no admissible key
    has P = 0, O = 0, m = -inf and l = 0.
    Returns O (T, Hq, Dv), lse, m, l (T, Hq)."""
    Tq, Hq, _ = q.shape
    Dv = v.shape[2]
    O = np.zeros((Tq, Hq, Dv))
    lse, m, l = (np.zeros((Tq, Hq)) for _ in range(3))
    for t, hs, h2, pos, allowed in _selected_token_rows(q, k, v, topk, cu_q, cu_kv,
                                                        block_size, scale, sparse_mode, atten_mask):
        f = head_forward(q[t, hs], k[pos, h2], v[pos, h2], scale,
                         np.broadcast_to(allowed, (hs.stop - hs.start, pos.size)))
        O[t, hs], lse[t, hs], m[t, hs], l[t, hs] = f["O"], f["lse"], f["m"], f["l"]
    return {"O": O, "lse": lse, "m": m, "l": l}


def selected_backward(q, k, v, do, topk, cu_q, cu_kv, block_size: int, scale: float,
                      sparse_mode: int, atten_mask=None) -> dict:
    """Exact gradients of the gathered attention: per token, the dense head
    backward over the gathered keys, then dK/dV scattered back to the gathered
    positions with duplicates accumulating.  atten_mask: see
    _selected_token_rows."""
    dq, dk, dv = np.zeros(q.shape), np.zeros(k.shape), np.zeros(v.shape)
    for t, hs, h2, pos, allowed in _selected_token_rows(q, k, v, topk, cu_q, cu_kv,
                                                        block_size, scale, sparse_mode, atten_mask):
        g = head_backward(q[t, hs], k[pos, h2], v[pos, h2], do[t, hs], scale,
                          np.broadcast_to(allowed, (hs.stop - hs.start, pos.size)))
        dq[t, hs] = g["dq"]
        np.add.at(dk[:, h2], pos, g["dk"])
        np.add.at(dv[:, h2], pos, g["dv"])
    return {"dq": dq, "dk": dk, "dv": dv}
