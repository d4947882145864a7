"""Pins for the packed-varlen and the NSA selected-attention parts of the oracle.

* varlen: per-sequence dense results, locality, finite differences on a pack.
* selected: equivalence with dense attention under the matching block mask
  (torch fp64 autograd with an additive log-multiplicity bias), finite
  differences with duplicated blocks, the all-blocks-once special case, and the
  Ascend page's example program (aclnnNsaSelectedAttentionGrad, "Example"
  section) whose constant inputs give a closed form.
* index path: brute-force enumeration and an independent stable sort.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import synth

RNG = np.random.default_rng(99)
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(*shape):
    return RNG.standard_normal(shape)


# ----------------------------------------------------------------------------
# varlen
# ----------------------------------------------------------------------------

def test_varlen_equals_per_sequence_dense():
    lengths = [5, 12, 1, 9]
    cu = np.cumsum(lengths)
    T, H, D = int(cu[-1]), 3, 4
    q, k, v, do = (_rand(T, H, D) for _ in range(4))
    g = oracle.varlen_backward(q, k, v, do, cu, cu, 0.5, True)
    f = oracle.varlen_forward(q, k, v, cu, cu, 0.5, True)
    s0 = 0
    for L in lengths:
        sl = slice(s0, s0 + L)
        tq = lambda x: x[sl].transpose(1, 0, 2)[None]  # noqa: E731
        gd = oracle.dense_backward(tq(q), tq(k), tq(v), tq(do), 0.5, True)
        fd = oracle.dense_forward(tq(q), tq(k), tq(v), 0.5, True)
        for key in ("dq", "dk", "dv"):
            np.testing.assert_array_equal(g[key][sl], gd[key][0].transpose(1, 0, 2))
        np.testing.assert_array_equal(f["O"][sl], fd["O"][0].transpose(1, 0, 2))
        np.testing.assert_array_equal(f["lse"][sl], fd["lse"][0].T)
        s0 += L


def test_varlen_locality():
    lengths = [6, 7, 4]
    cu = np.cumsum(lengths)
    T, H, D = int(cu[-1]), 2, 3
    q, k, v, do = (_rand(T, H, D) for _ in range(4))
    g1 = oracle.varlen_backward(q, k, v, do, cu, cu, 0.8, True)
    q2, v2 = q.copy(), v.copy()
    q2[6:13] += 1.0      # perturb sequence 1 only
    v2[6:13] -= 0.5
    g2 = oracle.varlen_backward(q2, k, v2, do, cu, cu, 0.8, True)
    for key in ("dq", "dk", "dv"):
        np.testing.assert_array_equal(g1[key][:6], g2[key][:6])
        np.testing.assert_array_equal(g1[key][13:], g2[key][13:])
        assert not np.array_equal(g1[key][6:13], g2[key][6:13])


def test_varlen_finite_differences():
    lengths = [3, 4]
    cu = np.cumsum(lengths)
    T, H, D = 7, 1, 2
    q, k, v, do = (_rand(T, H, D) for _ in range(4))
    g = oracle.varlen_backward(q, k, v, do, cu, cu, 0.9, True)

    def loss(q_, k_, v_):
        return float(np.sum(do * oracle.varlen_forward(q_, k_, v_, cu, cu, 0.9, True)["O"]))

    h = 1e-6
    for name, x, ref in (("dq", q, g["dq"]), ("dk", k, g["dk"]), ("dv", v, g["dv"])):
        fd = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            args = {"dq": [q, k, v], "dk": [q, k, v], "dv": [q, k, v]}[name]
            args = [a.copy() for a in args]
            j = {"dq": 0, "dk": 1, "dv": 2}[name]
            args[j][idx] += h
            lp = loss(*args)
            args[j][idx] -= 2 * h
            lm = loss(*args)
            fd[idx] = (lp - lm) / (2 * h)
        assert np.max(np.abs(fd - ref)) / np.max(np.abs(ref)) < 1e-7, name


# ----------------------------------------------------------------------------
# selected (NSA)
# ----------------------------------------------------------------------------

def _multiplicity_bias(topk, cu_q, cu_kv, bs, sparse_mode, Tk, mask=None):
    """Dense additive bias per (token, kv head, key): ln(number of slots that
    name the key's block), -inf if none, if causally excluded or if the user
    mask (sequence-local query, key) excludes it."""
    T, N2, count = topk.shape
    bias = np.full((T, N2, Tk), -np.inf)
    starts_q = np.concatenate([[0], cu_q[:-1]])
    starts_k = np.concatenate([[0], cu_kv[:-1]])
    for s0, s1, k0, k1 in zip(starts_q, cu_q, starts_k, cu_kv):
        for t in range(s0, s1):
            for h2 in range(N2):
                mult = np.bincount(topk[t, h2], minlength=(k1 - k0) // bs)
                for j in range(k1 - k0):
                    if sparse_mode == 2 and j > t - s0:
                        continue
                    if mask is not None and mask[t - s0, j]:
                        continue
                    if mult[j // bs]:
                        bias[t, h2, k0 + j] = math.log(mult[j // bs])
    return bias


def _torch_biased(q, k, v, do, bias, scale):
    """Dense attention with an additive bias, fp64 autograd (per token rows)."""
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    T, Hq, D = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    kk = tk.repeat_interleave(G, dim=1)           # (Tk, Hq, D)
    vv = tv.repeat_interleave(G, dim=1)
    s = scale * torch.einsum("thd,khd->htk", tq, kk)
    b = torch.tensor(np.repeat(bias, G, axis=1).transpose(1, 0, 2))  # (Hq, T, Tk)
    p = torch.softmax(s + b, dim=-1)
    o = torch.einsum("htk,khd->thd", p, vv)
    g = torch.autograd.grad(o, (tq, tk, tv), torch.tensor(do))
    return o.detach().numpy(), [x.numpy() for x in g]


def _tiny_selected(lengths=(32,), N2=1, G=2, D=4, bs=4, count=3, seed=0, Dv=None):
    lengths = np.array(lengths)
    cu = np.cumsum(lengths)
    T = int(cu[-1])
    Dv = D if Dv is None else Dv
    rng = np.random.default_rng(seed)
    q, do = rng.standard_normal((T, N2 * G, D)), rng.standard_normal((T, N2 * G, Dv))
    k, v = rng.standard_normal((T, N2, D)), rng.standard_normal((T, N2, Dv))
    topk = synth.draw_topk(lengths, N2, bs, count, config_id=77)
    return q, k, v, do, topk, cu


@pytest.mark.parametrize("sparse_mode", [0, 2])
@pytest.mark.parametrize("D,Dv", [(4, 4), (6, 3)])
def test_selected_equals_biased_dense(sparse_mode, D, Dv):
    """Also with a value head dim unlike the query/key one (the Ascend page
    supports unequal D for K and V)."""
    q, k, v, do, topk, cu = _tiny_selected(lengths=(24, 16), N2=2, G=2, count=3, D=D, Dv=Dv)
    # inject duplicates and out-of-order entries on some rows
    topk[5, 0] = [1, 1, 0]
    topk[30, 1] = [2, 0, 2]
    bs, scale = 4, 0.45
    f = oracle.selected_forward(q, k, v, topk, cu, cu, bs, scale, sparse_mode)
    g = oracle.selected_backward(q, k, v, do, topk, cu, cu, bs, scale, sparse_mode)
    bias = _multiplicity_bias(topk, cu, cu, bs, sparse_mode, k.shape[0])
    o_t, (dq_t, dk_t, dv_t) = _torch_biased(q, k, v, do, bias, scale)
    np.testing.assert_allclose(f["O"], o_t, atol=1e-12)
    np.testing.assert_allclose(g["dq"], dq_t, atol=1e-12)
    np.testing.assert_allclose(g["dk"], dk_t, atol=1e-12)
    np.testing.assert_allclose(g["dv"], dv_t, atol=1e-12)


def _random_keep_out(sq, sk, seed, p=0.3):
    """A user attention mask (True = masked out) of the given shape."""
    return np.random.default_rng(seed).random((sq, sk)) < p


@pytest.mark.parametrize("sparse_mode", [0, 2])
def test_selected_user_mask_equals_biased_dense(sparse_mode):
    """The user mask (Ascend attenMaskOptional, read as True = masked out over
    sequence-local (query, key) positions, shared by sequences and heads) is
    the dense biased attention with -inf where the mask is set: pinned against
    torch fp64 autograd on a mask built independently of the oracle."""
    q, k, v, do, topk, cu = _tiny_selected(lengths=(24, 16), N2=2, G=2, count=3, D=5, Dv=3, seed=9)
    topk[5, 0] = [1, 1, 0]
    bs, scale = 4, 0.45
    mask = _random_keep_out(24, 24, seed=4)
    bias = _multiplicity_bias(topk, cu, cu, bs, sparse_mode, k.shape[0], mask)
    # rows the mask leaves without any key are tested separately
    live = np.isfinite(bias).any(axis=2).all(axis=1)
    f = oracle.selected_forward(q, k, v, topk, cu, cu, bs, scale, sparse_mode, atten_mask=mask)
    g = oracle.selected_backward(q, k, v, do, topk, cu, cu, bs, scale, sparse_mode, atten_mask=mask)
    do_live = do * live[:, None, None]
    g_live = oracle.selected_backward(q, k, v, do_live, topk, cu, cu, bs, scale, sparse_mode, atten_mask=mask)
    bias_live = np.where(live[:, None, None], bias, 0.0)    # dead rows: any finite bias, zero dO
    o_t, (dq_t, dk_t, dv_t) = _torch_biased(q, k, v, do_live, bias_live, scale)
    np.testing.assert_allclose(f["O"][live], o_t[live], atol=1e-12)
    np.testing.assert_allclose(g_live["dq"][live], dq_t[live], atol=1e-12)
    np.testing.assert_allclose(g_live["dk"], dk_t, atol=1e-12)
    np.testing.assert_allclose(g_live["dv"], dv_t, atol=1e-12)
    # a token whose every gathered key is masked: O = 0, m = -inf, l = 0 and
    # no gradient flows through it
    for t in np.flatnonzero(~live):
        for h in range(q.shape[1]):
            h2 = h // 2
            if not np.isfinite(bias[t, h2]).any():
                assert np.all(f["O"][t, h] == 0) and f["m"][t, h] == -np.inf and f["l"][t, h] == 0
                assert np.all(g["dq"][t, h] == 0)


def test_selected_user_mask_special_cases():
    """An all-False mask changes nothing (bitwise); a mask that is the causal
    pattern under sparse_mode 0 is sparse_mode 2 without a mask (bitwise)."""
    q, k, v, do, topk, cu = _tiny_selected(lengths=(20, 12), N2=1, G=3, count=3, D=4, seed=2)
    bs, scale = 4, 0.5
    none = np.zeros((20, 20), bool)
    a = oracle.selected_backward(q, k, v, do, topk, cu, cu, bs, scale, 2)
    b = oracle.selected_backward(q, k, v, do, topk, cu, cu, bs, scale, 2, atten_mask=none)
    causal_keep_out = np.arange(20)[None, :] > np.arange(20)[:, None]
    c = oracle.selected_backward(q, k, v, do, topk, cu, cu, bs, scale, 0, atten_mask=causal_keep_out)
    for key in ("dq", "dk", "dv"):
        assert np.array_equal(a[key], b[key])
        assert np.array_equal(a[key], c[key])


def test_selected_user_mask_finite_differences():
    q, k, v, do, topk, cu = _tiny_selected(lengths=(32,), N2=1, G=2, D=3, bs=4, count=3, seed=6, Dv=2)
    bs, scale, mode = 4, 0.6, 0
    mask = _random_keep_out(32, 32, seed=8, p=0.4)
    mask[:, 0] = False                          # every token keeps key 0 when block 0 is chosen
    topk[:, 0, 0] = 0
    g = oracle.selected_backward(q, k, v, do, topk, cu, cu, bs, scale, mode, atten_mask=mask)

    def loss(q_, k_, v_):
        return float(np.sum(do * oracle.selected_forward(q_, k_, v_, topk, cu, cu, bs, scale, mode,
                                                          atten_mask=mask)["O"]))

    h = 1e-6
    for j, ref in enumerate((g["dq"], g["dk"], g["dv"])):
        base = [q, k, v]
        x = base[j]
        for idx in [(20, 0, 1), (9, 0, 2), (0, 0, 0), (3, 0, 1), (31, 0, 2), (14, 0, 0)]:
            idx = (idx[0], min(idx[1], x.shape[1] - 1), min(idx[2], x.shape[2] - 1))
            args = [a.copy() for a in base]
            args[j][idx] += h
            lp = loss(*args)
            args[j][idx] -= 2 * h
            lm = loss(*args)
            fd = (lp - lm) / (2 * h)
            assert abs(fd - ref[idx]) <= 1e-7 * max(1.0, np.max(np.abs(ref))), (j, idx, fd, ref[idx])


def test_selected_finite_differences_with_duplicates():
    q, k, v, do, topk, cu = _tiny_selected(lengths=(32,), N2=1, G=2, D=3, bs=4, count=3, seed=3, Dv=2)
    topk[20, 0] = [2, 2, 5]
    bs, scale, mode = 4, 0.6, 2
    g = oracle.selected_backward(q, k, v, do, topk, cu, cu, bs, scale, mode)

    def loss(q_, k_, v_):
        return float(np.sum(do * oracle.selected_forward(q_, k_, v_, topk, cu, cu, bs, scale, mode)["O"]))

    h = 1e-6
    for j, ref in enumerate((g["dq"], g["dk"], g["dv"])):
        base = [q, k, v]
        x = base[j]
        # a sample of coordinates keeps the test quick
        for idx in [(20, 0, 1), (9, 0, 2), (21, 0, 0), (3, 0, 1), (31, 0, 2)]:
            idx = (idx[0], min(idx[1], x.shape[1] - 1), min(idx[2], x.shape[2] - 1))
            args = [a.copy() for a in base]
            args[j][idx] += h
            lp = loss(*args)
            args[j][idx] -= 2 * h
            lm = loss(*args)
            fd = (lp - lm) / (2 * h)
            assert abs(fd - ref[idx]) <= 1e-7 * max(1.0, np.max(np.abs(ref))), (j, idx, fd, ref[idx])


def test_selected_all_blocks_once_is_dense_causal():
    T, N2, G, D, bs = 16, 1, 3, 4, 4
    count = T // bs
    rng = np.random.default_rng(5)
    q, do = rng.standard_normal((T, G, D)), rng.standard_normal((T, G, D))
    k, v = rng.standard_normal((T, N2, D)), rng.standard_normal((T, N2, D))
    topk = np.tile(np.arange(count, dtype=np.int32), (T, N2, 1))
    cu = np.array([T])
    g = oracle.selected_backward(q, k, v, do, topk, cu, cu, bs, 0.5, 2)
    gd = oracle.varlen_backward(q, k, v, do, cu, cu, 0.5, True)
    for key in ("dq", "dk", "dv"):
        np.testing.assert_allclose(g[key], gd[key], atol=1e-13)


def test_ascend_example_closed_form():
    """The page's example: one query token, 1024 keys, every input 2.0 and the
    16 blocks 0..15 of 64 keys selected once (aclnnNsaSelectedAttentionGrad,
    "Example" section; the fill value is read as 2.0).  Every score is equal,
    so P = 1/1024 on each key, dP_j = dY.V_j = 4*D is constant and
    dS = P*(dP - P.dP) = 0: dQ = dK = 0, dV = dY/1024."""
    with open(os.path.join(GOLDEN, "ascend_example.json")) as fh:
        ex = json.load(fh)
    s1, s2, d = ex["s1"], ex["s2"], ex["d"]
    bs, count = ex["selectedBlockSize"], ex["selectedBlockCount"]
    fill = ex["fill_value"]
    q = np.full((s1, ex["n1"], d), fill)
    k = np.full((s2, ex["n2"], d), fill)
    v = np.full((s2, ex["n2"], d), fill)
    dy = np.full((s1, ex["n1"], d), fill)
    topk = np.array(ex["topkIndices"], dtype=np.int32).reshape(s1, ex["n2"], count)
    g = oracle.selected_backward(q, k, v, dy, topk, np.array([s1]), np.array([s2]), bs,
                                 ex["scaleValue"], ex["sparseMode"])
    assert np.all(g["dq"] == 0) and np.all(g["dk"] == 0)
    np.testing.assert_allclose(g["dv"], fill / (count * bs), rtol=1e-15)


# ----------------------------------------------------------------------------
# index path
# ----------------------------------------------------------------------------

def test_positions_brute_force():
    topk = np.array([[[3, 0, 3]], [[1, 2, 0]]], dtype=np.int32)
    pos = oracle.selected_key_positions(topk, 4)
    expect = []
    for t in range(2):
        row = []
        for i in range(3):
            for r in range(4):
                row.append(int(topk[t, 0, i]) * 4 + r)
        expect.append([row])
    np.testing.assert_array_equal(pos, np.array(expect))


@pytest.mark.parametrize("lengths,N2,bs,count", [((64,), 1, 8, 3), ((32, 48, 16), 2, 16, 2)])
def test_block_lists_against_stable_sort(lengths, N2, bs, count):
    topk = synth.draw_topk(np.array(lengths), N2, bs, count, config_id=11)
    cu = np.cumsum(lengths)
    offsets, entries = oracle.selected_block_lists(topk, cu, cu, bs)
    T = int(cu[-1])
    NB = T // bs
    # independent construction: bucket key per (t, h2, slot), stable argsort
    starts = np.concatenate([[0], cu[:-1]])
    seq = np.searchsorted(cu, np.arange(T), side="right")
    blk0 = starts[seq] // bs
    bucket = (np.arange(N2)[None, :, None] * NB + (blk0[:, None, None] + topk)).transpose(1, 0, 2)
    e = (np.arange(T)[:, None] * count + np.arange(count)[None, :])[None].repeat(N2, 0)
    order = np.argsort(bucket.ravel(), kind="stable")
    np.testing.assert_array_equal(entries, e.ravel()[order])
    np.testing.assert_array_equal(offsets, np.searchsorted(np.sort(bucket.ravel()), np.arange(N2 * NB + 1)))
    # invariants: monotone offsets, total = T*N2*count, each list strictly increasing
    assert offsets[0] == 0 and offsets[-1] == T * N2 * count
    assert np.all(np.diff(offsets) >= 0)
    for i in range(N2 * NB):
        seg = entries[offsets[i]:offsets[i + 1]]
        assert np.all(np.diff(seg) > 0)


def test_topk_recipe():
    """The NSA workload's top-k rows: own block present, distinct sorted blocks
    when enough exist, padding with the own block otherwise, all causal."""
    topk = synth.draw_topk(np.array([640]), 1, 64, 4, config_id=5)
    for t in range(640):
        row = topk[t, 0]
        b = t // 64
        assert b in row and np.all(row <= b)
        if b + 1 >= 4:
            assert len(set(row.tolist())) == 4 and list(row) == sorted(row)
        else:
            assert list(row[:b + 1]) == list(range(b + 1)) and np.all(row[b + 1:] == b)
