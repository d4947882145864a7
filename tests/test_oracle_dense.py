"""Pins for the dense part of the fp64 oracle.

Each test checks the oracle against something other than its own formula:
central finite differences of the scalar loss sum(dO * O), closed forms,
invariants of the softmax gradient, and torch fp64 autograd on the CPU (the
cuDNN sample's own checking recipe, run in fp64: cudnn-frontend notebook, last
code cell).
"""
import math

import numpy as np
import pytest
import torch

import oracle

RNG = np.random.default_rng(1234)


def _rand(*shape):
    return RNG.standard_normal(shape)


def _loss(q, k, v, do, scale, allowed):
    return float(np.sum(do * oracle.head_forward(q, k, v, scale, allowed)["O"]))


def _finite_diff(q, k, v, do, scale, allowed, h=1e-6):
    grads = []
    for which in range(3):
        args = [q.copy(), k.copy(), v.copy()]
        x = args[which]
        g = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            old = x[idx]
            x[idx] = old + h
            lp = _loss(*args, do, scale, allowed)
            x[idx] = old - h
            lm = _loss(*args, do, scale, allowed)
            x[idx] = old
            g[idx] = (lp - lm) / (2 * h)
        grads.append(g)
    return grads


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("sq,sk,d,dv", [(5, 5, 3, 3), (7, 7, 4, 2), (3, 6, 2, 4), (6, 3, 3, 2)])
def test_finite_differences(causal, sq, sk, d, dv):
    q, k, v, do = _rand(sq, d), _rand(sk, d), _rand(sk, dv), _rand(sq, dv)
    scale = 0.7
    allowed = oracle.causal_mask(sq, sk) if causal else None
    g = oracle.head_backward(q, k, v, do, scale, allowed)
    fq, fk, fv = _finite_diff(q, k, v, do, scale, allowed)
    for name, a, b in (("dq", g["dq"], fq), ("dk", g["dk"], fk), ("dv", g["dv"], fv)):
        err = np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-30)
        assert err < 1e-7, (name, err)


def test_softmax_jacobian_explicit():
    """dS from the oracle equals J(p_i) dP_i with J = diag(p) - p p^T formed
    explicitly, row by row."""
    sq, sk, d = 6, 6, 3
    q, k, v, do = _rand(sq, d), _rand(sk, d), _rand(sk, d), _rand(sq, d)
    g = oracle.head_backward(q, k, v, do, 0.5, oracle.causal_mask(sq, sk))
    for i in range(sq):
        p = g["P"][i]
        J = np.diag(p) - np.outer(p, p)
        np.testing.assert_allclose(g["dS"][i], J @ g["dP"][i], rtol=0, atol=1e-13)


def test_flash_backward_identity():
    """The FlashAttention-2 form dS = P * (dP - Delta), Delta_i = rowsum(dO*O),
    reproduces the oracle's Jacobian route (the GPU relies on this)."""
    sq, sk, d = 9, 9, 5
    q, k, v, do = _rand(sq, d), _rand(sk, d), _rand(sk, d), _rand(sq, d)
    for allowed in (None, oracle.causal_mask(sq, sk)):
        g = oracle.head_backward(q, k, v, do, 0.3, allowed)
        delta = oracle.rowsum_do_o(do, g["O"])
        np.testing.assert_allclose(g["P"] * (g["dP"] - delta[:, None]), g["dS"],
                                   rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_invariants(causal):
    sq = sk = 11
    d = 4
    q, k, v, do = _rand(sq, d), _rand(sk, d), _rand(sk, d), _rand(sq, d)
    allowed = oracle.causal_mask(sq, sk) if causal else None
    g = oracle.head_backward(q, k, v, do, 0.4, allowed)
    # every row of dS sums to zero (softmax rows sum to one)
    np.testing.assert_allclose(g["dS"].sum(axis=1), 0.0, atol=1e-13)
    # column sum of dV equals the column sum of dO
    np.testing.assert_allclose(g["dv"].sum(axis=0), do.sum(axis=0), atol=1e-12)
    # shifting every key by the same vector leaves the softmax unchanged -> sum dK = 0
    np.testing.assert_allclose(g["dk"].sum(axis=0), 0.0, atol=1e-12)
    # V -> V + 1 c^T shifts O by c and leaves dQ and dK unchanged
    c = _rand(d)
    g2 = oracle.head_backward(q, k, v + c[None, :], do, 0.4, allowed)
    np.testing.assert_allclose(g2["dq"], g["dq"], atol=1e-12)
    np.testing.assert_allclose(g2["dk"], g["dk"], atol=1e-12)


def test_closed_forms():
    d = 4
    # one key: softmax is the constant 1, so dQ = dK = 0 and dV = sum_i dO_i
    q, k, v, do = _rand(6, d), _rand(1, d), _rand(1, d), _rand(6, d)
    g = oracle.head_backward(q, k, v, do, 0.9)
    assert np.all(g["dq"] == 0) and np.all(g["dk"] == 0)
    np.testing.assert_allclose(g["dv"][0], do.sum(axis=0), atol=1e-13)
    # causal row 0 sees only key 0 -> its dQ is zero
    q, k, v, do = _rand(5, d), _rand(5, d), _rand(5, d), _rand(5, d)
    g = oracle.head_backward(q, k, v, do, 0.9, oracle.causal_mask(5, 5))
    np.testing.assert_allclose(g["dq"][0], 0.0, atol=1e-15)
    # constant V -> O constant in Q, K -> dQ = dK = 0
    vc = np.tile(_rand(1, d), (5, 1))
    g = oracle.head_backward(q, k, vc, do, 0.9, oracle.causal_mask(5, 5))
    np.testing.assert_allclose(g["dq"], 0.0, atol=1e-13)
    np.testing.assert_allclose(g["dk"], 0.0, atol=1e-13)
    # constant K -> uniform P over the admissible set:
    #   LSE_i = s q_i.k + ln n_i, O_i = mean of the admissible V rows
    kc = np.tile(_rand(1, d), (5, 1))
    f = oracle.head_forward(q, kc, v, 0.9, oracle.causal_mask(5, 5))
    n = np.arange(1, 6)
    np.testing.assert_allclose(f["lse"], 0.9 * q @ kc[0] + np.log(n), atol=1e-13)
    np.testing.assert_allclose(f["O"], np.cumsum(v, axis=0) / n[:, None], atol=1e-13)
    np.testing.assert_allclose(f["m"], 0.9 * q @ kc[0], atol=1e-13)
    np.testing.assert_allclose(f["l"], n, atol=1e-13)


def test_two_key_sigmoid_closed_form():
    """With two keys the softmax is a logistic function: p = sigma(z),
    z = s q.(k1 - k2), O = p v1 + (1-p) v2.  Its gradients in closed form:
    dL/dq = s p (1-p) (dO.(v1-v2)) (k1-k2), dL/dk1 = s p(1-p) (dO.(v1-v2)) q,
    dL/dk2 = -dL/dk1, dL/dv1 = p dO, dL/dv2 = (1-p) dO."""
    s = 0.6
    q = np.array([[0.3, -1.2, 0.5]])
    k = np.array([[1.0, 0.2, -0.4], [-0.7, 0.9, 0.1]])
    v = np.array([[0.5, 2.0, -1.0], [1.5, -0.25, 0.75]])
    do = np.array([[0.2, -0.3, 1.1]])
    z = s * float(q[0] @ (k[0] - k[1]))
    p = 1.0 / (1.0 + math.exp(-z))
    w = p * (1 - p) * float(do[0] @ (v[0] - v[1]))
    g = oracle.head_backward(q, k, v, do, s)
    np.testing.assert_allclose(g["dq"][0], s * w * (k[0] - k[1]), atol=1e-15)
    np.testing.assert_allclose(g["dk"][0], s * w * q[0], atol=1e-15)
    np.testing.assert_allclose(g["dk"][1], -s * w * q[0], atol=1e-15)
    np.testing.assert_allclose(g["dv"][0], p * do[0], atol=1e-15)
    np.testing.assert_allclose(g["dv"][1], (1 - p) * do[0], atol=1e-15)
    np.testing.assert_allclose(g["lse"][0], math.log(math.exp(s * q[0] @ k[0]) + math.exp(s * q[0] @ k[1])),
                               atol=1e-15)


def _torch_reference(q, k, v, do, scale, causal):
    """torch fp64 CPU SDPA + autograd (the sample's checking recipe, in fp64)."""
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    hq, hkv = q.shape[1], k.shape[1]
    o = torch.nn.functional.scaled_dot_product_attention(
        tq, tk, tv, is_causal=causal, scale=scale, enable_gqa=(hq != hkv))
    gq, gk, gv = torch.autograd.grad(o, (tq, tk, tv), torch.tensor(do, dtype=torch.float64))
    return o.detach().numpy(), gq.numpy(), gk.numpy(), gv.numpy()


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("hq,hkv", [(2, 2), (4, 2), (6, 1)])
def test_against_torch_fp64(causal, hq, hkv):
    B, S, D = 2, 33, 16
    q, do = _rand(B, hq, S, D), _rand(B, hq, S, D)
    k, v = _rand(B, hkv, S, D), _rand(B, hkv, S, D)
    scale = 1 / math.sqrt(D)
    f = oracle.dense_forward(q, k, v, scale, causal)
    g = oracle.dense_backward(q, k, v, do, scale, causal)
    o_t, dq_t, dk_t, dv_t = _torch_reference(q, k, v, do, scale, causal)
    np.testing.assert_allclose(f["O"], o_t, atol=1e-12)
    np.testing.assert_allclose(g["dq"], dq_t, atol=1e-12)
    np.testing.assert_allclose(g["dk"], dk_t, atol=1e-12)
    np.testing.assert_allclose(g["dv"], dv_t, atol=1e-12)
    # the stats: LSE, and the max/sum pair it is built from
    np.testing.assert_allclose(f["lse"], f["m"] + np.log(f["l"]), atol=1e-13)
    ref_lse = torch.logsumexp(
        torch.tensor(scale * np.einsum("bhqd,bhkd->bhqk", q, np.repeat(k, hq // hkv, axis=1)))
        .masked_fill(~torch.tensor(oracle.causal_mask(S, S)) if causal else torch.zeros(S, S, dtype=torch.bool),
                     float("-inf")), dim=-1).numpy()
    np.testing.assert_allclose(f["lse"], ref_lse, atol=1e-12)


@pytest.mark.parametrize("sq,sk", [(19, 45), (45, 19)])
def test_causal_unequal_lengths_against_torch_fp64(sq, sk):
    """Causal with Sq != Sk: the top-left alignment of torch's is_causal (the
    sample's checking recipe).  Keys past the last query get no gradient, and
    queries past the last key equal the unmasked rows."""
    B, H, D = 2, 2, 8
    q, do = _rand(B, H, sq, D), _rand(B, H, sq, D)
    k, v = _rand(B, H, sk, D), _rand(B, H, sk, D)
    scale = 0.3
    f = oracle.dense_forward(q, k, v, scale, True)
    g = oracle.dense_backward(q, k, v, do, scale, True)
    o_t, dq_t, dk_t, dv_t = _torch_reference(q, k, v, do, scale, True)
    for got, ref in ((f["O"], o_t), (g["dq"], dq_t), (g["dk"], dk_t), (g["dv"], dv_t)):
        np.testing.assert_allclose(got, ref, atol=1e-12)
    if sk > sq:
        assert np.all(g["dk"][:, :, sq:] == 0) and np.all(g["dv"][:, :, sq:] == 0)
    else:
        full = oracle.dense_forward(q, k, v, scale, False)
        np.testing.assert_allclose(f["O"][:, :, sk:], full["O"][:, :, sk:], atol=1e-13)
        np.testing.assert_allclose(f["lse"][:, :, sk:], full["lse"][:, :, sk:], atol=1e-13)


def test_dense_heads_subset_matches_full():
    B, H, S, D = 2, 3, 17, 8
    q, k, v, do = (_rand(B, H, S, D) for _ in range(4))
    full = oracle.dense_backward(q, k, v, do, 0.35, True)
    part = oracle.dense_backward(q, k, v, do, 0.35, True, heads=[(1, 2)])
    for key in ("dq", "dk", "dv"):
        np.testing.assert_array_equal(part[key][1, 2], full[key][1, 2])
        assert np.all(part[key][0] == 0)
