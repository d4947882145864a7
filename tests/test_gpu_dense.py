"""GPU parity of the dense path (sdpa_fwd_stats, sdpa_bwd) against the fp64 oracle.

Bars: max|err|/max|ref| <= 5e-3 (fp16) / 2e-2 (bf16) for dQ, dK, dV; the fp32
LSE within 1e-4 absolute.  Outputs are pre-filled with NaN so an element the
kernels fail to write fails the comparison."""
import math

import numpy as np
import pytest
import torch

import oracle
import sdpa_backward_fa2_amd as sb
import synth
from gpu_util import (REL_TOL, STATS_ABS_TOL, TORCH_DTYPE, assert_rel, dense_input,
                      empty_like_layout, to_device, to_f64)

pytestmark = pytest.mark.gpu


def _nan_like(t):
    return empty_like_layout(t).fill_(float("nan"))


def _run_bwd(q, k, v, o, do, lse, scale, causal, det):
    dq, dk, dv = _nan_like(q), _nan_like(k), _nan_like(v)
    sb.bwd(q, k, v, o, do, lse, scale, causal, deterministic=det, dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    return dq, dk, dv


def _random_case(B, Hq, Hkv, Sq, Sk, D, dtype, layout, seed, Dv=None):
    """Small random problem: physical layout bshd or bhsd, N(0,1) inputs; V and
    dO have head dim Dv (default D)."""
    rng = np.random.default_rng(seed)
    Dv = D if Dv is None else Dv
    out = {}
    for name, H, S, d in (("q", Hq, Sq, D), ("k", Hkv, Sk, D), ("v", Hkv, Sk, Dv), ("do", Hq, Sq, Dv)):
        shape = (B, S, H, d) if layout == "bshd" else (B, H, S, d)
        bits = synth.encode(rng.standard_normal(shape), dtype)
        t = to_device(bits, dtype)
        x = synth.decode(bits, dtype)
        if layout == "bshd":
            t, x = t.permute(0, 2, 1, 3), x.transpose(0, 2, 1, 3)
        out[name] = (t, x)
    return out


def _check_case(B, Hq, Hkv, Sq, Sk, D, dtype, causal, layout, seed=0, stats="gpu", Dv=None):
    case = _random_case(B, Hq, Hkv, Sq, Sk, D, dtype, layout, seed, Dv)
    (q, qx), (k, kx), (v, vx), (do, dox) = case["q"], case["k"], case["v"], case["do"]
    scale = 1.0 / math.sqrt(D)
    f = oracle.dense_forward(qx, kx, vx, scale, causal)
    if stats == "gpu":
        o = _nan_like(do)
        lse = torch.full((B, Hq, Sq), float("nan"), device="cuda")
        sb.fwd_stats(q, k, v, scale, causal, o=o, lse=lse)
        torch.cuda.synchronize()
        assert np.max(np.abs(to_f64(lse) - f["lse"])) <= STATS_ABS_TOL
        assert_rel(to_f64(o), f["O"], dtype, "O")
    else:
        o = to_device(synth.encode(f["O"], dtype), dtype)
        lse = torch.tensor(f["lse"], dtype=torch.float32, device="cuda")
    g = oracle.dense_backward(qx, kx, vx, dox, scale, causal)
    for det in _modes(D, v.shape[-1]):
        dq, dk, dv = _run_bwd(q, k, v, o, do, lse, scale, causal, det)
        for name, got, ref in (("dq", dq, g["dq"]), ("dk", dk, g["dk"]), ("dv", dv, g["dv"])):
            assert_rel(to_f64(got), ref, dtype, f"{name} det={det}")


def _modes(D, Dv=None):
    """dQ modes offered at head dims (D, Dv): no fp32-atomic form at D=192."""
    return (0, 1) if D == 192 or (Dv is not None and Dv != D) else (0, 1, 2)


# ----------------------------------------------------------------------------
# The benchmark workloads
# ----------------------------------------------------------------------------

def test_config1_tiny_dense():
    """B=1, H=2, S=128, D=64 fp16, BHSD, non-causal; O and LSE from the oracle."""
    wl = synth.workload(1)
    q, qx = dense_input(wl, synth.TID_Q, wl.Hq)
    k, kx = dense_input(wl, synth.TID_K, wl.Hkv)
    v, vx = dense_input(wl, synth.TID_V, wl.Hkv)
    do, dox = dense_input(wl, synth.TID_DO, wl.Hq)
    f = oracle.dense_forward(qx, kx, vx, wl.scale, wl.causal)
    o = to_device(synth.encode(f["O"], wl.dtype), wl.dtype)
    lse = torch.tensor(f["lse"][..., None], dtype=torch.float32, device="cuda")   # (B,H,S,1)
    g = oracle.dense_backward(qx, kx, vx, dox, wl.scale, wl.causal)
    for det in (0, 1, 2):
        dq, dk, dv = _run_bwd(q, k, v, o, do, lse, wl.scale, wl.causal, det)
        for name, got, ref in (("dq", dq, g["dq"]), ("dk", dk, g["dk"]), ("dv", dv, g["dv"])):
            assert_rel(to_f64(got), ref, wl.dtype, f"config1 {name} det={det}")


def _gpu_stats_config(cid, heads=None):
    wl = synth.workload(cid)
    q, qx = dense_input(wl, synth.TID_Q, wl.Hq)
    k, kx = dense_input(wl, synth.TID_K, wl.Hkv)
    v, vx = dense_input(wl, synth.TID_V, wl.Hkv)
    do, dox = dense_input(wl, synth.TID_DO, wl.Hq)
    o, lse = sb.fwd_stats(q, k, v, wl.scale, wl.causal, o=_nan_like(q))
    torch.cuda.synchronize()
    return wl, (q, k, v, do, o, lse), (qx, kx, vx, dox)


def _sampled_forward(qx, kx, vx, scale, causal, heads):
    out = {}
    for b, h in heads:
        allowed = oracle.causal_mask(qx.shape[2], kx.shape[2]) if causal else None
        out[(b, h)] = oracle.head_forward(qx[b, h], kx[b, h], vx[b, h], scale, allowed)
    return out


def test_config2_gpt2_shape():
    """B=4, H=12, S=1024, D=64 fp16, BSHD physical / BHSD logical, causal, LSE from
    the GPU forward.  Full oracle comparison."""
    wl, (q, k, v, do, o, lse), (qx, kx, vx, dox) = _gpu_stats_config(2)
    f = oracle.dense_forward(qx, kx, vx, wl.scale, wl.causal)
    assert np.max(np.abs(to_f64(lse) - f["lse"])) <= STATS_ABS_TOL
    assert_rel(to_f64(o), f["O"], wl.dtype, "config2 O")
    g = oracle.dense_backward(qx, kx, vx, dox, wl.scale, wl.causal)
    for det in (0, 1, 2):
        dq, dk, dv = _run_bwd(q, k, v, o, do, lse, wl.scale, wl.causal, det)
        for name, got, ref in (("dq", dq, g["dq"]), ("dk", dk, g["dk"]), ("dv", dv, g["dv"])):
            assert_rel(to_f64(got), ref, wl.dtype, f"config2 {name} det={det}")


def test_config3_long_context_sampled_heads():
    """B=2, H=16, S=4096, D=128 bf16, BSHD, causal: the GPU runs the full
    problem; the oracle checks three whole heads (every row and key of them)."""
    wl, (q, k, v, do, o, lse), (qx, kx, vx, dox) = _gpu_stats_config(3)
    heads = [(0, 0), (1, 7), (1, 15)]
    fs = _sampled_forward(qx, kx, vx, wl.scale, wl.causal, heads)
    lse_np, o_np = to_f64(lse), None
    for (b, h), f in fs.items():
        assert np.max(np.abs(lse_np[b, h] - f["lse"])) <= STATS_ABS_TOL
        assert_rel(to_f64(o[b, h]), f["O"], wl.dtype, f"config3 O[{b},{h}]")
    g = oracle.dense_backward(qx, kx, vx, dox, wl.scale, wl.causal, heads=heads)
    for det in (0, 1, 2):
        dq, dk, dv = _run_bwd(q, k, v, o, do, lse, wl.scale, wl.causal, det)
        for b, h in heads:
            for name, got, ref in (("dq", dq, g["dq"]), ("dk", dk, g["dk"]), ("dv", dv, g["dv"])):
                assert_rel(to_f64(got[b, h]), ref[b, h], wl.dtype, f"config3 {name}[{b},{h}] det={det}")
        # nothing left unwritten anywhere
        for t in (dq, dk, dv):
            assert not torch.isnan(t).any()


# ----------------------------------------------------------------------------
# Shape sweep: ragged tails, both causal settings, D 64/128, both dtypes, GQA
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("D", [64, 128, 192])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("S", [1, 37, 128, 200, 385])
def test_sweep_square(dtype, D, causal, S):
    _check_case(2, 2, 2, S, S, D, dtype, causal, "bshd", seed=S + D)


@pytest.mark.parametrize("Sq,Sk", [(64, 300), (257, 129), (5, 1)])
def test_sweep_rectangular_noncausal(Sq, Sk):
    _check_case(1, 3, 3, Sq, Sk, 64, "f16", False, "bhsd", seed=Sq * Sk)


@pytest.mark.parametrize("D,dtype", [(64, "f16"), (128, "bf16"), (192, "f16")])
@pytest.mark.parametrize("Sq,Sk", [(64, 300), (257, 129), (5, 1), (1, 77), (200, 64), (130, 131)])
def test_sweep_rectangular_causal(Sq, Sk, D, dtype):
    """Causal with Sq != Sk, top-left aligned: keys past the last query get
    dK = dV = 0, queries past the last key see every key."""
    _check_case(1, 3, 3, Sq, Sk, D, dtype, True, "bshd", seed=Sq * Sk + D)


def test_rectangular_causal_gqa():
    _check_case(2, 4, 2, 96, 230, 128, "f16", True, "bhsd", seed=77)


@pytest.mark.parametrize("D", [64, 128, 192])
@pytest.mark.parametrize("Hq,Hkv", [(4, 2), (6, 1)])
@pytest.mark.parametrize("causal", [False, True])
def test_gqa(Hq, Hkv, causal, D):
    _check_case(2, Hq, Hkv, 160, 160, D, "bf16", causal, "bshd", seed=Hq + D)


def test_oracle_stats_max_sum_form():
    """Dense call fed the (max, sum) statistics instead of LSE."""
    case = _random_case(1, 2, 2, 96, 96, 64, "f16", "bhsd", 3)
    (q, qx), (k, kx), (v, vx), (do, dox) = case["q"], case["k"], case["v"], case["do"]
    f = oracle.dense_forward(qx, kx, vx, 0.125, True)
    o = to_device(synth.encode(f["O"], "f16"), "f16")
    m = torch.tensor(f["m"], dtype=torch.float32, device="cuda")
    s = torch.tensor(f["l"], dtype=torch.float32, device="cuda")
    g = oracle.dense_backward(qx, kx, vx, dox, 0.125, True)
    dq, dk, dv = _run_bwd(q, k, v, o, do, (m, s), 0.125, True, False)
    for name, got, ref in (("dq", dq, g["dq"]), ("dk", dk, g["dk"]), ("dv", dv, g["dv"])):
        assert_rel(to_f64(got), ref, "f16", name)


@pytest.mark.parametrize("cid", [2, 3])
def test_dq_modes(cid):
    """Mode 1 is bitwise stable; mode 0 (fastest) is today the same atomic-free
    pass, so bitwise equal to it; mode 2 (fp32 atomics, D=64 and D=128) agrees within
    the tolerance."""
    wl, (q, k, v, do, o, lse), _ = _gpu_stats_config(cid)
    a = _run_bwd(q, k, v, o, do, lse, wl.scale, wl.causal, 1)
    b = _run_bwd(q, k, v, o, do, lse, wl.scale, wl.causal, 1)
    f = _run_bwd(q, k, v, o, do, lse, wl.scale, wl.causal, 0)
    for x, y, z in zip(a, b, f):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))
        assert torch.equal(x.view(torch.int16), z.view(torch.int16))
    c = _run_bwd(q, k, v, o, do, lse, wl.scale, wl.causal, 2)
    for x, y in zip(a, c):
        e = float((x.float() - y.float()).abs().max() / x.float().abs().max())
        assert e <= REL_TOL[wl.dtype]


def test_d192_longer_causal_from_gpu_forward():
    """D=192 over several 128-key tiles and 64-row query tiles with a ragged
    tail, O and LSE from the library's own forward."""
    _check_case(2, 4, 2, 700, 700, 192, "bf16", True, "bshd", seed=192)


def test_d192_atomic_mode_is_unsupported():
    case = _random_case(1, 2, 2, 64, 64, 192, "f16", "bhsd", 1)
    q, k, v, do = (case[n][0] for n in ("q", "k", "v", "do"))
    o, lse = sb.fwd_stats(q, k, v, 0.1, True)
    with pytest.raises(sb.SdpaError) as e:
        sb.bwd(q, k, v, o, do, lse, 0.1, True, deterministic=2)
    assert e.value.status == 3   # SDPA_ERR_UNSUPPORTED


# ----------------------------------------------------------------------------
# Query/key head dim 192 with value head dim 128
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("S", [1, 37, 128, 200, 385])
def test_dqk192_dv128_square(dtype, causal, S):
    _check_case(2, 2, 2, S, S, 192, dtype, causal, "bshd", seed=S + 320, Dv=128)


@pytest.mark.parametrize("Sq,Sk", [(64, 300), (257, 129), (5, 1), (130, 131)])
def test_dqk192_dv128_rectangular_causal(Sq, Sk):
    _check_case(1, 3, 3, Sq, Sk, 192, "bf16", True, "bhsd", seed=Sq + Sk, Dv=128)


@pytest.mark.parametrize("Hq,Hkv", [(4, 2), (6, 1)])
def test_dqk192_dv128_gqa(Hq, Hkv):
    _check_case(2, Hq, Hkv, 160, 160, 192, "f16", True, "bshd", seed=Hq * 7, Dv=128)


def test_dqk192_dv128_longer_causal():
    """Several key tiles and a ragged tail; O and LSE from the library's forward."""
    _check_case(2, 4, 2, 700, 700, 192, "bf16", True, "bshd", seed=1920, Dv=128)


def test_dqk192_dv128_oracle_stats():
    """Statistics and O from the oracle instead of the library's forward."""
    _check_case(1, 2, 2, 300, 300, 192, "f16", False, "bhsd", seed=5, stats="oracle", Dv=128)


def test_dqk192_dv128_atomic_mode_is_unsupported():
    case = _random_case(1, 2, 2, 64, 64, 192, "f16", "bhsd", 1, Dv=128)
    q, k, v, do = (case[n][0] for n in ("q", "k", "v", "do"))
    o, lse = sb.fwd_stats(q, k, v, 0.1, True)
    assert o.shape[-1] == 128
    with pytest.raises(sb.SdpaError) as e:
        sb.bwd(q, k, v, o, do, lse, 0.1, True, deterministic=2)
    assert e.value.status == 3   # SDPA_ERR_UNSUPPORTED
