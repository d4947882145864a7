"""GPU parity of the causal D=64 launch in its two-wavefront form (taken for
causal problems of at most 2048 keys with at least one work item per
workgroup slot, four slots per CU: 1024 items on a 256-CU MI355X).  Each case
satisfies that rule; the GPU runs the whole problem with O and the LSE from
the GPU forward, and the fp64 oracle checks sampled (batch, KV head) groups in
full.  Outputs start as NaN.  Bars: max|err|/max|ref| <= 5e-3 (fp16), 2e-2
(bf16)."""
import math

import numpy as np
import pytest
import torch

import oracle
import sdpa_backward_fa2_amd as sb
import synth
from gpu_util import STATS_ABS_TOL, assert_rel, empty_like_layout, to_device, to_f64

pytestmark = pytest.mark.gpu

CUS = 256


def _two_wave(B, Hq, Hkv, Sq, Sk):
    items = B * Hkv * math.ceil(Sk / 64) + B * Hq * math.ceil(Sq / 64)
    return math.ceil(Sk / 64) <= 32 and items >= 4 * CUS


def _nan_like(t):
    return empty_like_layout(t).fill_(float("nan"))


def _case(B, Hq, Hkv, Sq, Sk, dtype, groups, seed, grad_dtype=None):
    D = 64
    assert _two_wave(B, Hq, Hkv, Sq, Sk), "case must take the two-wavefront form"
    assert torch.cuda.get_device_properties(0).multi_processor_count == CUS
    rng = np.random.default_rng(seed)
    dev, host = {}, {}
    for name, H, S in (("q", Hq, Sq), ("k", Hkv, Sk), ("v", Hkv, Sk), ("do", Hq, Sq)):
        bits = synth.encode(rng.standard_normal((B, S, H, D)), dtype)   # BSHD physical
        dev[name] = to_device(bits, dtype).permute(0, 2, 1, 3)
        host[name] = synth.decode(bits, dtype).transpose(0, 2, 1, 3)
    scale = 1.0 / math.sqrt(D)
    q, k, v, do = dev["q"], dev["k"], dev["v"], dev["do"]
    print(f"two-wave case B={B} Hq={Hq} Hkv={Hkv} Sq={Sq} Sk={Sk} {dtype} grads={grad_dtype}", flush=True)
    o, lse = sb.fwd_stats(q, k, v, scale, True)
    torch.cuda.synchronize()
    G = Hq // Hkv
    allowed = oracle.causal_mask(Sq, Sk)
    lse_np = to_f64(lse)
    for b, hk in groups:
        for h in range(hk * G, (hk + 1) * G):
            f = oracle.head_forward(host["q"][b, h], host["k"][b, hk], host["v"][b, hk], scale, allowed)
            assert np.max(np.abs(lse_np[b, h] - f["lse"])) <= STATS_ABS_TOL
    g = oracle.dense_backward(host["q"], host["k"], host["v"], host["do"], scale, True, heads=groups)
    gt = q.dtype if grad_dtype is None else grad_dtype
    results = []
    for det in (0, 1):
        dq = _nan_like(q).to(gt)
        dk = _nan_like(k).to(gt)
        dv = _nan_like(v).to(gt)
        sb.bwd(q, k, v, o, do, lse, scale, True, deterministic=det, dq=dq, dk=dk, dv=dv)
        torch.cuda.synchronize()
        for t in (dq, dk, dv):
            assert not torch.isnan(t).any(), "unwritten gradient elements"
        for b, hk in groups:
            assert_rel(to_f64(dk[b, hk]), g["dk"][b, hk], dtype, f"dk[{b},{hk}] det={det}")
            assert_rel(to_f64(dv[b, hk]), g["dv"][b, hk], dtype, f"dv[{b},{hk}] det={det}")
            for h in range(hk * G, (hk + 1) * G):
                assert_rel(to_f64(dq[b, h]), g["dq"][b, h], dtype, f"dq[{b},{h}] det={det}")
        results.append((dq, dk, dv))
    for x, y in zip(*results):            # atomic-free: both modes give the same bits
        assert torch.equal(x, y)


def test_ragged_rows():
    """S=1000: the last query and key tiles are partial."""
    _case(8, 12, 12, 1000, 1000, "f16", [(0, 0), (5, 7), (7, 11)], seed=41)


def test_bf16():
    _case(6, 16, 16, 1024, 1024, "bf16", [(1, 3), (5, 15)], seed=42)


def test_gqa():
    """Four query heads per KV head: dK/dV sum over the group; key-tile items
    first, then query tiles (no alternating order)."""
    _case(8, 16, 4, 1024, 1024, "f16", [(0, 1), (7, 3)], seed=43)


def test_long_keys():
    """2000 keys: the longest items at the form's limit."""
    _case(2, 16, 16, 2000, 2000, "f16", [(0, 0), (1, 15)], seed=46)


@pytest.mark.parametrize("Sq,Sk", [(1000, 1200), (1200, 1000)])
def test_rectangular(Sq, Sk):
    """Top-left aligned causal with Sq != Sk."""
    _case(8, 12, 12, Sq, Sk, "f16", [(0, 2), (7, 9)], seed=44)


def test_fp32_gradients():
    _case(8, 12, 12, 1024, 1024, "f16", [(2, 5)], seed=45, grad_dtype=torch.float32)
