"""GPU parity of the causal D=64 launch in its four-wavefront form at sizes
where its query-tile items cover 128 rows: causal, when 64-row items would
outnumber the GPU's workgroup slots (two per CU, 512 on a 256-CU MI355X) but
the problem does not take the two-wavefront form (more than 2048 keys, or
fewer than 1024 two-wavefront items).  Non-causal shapes of the same size
keep 64-row items and are covered too.  The GPU runs
the whole problem, with O and the LSE from the GPU forward; the fp64 oracle
checks sampled (batch, KV head) groups in full, forward statistics included.
Outputs start as NaN, so an element no kernel writes fails the check.  Bars as
for every backward test: max|err|/max|ref| <= 5e-3 (fp16), 2e-2 (bf16)."""
import math

import numpy as np
import pytest
import torch

import oracle
import sdpa_backward_fa2_amd as sb
import synth
from gpu_util import STATS_ABS_TOL, assert_rel, empty_like_layout, to_device, to_f64

pytestmark = pytest.mark.gpu


def _nan_like(t):
    return empty_like_layout(t).fill_(float("nan"))


def _items64(B, Hq, Hkv, Sq, Sk):
    """Work items of the 64-row form: key tiles per (batch, KV head) plus
    64-row query tiles per (batch, query head)."""
    return B * Hkv * math.ceil(Sk / 64) + B * Hq * math.ceil(Sq / 64)


def _dense(B, Hq, Hkv, Sq, Sk, dtype, causal, groups, seed):
    D = 64
    n = _items64(B, Hq, Hkv, Sq, Sk)
    assert n > 512 and (n < 1024 or math.ceil(Sk / 64) > 32), "case must take the 128-row four-wavefront form"
    rng = np.random.default_rng(seed)
    dev, host = {}, {}
    for name, H, S in (("q", Hq, Sq), ("k", Hkv, Sk), ("v", Hkv, Sk), ("do", Hq, Sq)):
        bits = synth.encode(rng.standard_normal((B, S, H, D)), dtype)   # BSHD physical
        dev[name] = to_device(bits, dtype).permute(0, 2, 1, 3)
        host[name] = synth.decode(bits, dtype).transpose(0, 2, 1, 3)
    scale = 1.0 / math.sqrt(D)
    q, k, v, do = dev["q"], dev["k"], dev["v"], dev["do"]
    o = _nan_like(q)
    lse = torch.full((B, Hq, Sq), float("nan"), device="cuda")
    sb.fwd_stats(q, k, v, scale, causal, o=o, lse=lse)
    torch.cuda.synchronize()
    G = Hq // Hkv
    allowed = oracle.causal_mask(Sq, Sk) if causal else None
    lse_np = to_f64(lse)
    for b, hk in groups:
        for h in range(hk * G, (hk + 1) * G):
            f = oracle.head_forward(host["q"][b, h], host["k"][b, hk], host["v"][b, hk], scale, allowed)
            assert np.max(np.abs(lse_np[b, h] - f["lse"])) <= STATS_ABS_TOL
            assert_rel(to_f64(o[b, h]), f["O"], dtype, f"O[{b},{h}]")
    g = oracle.dense_backward(host["q"], host["k"], host["v"], host["do"], scale, causal, heads=groups)
    results = []
    for det in (0, 1):
        dq, dk, dv = _nan_like(q), _nan_like(k), _nan_like(v)
        sb.bwd(q, k, v, o, do, lse, scale, causal, deterministic=det, dq=dq, dk=dk, dv=dv)
        torch.cuda.synchronize()
        for t in (dq, dk, dv):
            assert not torch.isnan(t).any(), "unwritten gradient elements"
        for b, hk in groups:
            assert_rel(to_f64(dk[b, hk]), g["dk"][b, hk], dtype, f"dk[{b},{hk}] det={det}")
            assert_rel(to_f64(dv[b, hk]), g["dv"][b, hk], dtype, f"dv[{b},{hk}] det={det}")
            for h in range(hk * G, (hk + 1) * G):
                assert_rel(to_f64(dq[b, h]), g["dq"][b, h], dtype, f"dq[{b},{h}] det={det}")
        results.append((dq, dk, dv))
    # the launch is atomic-free: both modes give the same bits
    for x, y in zip(*results):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))


@pytest.mark.parametrize("causal", [True, False])
def test_ragged_rows(causal):
    """S=1000: the last 128-row query tile holds 104 rows, the last key tile 40
    keys.  Causal takes the three-item order; non-causal, 64-row items."""
    _dense(2, 10, 10, 1000, 1000, "f16", causal, [(0, 0), (1, 5), (1, 9)], seed=31)


def test_bf16_causal():
    _dense(2, 10, 10, 1024, 1024, "bf16", True, [(1, 3), (0, 9)], seed=32)


def test_gqa_causal():
    """Four query heads per KV head: the dK/dV items sum over the group; the
    key tiles go first (no two- or three-item order)."""
    _dense(2, 16, 4, 1024, 1024, "f16", True, [(0, 1), (1, 3)], seed=33)


@pytest.mark.parametrize("Sq,Sk", [(1000, 1200), (1200, 1000)])
def test_rectangular_causal(Sq, Sk):
    """Causal, top-left aligned: with Sq < Sk the last keys are seen by no
    query (zero dK, dV); with Sq > Sk the rows past Sk see every key."""
    _dense(2, 8, 8, Sq, Sk, "f16", True, [(0, 2), (1, 4)], seed=34)


def test_packed_ragged_sequences():
    """Six packed sequences of uneven lengths, H=16: the three-item order runs
    over the longest sequence's tiles; shorter sequences' tiles past their end
    do nothing."""
    D, H, dtype = 64, 16, "f16"
    lengths = [2100, 333, 1024, 64, 777, 1201]      # longest above 2048 keys
    cu = np.cumsum(lengths)
    T = int(cu[-1])
    assert len(lengths) * H * (2 * math.ceil(max(lengths) / 64)) >= 1024
    rng = np.random.default_rng(35)
    dev, host = {}, {}
    for name in ("q", "k", "v", "do"):
        bits = synth.encode(rng.standard_normal((T, H, D)), dtype)
        dev[name] = to_device(bits, dtype)
        host[name] = synth.decode(bits, dtype)
    scale = 1.0 / math.sqrt(D)
    o, lse = sb.fwd_stats_varlen(dev["q"], dev["k"], dev["v"], cu, cu, scale, True)
    torch.cuda.synchronize()
    seqs = [0, 3, 5]
    g = oracle.varlen_backward(host["q"], host["k"], host["v"], host["do"], cu, cu, scale, True, seqs=seqs)
    dq, dk, dv = (torch.full_like(dev[n], float("nan")) for n in ("q", "k", "v"))
    sb.bwd_varlen(dev["q"], dev["k"], dev["v"], o, dev["do"], lse, cu, cu, scale, True, dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    for t in (dq, dk, dv):
        assert not torch.isnan(t).any(), "unwritten gradient elements"
    starts = np.concatenate([[0], cu[:-1]])
    for s in seqs:
        r = slice(int(starts[s]), int(cu[s]))
        f = oracle.varlen_forward(host["q"][r], host["k"][r], host["v"][r], [lengths[s]], [lengths[s]], scale, True)
        assert np.max(np.abs(to_f64(lse[r]) - f["lse"])) <= STATS_ABS_TOL
        for name, got, ref in (("dq", dq, g["dq"]), ("dk", dk, g["dk"]), ("dv", dv, g["dv"])):
            assert_rel(to_f64(got[r]), ref[r], dtype, f"{name} seq {s}")
