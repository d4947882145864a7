"""GPU parity of fp32 gradient outputs (grad_dtype = SDPA_F32; the Ascend
parameter table lists FLOAT32 for dqOut, dkOut and dvOut) on the dense, packed
and selected backward.

Two checks per case: the fp32 gradients against the fp64 oracle within the
bars of the 16-bit path (the error comes from the 16-bit P and dS operands, not
from the output type); and, for the atomic-free dQ modes, rounding the fp32
gradients to the input type (round to nearest even) gives the 16-bit outputs
of the same call bit for bit, since both store the same fp32 values.  Outputs
are pre-filled with NaN."""
import math

import numpy as np
import pytest
import torch

import oracle
import sdpa_backward_fa2_amd as sb
import synth
from gpu_util import TORCH_DTYPE, assert_rel, to_device, to_f64

pytestmark = pytest.mark.gpu


def _nan32(t):
    return torch.empty_strided(t.shape, t.stride(), dtype=torch.float32, device=t.device).fill_(float("nan"))


def _nan16(t):
    return torch.empty_strided(t.shape, t.stride(), dtype=t.dtype, device=t.device).fill_(float("nan"))


def _compare(g32, g16, ref, dtype, exact, what):
    for name, a, b, r in zip(("dq", "dk", "dv"), g32, g16, (ref["dq"], ref["dk"], ref["dv"])):
        assert a.dtype == torch.float32
        assert_rel(to_f64(a), r, dtype, f"{name} fp32 {what}")
        if exact:
            same = a.to(TORCH_DTYPE[dtype]).view(torch.int16) == b.view(torch.int16)
            assert bool(same.all()), f"{name} {what}: {int((~same).sum())} elements differ after rounding"


def _inputs(shapes, dtype, rng):
    bits = {n: synth.encode(rng.standard_normal(s), dtype) for n, s in shapes.items()}
    return ({n: synth.decode(b, dtype) for n, b in bits.items()},
            {n: to_device(b, dtype) for n, b in bits.items()})


@pytest.mark.parametrize("dtype,D", [("f16", 64), ("bf16", 64), ("f16", 128), ("bf16", 128)])
@pytest.mark.parametrize("causal,Sq,Sk", [(True, 200, 200), (False, 77, 150), (True, 150, 77)])
def test_dense(dtype, D, causal, Sq, Sk):
    rng = np.random.default_rng(D + Sq + 3 * Sk + causal)
    B, Hq, Hkv = 2, 4, 2
    x, t = _inputs({"q": (B, Hq, Sq, D), "k": (B, Hkv, Sk, D), "v": (B, Hkv, Sk, D),
                    "do": (B, Hq, Sq, D)}, dtype, rng)
    scale = 1 / math.sqrt(D)
    f = oracle.dense_forward(x["q"], x["k"], x["v"], scale, causal)
    g = oracle.dense_backward(x["q"], x["k"], x["v"], x["do"], scale, causal)
    o = to_device(synth.encode(f["O"], dtype), dtype)
    lse = torch.tensor(f["lse"], dtype=torch.float32, device="cuda")
    q, k, v, do = t["q"], t["k"], t["v"], t["do"]
    for det in (0, 1, 2):
        g32 = (_nan32(q), _nan32(k), _nan32(v))
        g16 = (_nan16(q), _nan16(k), _nan16(v))
        sb.bwd(q, k, v, o, do, lse, scale, causal, deterministic=det, dq=g32[0], dk=g32[1], dv=g32[2])
        sb.bwd(q, k, v, o, do, lse, scale, causal, deterministic=det, dq=g16[0], dk=g16[1], dv=g16[2])
        torch.cuda.synchronize()
        exact = det != 2 or D == 64     # D=64 has no atomic kernel
        _compare(g32, g16, g, dtype, exact, f"det={det}")


def test_dense_allocates_fp32_when_asked():
    rng = np.random.default_rng(5)
    x, t = _inputs({n: (1, 2, 96, 64) for n in ("q", "k", "v", "do")}, "f16", rng)
    f = oracle.dense_forward(x["q"], x["k"], x["v"], 0.125, True)
    o = to_device(synth.encode(f["O"], "f16"), "f16")
    lse = torch.tensor(f["lse"], dtype=torch.float32, device="cuda")
    dq, dk, dv = sb.bwd(t["q"], t["k"], t["v"], o, t["do"], lse, 0.125, True, grad_dtype=torch.float32)
    torch.cuda.synchronize()
    g = oracle.dense_backward(x["q"], x["k"], x["v"], x["do"], 0.125, True)
    for name, a in (("dq", dq), ("dk", dk), ("dv", dv)):
        assert a.dtype == torch.float32
        assert_rel(to_f64(a), g[name], "f16", name)


@pytest.mark.parametrize("D", [64, 128])
def test_packed(D):
    rng = np.random.default_rng(40 + D)
    lq, lk = [1, 200, 0, 129, 64], [1, 150, 30, 129, 300]
    cu_q, cu_k = np.cumsum(lq), np.cumsum(lk)
    Tq, Tk = int(cu_q[-1]), int(cu_k[-1])
    dtype = "bf16"
    x, t = _inputs({"q": (Tq, 2, D), "k": (Tk, 2, D), "v": (Tk, 2, D), "do": (Tq, 2, D)}, dtype, rng)
    scale = 1 / math.sqrt(D)
    f = oracle.varlen_forward(x["q"], x["k"], x["v"], cu_q, cu_k, scale, True)
    g = oracle.varlen_backward(x["q"], x["k"], x["v"], x["do"], cu_q, cu_k, scale, True)
    o = to_device(synth.encode(f["O"], dtype), dtype)
    stats = (torch.tensor(f["m"], dtype=torch.float32, device="cuda"),
             torch.tensor(f["l"], dtype=torch.float32, device="cuda"))
    q, k, v, do = t["q"], t["k"], t["v"], t["do"]
    for det in (0, 2):
        g32 = (_nan32(q), _nan32(k), _nan32(v))
        g16 = (_nan16(q), _nan16(k), _nan16(v))
        for outs in (g32, g16):
            sb.bwd_varlen(q, k, v, o, do, stats, cu_q, cu_k, scale, True, deterministic=det,
                          dq=outs[0], dk=outs[1], dv=outs[2])
        torch.cuda.synchronize()
        _compare(g32, g16, g, dtype, det == 0 or D == 64, f"det={det}")


@pytest.mark.parametrize("dtype,D,Dv", [("f16", 64, 64), ("bf16", 128, 128), ("bf16", 192, 128), ("bf16", 192, 192)])
@pytest.mark.parametrize("lengths,G,bs,count", [((256, 128), 2, 64, 2), ((96, 160, 80), 16, 16, 5)])
def test_selected(dtype, D, Dv, lengths, G, bs, count):
    """One-piece blocks (written by the dK/dV kernel) and split blocks (summed
    by the reduction) both store through the fp32 path."""
    rng = np.random.default_rng(G + bs + D)
    lengths = np.array(lengths)
    cu = np.cumsum(lengths)
    T = int(cu[-1])
    topk = synth.draw_topk(lengths, 1, bs, count, config_id=44)
    x, t = _inputs({"q": (T, G, D), "k": (T, 1, D), "v": (T, 1, Dv), "do": (T, G, Dv)}, dtype, rng)
    scale = 1 / math.sqrt(D)
    f = oracle.selected_forward(x["q"], x["k"], x["v"], topk, cu, cu, bs, scale, 2)
    g = oracle.selected_backward(x["q"], x["k"], x["v"], x["do"], topk, cu, cu, bs, scale, 2)
    o = to_device(synth.encode(f["O"], dtype), dtype)
    stats = (torch.tensor(f["m"], dtype=torch.float32, device="cuda"),
             torch.tensor(f["l"], dtype=torch.float32, device="cuda"))
    topk_dev = torch.from_numpy(np.ascontiguousarray(topk, dtype=np.int32)).cuda()
    q, k, v, do = t["q"], t["k"], t["v"], t["do"]
    g32 = (_nan32(q), _nan32(k), _nan32(v))
    g16 = (_nan16(q), _nan16(k), _nan16(v))
    for outs in (g32, g16):
        sb.bwd_selected(q, k, v, o, do, stats, topk_dev, cu, cu, bs, scale, 2,
                        dq=outs[0], dk=outs[1], dv=outs[2])
    torch.cuda.synchronize()
    _compare(g32, g16, g, dtype, True, "selected")
