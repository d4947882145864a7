"""GPU test of the allocation-free dense backward (sdpa_bwd_noalloc).

It runs the same kernels as sdpa_bwd with the library's fixed per-GPU scratch
array in place of a caller workspace.  Two calls in a row, the second on a
smaller problem (so the array is reused with stale contents from the first):
each is compared with sdpa_bwd on the same inputs (bitwise in the
atomic-free dQ modes, which are deterministic; within the parity bound in the
fp32-atomic mode) and with the fp64 oracle (max|err|/max|ref| <= 5e-3 fp16,
2e-2 bf16)."""
import math

import numpy as np
import pytest
import torch

import oracle
import sdpa_backward_fa2_amd as sb
import synth
from gpu_util import REL_TOL, assert_rel, to_device, to_f64

pytestmark = pytest.mark.gpu


def _case(B, H, S, D, dtype, causal, seed):
    rng = np.random.default_rng(seed)
    ts, xs = {}, {}
    for name in ("q", "k", "v", "do"):
        bits = synth.encode(rng.standard_normal((B, S, H, D)), dtype)      # BSHD physical
        ts[name] = to_device(bits, dtype).permute(0, 2, 1, 3)
        xs[name] = synth.decode(bits, dtype).transpose(0, 2, 1, 3)
    scale = 1.0 / math.sqrt(D)
    o, lse = sb.fwd_stats(ts["q"], ts["k"], ts["v"], scale, causal)
    torch.cuda.synchronize()
    return ts, xs, o, lse, scale


def _nan(t):
    return torch.empty_strided(t.shape, t.stride(), dtype=t.dtype, device=t.device).fill_(float("nan"))


def _both(ts, o, lse, scale, causal, mode):
    q, k, v, do = ts["q"], ts["k"], ts["v"], ts["do"]
    ref = sb.bwd(q, k, v, o, do, lse, scale, causal, deterministic=mode,
                 dq=_nan(q), dk=_nan(k), dv=_nan(v))
    got = sb.bwd_noalloc(q, k, v, o, do, lse, scale, causal, deterministic=mode,
                         dq=_nan(q), dk=_nan(k), dv=_nan(v))
    torch.cuda.synchronize()
    return got, ref


@pytest.mark.parametrize("mode", [0, 2])
def test_noalloc_two_calls_second_smaller(mode):
    cases = [(2, 6, 1024, 64, "f16", True, 11),     # 12288 rows (mode 2: 3.2 MB of scratch)
             (1, 3, 333, 128, "bf16", False, 12)]   # smaller, ragged, other head dim
    for B, H, S, D, dtype, causal, seed in cases:
        print(f"noalloc mode={mode} B={B} H={H} S={S} D={D} {dtype} causal={causal}", flush=True)
        ts, xs, o, lse, scale = _case(B, H, S, D, dtype, causal, seed)
        got, ref = _both(ts, o, lse, scale, causal, mode)
        g = oracle.dense_backward(xs["q"], xs["k"], xs["v"], xs["do"], scale, causal)
        for name, a, r, x in zip(("dq", "dk", "dv"), got, ref, (g["dq"], g["dk"], g["dv"])):
            if mode == 2:       # fp32 atomics: rounding order may differ run to run
                e = float((a.float() - r.float()).abs().max() / r.float().abs().max())
                assert e <= REL_TOL[dtype], f"{name}: noalloc vs sdpa_bwd {e:.3e}"
            else:
                assert torch.equal(a.view(torch.int16), r.view(torch.int16)), f"{name} differs from sdpa_bwd"
            assert_rel(to_f64(a), x, dtype, f"noalloc {name} mode={mode} S={S}")



@pytest.mark.parametrize("mode", [0, 2])
def test_noalloc_graph_replay(mode):
    """The caller this entry point is for: a HIP graph that captures it.  The
    captured call is replayed three times with eager device work between
    replays; each replay matches the eager call (bitwise in the atomic-free
    mode, within the parity bound with fp32 atomics)."""
    B, H, S, D, dtype, causal = 2, 4, 512, 128, "bf16", True
    print(f"noalloc graph mode={mode} B={B} H={H} S={S} D={D} {dtype}", flush=True)
    ts, _xs, o, lse, scale = _case(B, H, S, D, dtype, causal, 21)
    q, k, v, do = ts["q"], ts["k"], ts["v"], ts["do"]
    eager = sb.bwd_noalloc(q, k, v, o, do, lse, scale, causal, deterministic=mode,
                           dq=_nan(q), dk=_nan(k), dv=_nan(v))
    torch.cuda.synchronize()
    eager = [t.clone() for t in eager]
    outs = (_nan(q), _nan(k), _nan(v))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        sb.bwd_noalloc(q, k, v, o, do, lse, scale, causal, deterministic=mode, dq=outs[0], dk=outs[1], dv=outs[2])
        side.synchronize()
        with torch.cuda.graph(graph, stream=side):
            sb.bwd_noalloc(q, k, v, o, do, lse, scale, causal, deterministic=mode,
                           dq=outs[0], dk=outs[1], dv=outs[2])
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for replay in range(3):
        for t in outs:
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, got, ref in zip(("dq", "dk", "dv"), outs, eager):
            if mode == 0:
                assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), f"replay {replay}: {name}"
            else:
                e = float((got.float() - ref.float()).abs().max() / ref.float().abs().max())
                assert e <= REL_TOL[dtype], f"replay {replay}: {name} {e}"
