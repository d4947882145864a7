"""GPU parity of the NSA selected-attention forward (sdpa_fwd_selected) against
the fp64 oracle's literal gather: O within the backward's relative bars; the
row max within 1e-4 absolute and the row sum within 1e-4 in the log domain
(|ln sum_gpu - ln sum_ref|; 1e-4 absolute is below fp32 resolution for sums of
hundreds); a token with no admissible key must give O = 0, max = -inf, sum = 0.
Outputs are pre-filled with NaN.  The selected backward then runs on the
GPU-made O and statistics and is checked against the oracle's gradients."""
import math

import numpy as np
import pytest
import torch

import oracle
import sdpa_backward_fa2_amd as sb
import synth
from gpu_util import STATS_ABS_TOL, assert_rel, to_device, to_f64

pytestmark = pytest.mark.gpu


def _topk_dev(topk):
    return torch.from_numpy(np.ascontiguousarray(topk, dtype=np.int32)).cuda()


def _check_stats(m_got, l_got, f, what):
    m_ref, l_ref = f["m"], f["l"]
    dead = ~np.isfinite(m_ref)
    assert np.array_equal(np.isneginf(m_got), dead), f"{what}: rows without keys differ"
    assert np.all(l_got[dead] == 0.0) and np.all(l_got[~dead] > 0.0), f"{what}: sums"
    live = ~dead
    if live.any():
        em = float(np.max(np.abs(m_got[live] - m_ref[live])))
        el = float(np.max(np.abs(np.log(l_got[live]) - np.log(l_ref[live]))))
        assert em <= STATS_ABS_TOL, f"{what}: max|max err| = {em:.3e}"
        assert el <= STATS_ABS_TOL, f"{what}: max|ln sum err| = {el:.3e}"


def _run_forward(t, topk_dev, cu, bs, scale, mode):
    o = torch.full_like(t["do"], float("nan"))      # O has the value head dim
    m = torch.full(t["q"].shape[:2], float("nan"), dtype=torch.float32, device="cuda")
    l = torch.full_like(m, float("nan"))
    sb.fwd_selected(t["q"], t["k"], t["v"], topk_dev, cu, cu, bs, scale, mode, o=o, m=m, l=l)
    torch.cuda.synchronize()
    return o, m, l


def _case(x, t, topk, cu, bs, scale, mode, dtype, backward=True):
    o, m, l = _run_forward(t, _topk_dev(topk), cu, bs, scale, mode)
    f = oracle.selected_forward(x["q"], x["k"], x["v"], topk, cu, cu, bs, scale, mode)
    assert_rel(to_f64(o), f["O"], dtype, "O")
    _check_stats(to_f64(m), to_f64(l), f, "stats")
    if not backward:
        return
    g = oracle.selected_backward(x["q"], x["k"], x["v"], x["do"], topk, cu, cu, bs, scale, mode)
    dq, dk, dv = sb.bwd_selected(t["q"], t["k"], t["v"], o, t["do"], (m, l), _topk_dev(topk), cu, cu,
                                 bs, scale, mode)
    torch.cuda.synchronize()
    for name, got, ref in (("dq", dq, g["dq"]), ("dk", dk, g["dk"]), ("dv", dv, g["dv"])):
        assert_rel(to_f64(got), ref, dtype, f"{name} from the GPU forward")


def _random_inputs(T, Hq, N2, D, dtype, rng, Dv=None):
    Dv = D if Dv is None else Dv
    bits = {n: synth.encode(rng.standard_normal(shape), dtype)
            for n, shape in (("q", (T, Hq, D)), ("k", (T, N2, D)), ("v", (T, N2, Dv)), ("do", (T, Hq, Dv)))}
    return ({n: synth.decode(b, dtype) for n, b in bits.items()},
            {n: to_device(b, dtype) for n, b in bits.items()})


def test_config5_forward():
    """T=4096, 16 query heads on 1 KV head, D=128 bf16, 16 blocks of 64 keys per
    token, causal within the selected keys: forward compared in full, then the
    backward on its output."""
    wl = synth.workload(5)
    cu = wl.cu_seqlens()
    bits = {n: wl.packed_bits(tid, H) for n, tid, H in (("q", 0, wl.Hq), ("k", 1, wl.Hkv),
                                                        ("v", 2, wl.Hkv), ("do", 3, wl.Hq))}
    x = {n: synth.decode(b, wl.dtype) for n, b in bits.items()}
    t = {n: to_device(b, wl.dtype) for n, b in bits.items()}
    _case(x, t, wl.topk(), cu, wl.block_size, wl.scale, 2, wl.dtype)


@pytest.mark.parametrize("dtype,D,Dv", [("f16", 64, 64), ("bf16", 128, 128), ("bf16", 192, 128), ("f16", 192, 192)])
@pytest.mark.parametrize("mode", [0, 2])
@pytest.mark.parametrize("lengths,G,N2,bs,count", [
    ((256, 128), 2, 2, 64, 2),
    ((96, 160, 80), 4, 1, 16, 5),
    ((384, 192), 16, 1, 64, 3),
    ((96, 192), 20, 1, 48, 2),     # 20 heads: two 16-head tiles, the second partly empty
])
def test_forward_small(dtype, D, Dv, mode, lengths, G, N2, bs, count):
    rng = np.random.default_rng(len(lengths) * 100 + G * 10 + bs + D + mode + 7)
    lengths = np.array(lengths)
    cu = np.cumsum(lengths)
    T = int(cu[-1])
    topk = synth.draw_topk(lengths, N2, bs, count, config_id=41)
    if mode == 0:
        starts = np.concatenate([[0], cu[:-1]])
        for s0, s1 in zip(starts, cu):
            topk[s0:s1] = rng.integers(0, (s1 - s0) // bs, size=topk[s0:s1].shape)
    x, t = _random_inputs(T, G * N2, N2, D, dtype, rng, Dv)
    _case(x, t, topk, cu, bs, 1 / math.sqrt(D), mode, dtype)


def test_token_without_admissible_key():
    """Causal selection whose first tokens only name a later block: those
    tokens see no key (O = 0, max = -inf, sum = 0)."""
    rng = np.random.default_rng(43)
    lengths = np.array([128])
    cu = np.cumsum(lengths)
    bs, count, D = 32, 2, 64
    topk = synth.draw_topk(lengths, 1, bs, count, config_id=43)
    topk[:3, 0, :] = 2          # tokens 0..2 name block 2 (keys 64..95) only
    x, t = _random_inputs(128, 2, 1, D, "f16", rng)
    _case(x, t, topk, cu, bs, 1 / math.sqrt(D), 2, "f16", backward=False)
