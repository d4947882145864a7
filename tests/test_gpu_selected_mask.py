"""GPU parity of selected attention with a user attention mask (the Ascend
page's attenMaskOptional: a 2-D bool/uint8 mask over sequence-local (query,
key) positions, nonzero = masked out, shared by sequences and heads, on top of
sparse_mode) against the fp64 oracle.

* Forward (sdpa_fwd_selected): O within the backward's relative bars, the
  statistics as in the unmasked forward test (max within 1e-4, ln sum within
  1e-4; a token whose gathered keys are all masked: O = 0, max = -inf, sum = 0).
* Backward (sdpa_bwd_selected): dQ, dK, dV within max|err|/max|ref| <= 5e-3
  (fp16) / 2e-2 (bf16), on the oracle's masked statistics and on the GPU
  forward's.
The mask rows are padded (row stride above the key length) and some tokens
lose every gathered key."""
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


def _mask(sq, sk, seed, p, as_bool):
    """(host bool mask [sq, sk], device mask with padded rows)."""
    rng = np.random.default_rng(seed)
    m = rng.random((sq, sk)) < p
    m[3, :] = True                      # token 3 of every sequence sees nothing
    stride = (sk + 15) // 16 * 16 + 32
    buf = np.zeros((sq, stride), dtype=np.uint8)
    buf[:, :sk] = m
    buf[:, sk:] = 1                     # padding past the keys is never read as a key
    dev = torch.from_numpy(buf).cuda()[:, :]
    if as_bool:
        dev = dev.bool()
    return m, dev


def _stats_ok(m_got, l_got, f):
    dead = ~np.isfinite(f["m"])
    assert dead.any(), "the case should have rows without keys"
    assert np.array_equal(np.isneginf(m_got), dead)
    assert np.all(l_got[dead] == 0.0) and np.all(l_got[~dead] > 0.0)
    live = ~dead
    assert float(np.max(np.abs(m_got[live] - f["m"][live]))) <= STATS_ABS_TOL
    assert float(np.max(np.abs(np.log(l_got[live]) - np.log(f["l"][live])))) <= STATS_ABS_TOL


@pytest.mark.parametrize("dtype,D,Dv", [("f16", 64, 64), ("bf16", 128, 128), ("bf16", 192, 128)])
@pytest.mark.parametrize("mode", [0, 2])
@pytest.mark.parametrize("lengths,G,N2,bs,count,p", [
    ((256, 128), 2, 2, 64, 2, 0.3),
    ((96, 160, 80), 4, 1, 16, 5, 0.5),
    ((384, 192), 16, 1, 64, 3, 0.2),
    ((96, 192), 2, 1, 48, 2, 0.4),     # 48-key blocks: halves shorter than 64 keys
    ((512,), 1, 1, 128, 3, 0.9),       # mostly masked
])
def test_selected_with_mask(dtype, D, Dv, mode, lengths, G, N2, bs, count, p):
    rng = np.random.default_rng(len(lengths) * 100 + G * 10 + bs + D + mode)
    lengths = np.array(lengths)
    cu = np.cumsum(lengths)
    T, L = int(cu[-1]), int(lengths.max())
    topk = synth.draw_topk(lengths, N2, bs, count, config_id=41)
    if mode == 0:
        starts = np.concatenate([[0], cu[:-1]])
        for s0, s1 in zip(starts, cu):
            topk[s0:s1] = rng.integers(0, (s1 - s0) // bs, size=topk[s0:s1].shape)
    Hq = G * N2
    bits = {n: synth.encode(rng.standard_normal(shape), dtype)
            for n, shape in (("q", (T, Hq, D)), ("k", (T, N2, D)), ("v", (T, N2, Dv)), ("do", (T, Hq, Dv)))}
    x = {n: synth.decode(b, dtype) for n, b in bits.items()}
    t = {n: to_device(b, dtype) for n, b in bits.items()}
    scale = 1 / math.sqrt(D)
    mask, mdev = _mask(L, L, seed=T + bs, p=p, as_bool=(dtype == "bf16"))
    print(f"mask case {dtype} D={D} Dv={Dv} mode={mode} lengths={tuple(lengths)} G={G} bs={bs}", flush=True)
    f = oracle.selected_forward(x["q"], x["k"], x["v"], topk, cu, cu, bs, scale, mode, atten_mask=mask)
    g = oracle.selected_backward(x["q"], x["k"], x["v"], x["do"], topk, cu, cu, bs, scale, mode, atten_mask=mask)
    tk = _topk_dev(topk)
    # forward
    o = torch.full_like(t["do"], float("nan"))
    m = torch.full((T, Hq), float("nan"), dtype=torch.float32, device="cuda")
    l = torch.full_like(m, float("nan"))
    sb.fwd_selected(t["q"], t["k"], t["v"], tk, cu, cu, bs, scale, mode, o=o, m=m, l=l, atten_mask=mdev)
    torch.cuda.synchronize()
    assert_rel(to_f64(o), f["O"], dtype, "masked O")
    _stats_ok(to_f64(m), to_f64(l), f)
    # backward on the oracle's statistics, then on the GPU forward's
    o_ref = to_device(synth.encode(f["O"], dtype), dtype)
    st_ref = (torch.tensor(f["m"], dtype=torch.float32, device="cuda"),
              torch.tensor(f["l"], dtype=torch.float32, device="cuda"))
    for label, oo, st in (("oracle stats", o_ref, st_ref), ("GPU forward", o, (m, l))):
        dq = torch.full_like(t["q"], float("nan"))
        dk = torch.full_like(t["k"], float("nan"))
        dv = torch.full_like(t["v"], float("nan"))
        sb.bwd_selected(t["q"], t["k"], t["v"], oo, t["do"], st, tk, cu, cu, bs, scale, mode,
                        dq=dq, dk=dk, dv=dv, atten_mask=mdev)
        torch.cuda.synchronize()
        for name, got, ref in (("dq", dq, g["dq"]), ("dk", dk, g["dk"]), ("dv", dv, g["dv"])):
            assert_rel(to_f64(got), ref, dtype, f"masked {name} ({label})")


def test_all_false_mask_is_bitwise_no_mask():
    """An all-zero mask takes the masked code path and must give the same bits
    as no mask at the NSA workload's grouping."""
    rng = np.random.default_rng(77)
    lengths = np.array([1024])
    cu = np.cumsum(lengths)
    T, G, D, bs, count, dtype = 1024, 16, 128, 64, 8, "bf16"
    topk = synth.draw_topk(lengths, 1, bs, count, config_id=5)
    bits = {n: synth.encode(rng.standard_normal(shape), dtype)
            for n, shape in (("q", (T, G, D)), ("k", (T, 1, D)), ("v", (T, 1, D)), ("do", (T, G, D)))}
    t = {n: to_device(b, dtype) for n, b in bits.items()}
    tk = _topk_dev(topk)
    scale = 1 / math.sqrt(D)
    zero = torch.zeros((T, T), dtype=torch.uint8, device="cuda")
    outs = []
    for mk in (None, zero):
        o, m, l = sb.fwd_selected(t["q"], t["k"], t["v"], tk, cu, cu, bs, scale, 2, atten_mask=mk)
        grads = sb.bwd_selected(t["q"], t["k"], t["v"], o, t["do"], (m, l), tk, cu, cu, bs, scale, 2,
                                atten_mask=mk)
        torch.cuda.synchronize()
        outs.append((o, m, l) + tuple(grads))
    for a, b in zip(*outs):
        assert torch.equal(a.view(torch.int16) if a.dtype != torch.float32 else a,
                           b.view(torch.int16) if b.dtype != torch.float32 else b)
