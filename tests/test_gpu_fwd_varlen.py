"""GPU parity of the packed forward (sdpa_fwd_stats_varlen) against the fp64
oracle: O within the backward's relative bars, the natural-log LSE within 1e-4
absolute (-inf exactly where a query sees no key).  Outputs are pre-filled with
NaN, so a row the kernel does not write fails.  Then the packed backward runs on
the GPU-made O and LSE and is checked against the oracle's gradients."""
import math

import numpy as np
import pytest
import torch

import oracle
import sdpa_backward_fa2_amd as sb
import synth
from gpu_util import STATS_ABS_TOL, assert_rel, to_device, to_f64

pytestmark = pytest.mark.gpu


def _packed(T, H, D, dtype, rng):
    bits = synth.encode(rng.standard_normal((T, H, D)), dtype)
    return to_device(bits, dtype), synth.decode(bits, dtype)


def _check_lse(got, ref, what):
    dead = np.isneginf(ref)
    assert np.array_equal(np.isneginf(got), dead), f"{what}: -inf rows differ"
    live = ~dead
    if live.any():
        e = float(np.max(np.abs(got[live] - ref[live])))
        assert e <= STATS_ABS_TOL, f"{what}: max|LSE err| = {e:.3e}"


def _fwd_case(lq, lk, Hq, Hkv, D, dtype, causal, seed, backward=True, Dv=None):
    rng = np.random.default_rng(seed)
    Dv = D if Dv is None else Dv
    cu_q, cu_k = np.cumsum(lq), np.cumsum(lk)
    Tq, Tk = int(cu_q[-1]), int(cu_k[-1])
    q, qx = _packed(Tq, Hq, D, dtype, rng)
    k, kx = _packed(Tk, Hkv, D, dtype, rng)
    v, vx = _packed(Tk, Hkv, Dv, dtype, rng)
    scale = 1 / math.sqrt(D)
    o = torch.full((Tq, Hq, Dv), float("nan"), dtype=q.dtype, device="cuda")
    lse = torch.full((Tq, Hq), float("nan"), dtype=torch.float32, device="cuda")
    sb.fwd_stats_varlen(q, k, v, cu_q, cu_k, scale, causal, o=o, lse=lse)
    torch.cuda.synchronize()
    f = oracle.varlen_forward(qx, kx, vx, cu_q, cu_k, scale, causal)
    assert_rel(to_f64(o), f["O"], dtype, "O")
    _check_lse(to_f64(lse), f["lse"], "LSE")
    if not backward:
        return
    do, dox = _packed(Tq, Hq, Dv, dtype, rng)
    g = oracle.varlen_backward(qx, kx, vx, dox, cu_q, cu_k, scale, causal)
    dq, dk, dv = sb.bwd_varlen(q, k, v, o, do, lse, cu_q, cu_k, scale, causal)
    torch.cuda.synchronize()
    for name, got, ref in (("dq", dq, g["dq"]), ("dk", dk, g["dk"]), ("dv", dv, g["dv"])):
        assert_rel(to_f64(got), ref, dtype, f"{name} from the GPU forward")


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("D", [64, 128, 192])
def test_ragged_causal(dtype, D):
    lengths = [1, 200, 0, 129, 64, 300]
    _fwd_case(lengths, lengths, 2, 2, D, dtype, True, seed=20 + D)


def test_noncausal_unequal_and_empty_key_sequence():
    # the second sequence has queries but no keys: O = 0, LSE = -inf
    _fwd_case([100, 7, 250], [37, 0, 129], 3, 3, 64, "f16", False, seed=21, backward=False)


@pytest.mark.parametrize("D", [64, 128, 192])
def test_causal_unequal_lengths(D):
    # top-left causal per sequence; the third sequence has no keys
    _fwd_case([100, 7, 64, 250], [37, 300, 0, 129], 2, 2, D, "f16", True, seed=25 + D)


@pytest.mark.parametrize("Hq,Hkv", [(4, 2), (16, 1)])
def test_gqa(Hq, Hkv):
    _fwd_case([130, 257], [130, 257], Hq, Hkv, 128, "bf16", True, seed=22 + Hq)


def test_more_sequences_than_one_launch_holds():
    """70 short sequences: the host splits the launches in chunks of 64."""
    rng = np.random.default_rng(23)
    lengths = [int(x) for x in rng.integers(0, 40, size=70)]
    lengths[0] = 33
    _fwd_case(lengths, lengths, 2, 2, 64, "bf16", True, seed=24)


def test_config4_packed_forward_matches_per_sequence_dense():
    """The packed-batch workload (8 sequences, H=32, D=128 bf16, causal): one
    packed launch gives the same bytes as the dense forward run per sequence."""
    wl = synth.workload(4)
    cu = wl.cu_seqlens()
    q, k, v = (to_device(wl.packed_bits(tid, wl.Hq if tid == synth.TID_Q else wl.Hkv), wl.dtype)
               for tid in (synth.TID_Q, synth.TID_K, synth.TID_V))
    o, lse = sb.fwd_stats_varlen(q, k, v, cu, cu, wl.scale, wl.causal)
    starts = np.concatenate([[0], cu[:-1]])
    v4 = lambda x: x.unsqueeze(0).permute(0, 2, 1, 3)  # noqa: E731  (1, H, L, D) view
    for s0, s1 in zip(starts, cu):
        sl = slice(int(s0), int(s1))
        od = torch.empty_like(q[sl])
        ld = torch.empty((1, wl.Hq, int(s1 - s0)), dtype=torch.float32, device="cuda")
        sb.fwd_stats(v4(q[sl]), v4(k[sl]), v4(v[sl]), wl.scale, wl.causal, o=v4(od), lse=ld)
        torch.cuda.synchronize()
        assert torch.equal(o[sl].view(torch.int16), od.view(torch.int16))
        assert torch.equal(lse[sl].t().contiguous(), ld[0])


@pytest.mark.parametrize("causal", [False, True])
def test_dqk192_dv128(causal):
    """Query/key head dim 192, value head dim 128: O is (T, H, 128)."""
    _fwd_case([1, 200, 0, 129, 64, 300], [1, 200, 5, 129, 64, 300], 4, 2, 192, "bf16", causal, seed=192128,
              Dv=128)
