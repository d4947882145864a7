"""GPU parity of the packed variable-length path (sdpa_bwd_varlen) against the
fp64 oracle.  Bars as for the dense path; outputs pre-filled with NaN."""
import math

import numpy as np
import pytest
import torch

import oracle
import sdpa_backward_fa2_amd as sb
import synth
from gpu_util import assert_rel, to_device, to_f64

pytestmark = pytest.mark.gpu


def _packed(T, H, D, dtype, rng):
    bits = synth.encode(rng.standard_normal((T, H, D)), dtype)
    return to_device(bits, dtype), synth.decode(bits, dtype)


def _nan(t):
    return torch.full_like(t, float("nan"))


def _run(q, k, v, o, do, stats, cu_q, cu_k, scale, causal, det):
    dq, dk, dv = _nan(q), _nan(k), _nan(v)
    sb.bwd_varlen(q, k, v, o, do, stats, cu_q, cu_k, scale, causal, deterministic=det, dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    return dq, dk, dv


def _case(lq, lk, Hq, Hkv, D, dtype, causal, seed, stats_form="max_sum", dets=(0, 1, 2), Dv=None):
    rng = np.random.default_rng(seed)
    Dv = D if Dv is None else Dv
    cu_q, cu_k = np.cumsum(lq), np.cumsum(lk)
    Tq, Tk = int(cu_q[-1]), int(cu_k[-1])
    q, qx = _packed(Tq, Hq, D, dtype, rng)
    k, kx = _packed(Tk, Hkv, D, dtype, rng)
    v, vx = _packed(Tk, Hkv, Dv, dtype, rng)
    do, dox = _packed(Tq, Hq, Dv, dtype, rng)
    scale = 1 / math.sqrt(D)
    f = oracle.varlen_forward(qx, kx, vx, cu_q, cu_k, scale, causal)
    o = to_device(synth.encode(f["O"], dtype), dtype)
    if stats_form == "lse":
        stats = torch.tensor(f["lse"], dtype=torch.float32, device="cuda")
    elif stats_form == "t_n_8":     # the Ascend [T, N, 8] layout, 8 copies per row
        m8 = torch.tensor(np.repeat(f["m"][..., None], 8, axis=2), dtype=torch.float32, device="cuda")
        l8 = torch.tensor(np.repeat(f["l"][..., None], 8, axis=2), dtype=torch.float32, device="cuda")
        stats = (m8, l8)
    else:
        stats = (torch.tensor(f["m"], dtype=torch.float32, device="cuda"),
                 torch.tensor(f["l"], dtype=torch.float32, device="cuda"))
    g = oracle.varlen_backward(qx, kx, vx, dox, cu_q, cu_k, scale, causal)
    for det in dets:
        dq, dk, dv = _run(q, k, v, o, do, stats, cu_q, cu_k, scale, causal, det)
        for name, got, ref in (("dq", dq, g["dq"]), ("dk", dk, g["dk"]), ("dv", dv, g["dv"])):
            assert_rel(to_f64(got), ref, dtype, f"{name} det={det}")


def test_config4_packed_varlen_sampled():
    """8 sequences, lengths U[256, 2048] (seeded), H=32, D=128 bf16, causal per
    sequence, max/sum statistics and O from the oracle forward.  The GPU runs
    the whole pack; the oracle checks every row and key of 2 sequences x 32 heads."""
    wl = synth.workload(4)
    cu = wl.cu_seqlens()
    q_bits = wl.packed_bits(synth.TID_Q, wl.Hq)
    k_bits = wl.packed_bits(synth.TID_K, wl.Hkv)
    v_bits = wl.packed_bits(synth.TID_V, wl.Hkv)
    do_bits = wl.packed_bits(synth.TID_DO, wl.Hq)
    qx, kx, vx, dox = (synth.decode(b, wl.dtype) for b in (q_bits, k_bits, v_bits, do_bits))
    q, k, v, do = (to_device(b, wl.dtype) for b in (q_bits, k_bits, v_bits, do_bits))
    starts = np.concatenate([[0], cu[:-1]])
    longest = int(np.argmax(wl.lengths))
    seqs = sorted({longest, (longest + 3) % len(wl.lengths)})
    # forward statistics and O for the whole pack (max/sum form)
    full = oracle.varlen_forward(qx, kx, vx, cu, cu, wl.scale, wl.causal)
    o_np, m_np, l_np = full["O"], full["m"], full["l"]
    o = to_device(synth.encode(o_np, wl.dtype), wl.dtype)
    m = torch.tensor(m_np, dtype=torch.float32, device="cuda")
    l = torch.tensor(l_np, dtype=torch.float32, device="cuda")
    g = oracle.varlen_backward(qx, kx, vx, dox, cu, cu, wl.scale, wl.causal, seqs=seqs)
    for det in (0, 1, 2):
        dq, dk, dv = _run(q, k, v, o, do, (m, l), cu, cu, wl.scale, wl.causal, det)
        for s in seqs:
            sl = slice(int(starts[s]), int(cu[s]))
            for name, got, ref in (("dq", dq, g["dq"]), ("dk", dk, g["dk"]), ("dv", dv, g["dv"])):
                assert_rel(to_f64(got[sl]), ref[sl], wl.dtype, f"config4 seq {s} {name} det={det}")
        for t in (dq, dk, dv):
            assert not torch.isnan(t).any()


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("D", [64, 128, 192])
def test_ragged_causal(dtype, D):
    lengths = [1, 200, 0, 129, 64, 300]
    _case(lengths, lengths, 2, 2, D, dtype, True, seed=D, dets=(0, 1) if D == 192 else (0, 1, 2))


def test_noncausal_unequal_lengths():
    _case([100, 1, 250], [37, 300, 129], 3, 3, 64, "f16", False, seed=5)


@pytest.mark.parametrize("D", [64, 128, 192])
def test_causal_unequal_lengths(D):
    """Causal per sequence with different query and key lengths (top-left in
    local positions); a sequence without keys gives dQ = 0 and one without
    queries dK = dV = 0."""
    _case([100, 1, 250, 0, 64, 9], [37, 300, 129, 20, 0, 9], 2, 2, D, "bf16", True, seed=30 + D,
          dets=(0, 1) if D == 192 else (0, 1, 2))


def test_zero_length_query_sequence_zeroes_its_keys():
    # a sequence with keys but no queries gets dK = dV = 0
    _case([50, 0, 70], [50, 90, 70], 2, 2, 64, "bf16", False, seed=6)


@pytest.mark.parametrize("D", [64, 128, 192])
@pytest.mark.parametrize("Hq,Hkv", [(4, 2), (16, 1)])
def test_gqa(Hq, Hkv, D):
    _case([130, 257], [130, 257], Hq, Hkv, D, "bf16", True, seed=Hq + D, dets=(0, 1) if D == 192 else (0, 1, 2))


@pytest.mark.parametrize("form", ["lse", "t_n_8"])
def test_stats_forms(form):
    _case([96, 160], [96, 160], 2, 2, 64, "f16", True, seed=9, stats_form=form)


def test_more_sequences_than_one_launch_holds():
    """70 short sequences: the host splits the launches in chunks of 64."""
    rng = np.random.default_rng(12)
    lengths = [int(x) for x in rng.integers(0, 40, size=70)]
    lengths[0] = 33
    _case(lengths, lengths, 2, 2, 64, "f16", True, seed=13)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_dqk192_dv128_ragged_causal(dtype):
    """Query/key head dim 192, value head dim 128, packed."""
    lengths = [1, 200, 0, 129, 64, 300]
    _case(lengths, lengths, 2, 2, 192, dtype, True, seed=321, dets=(0, 1), Dv=128)


def test_dqk192_dv128_unequal_lengths_gqa():
    _case([100, 1, 250, 0, 64], [37, 300, 129, 20, 0], 4, 2, 192, "bf16", True, seed=322, dets=(0, 1), Dv=128)
    _case([130, 257], [90, 300], 4, 1, 192, "f16", False, seed=323, dets=(0, 1), Dv=128)
