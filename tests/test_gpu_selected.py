"""GPU parity of the NSA selected-attention path against the fp64 oracle.

* sdpa_selected_build_index: offsets and entries bit-exact against the
  oracle's enumeration (integer work).
* sdpa_bwd_selected: max|err|/max|ref| per tensor against the oracle's literal
  gather (5e-3 fp16, 2e-2 bf16); the workload's statistics and O come from the
  oracle forward, O rounded to the I/O type.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import sdpa_backward_fa2_amd as sb
import synth
from gpu_util import assert_rel, to_device, to_f64

pytestmark = pytest.mark.gpu


def _topk_dev(topk):
    return torch.from_numpy(np.ascontiguousarray(topk, dtype=np.int32)).cuda()


def _check_index(topk, cu_q, cu_kv, bs):
    off_ref, ent_ref = oracle.selected_block_lists(topk, cu_q, cu_kv, bs)
    off, ent = sb.selected_build_index(_topk_dev(topk), cu_q, cu_kv, bs)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(off.cpu().numpy().astype(np.int64), off_ref)
    np.testing.assert_array_equal(ent.cpu().numpy().astype(np.int64), ent_ref)


def test_index_config5_exact():
    wl = synth.workload(5)
    cu = wl.cu_seqlens()
    _check_index(wl.topk(), cu, cu, wl.block_size)


@pytest.mark.parametrize("lengths,N2,bs,count", [((64, 128, 48), 2, 16, 3), ((256, 512), 1, 64, 4),
                                                  ((384,), 3, 128, 2), ((384, 480), 2, 48, 8)])
def test_index_small_exact(lengths, N2, bs, count):
    topk = synth.draw_topk(np.array(lengths), N2, bs, count, config_id=21)
    # scatter some duplicates and a fully repeated row
    topk[5 % topk.shape[0], 0, :] = topk[5 % topk.shape[0], 0, 0]
    cu = np.cumsum(lengths)
    _check_index(topk, cu, cu, bs)


def test_index_many_sequences_exact():
    """70 sequences: more than the 64 the kernel arguments carry, so the
    sequence table goes through the workspace."""
    rng = np.random.default_rng(70)
    lengths = rng.integers(2, 7, size=70) * 32
    topk = synth.draw_topk(lengths, 2, 32, 2, config_id=70)
    cu = np.cumsum(lengths)
    _check_index(topk, cu, cu, 32)


def test_index_long_sequence_exact():
    """T = 32768 with the NSA workload's recipe (16 blocks of 64 keys)."""
    lengths = np.array([32768])
    topk = synth.draw_topk(lengths, 1, 64, 16, config_id=5)
    cu = np.cumsum(lengths)
    _check_index(topk, cu, cu, 64)


def _random_topk(lq, lk, N2, bs, count, seed):
    """Blocks drawn uniformly (repeats allowed) from each token's own sequence."""
    rng = np.random.default_rng(seed)
    rows = [rng.integers(0, k // bs, size=(q, N2, count)) for q, k in zip(lq, lk)]
    return np.concatenate(rows).astype(np.int32)


def test_index_short_and_empty_query_sequences():
    """Query lengths 0 to 33 (several sequences share a 16-token tile of the
    index build) against longer key sequences."""
    lq = np.array([5, 0, 7, 33, 1, 0, 20, 2, 0])
    lk = np.array([64, 96, 64, 128, 64, 64, 96, 64, 64])
    topk = _random_topk(lq, lk, 2, 32, 2, seed=9)
    _check_index(topk, np.cumsum(lq), np.cumsum(lk), 32)


def test_index_many_blocks():
    """4097 key blocks (more than one pass of the rank kernel's block
    counters) and blocks x tiles above 2^22 (the tile doubles to 32 tokens)."""
    lq, lk = np.array([20000]), np.array([4097 * 16])
    topk = _random_topk(lq, lk, 2, 16, 2, seed=4097)
    _check_index(topk, np.cumsum(lq), np.cumsum(lk), 16)


def _run_selected(q, k, v, o, do, stats, topk, cu, bs, scale, mode, det=False):
    dq = torch.full_like(q, float("nan"))
    dk = torch.full_like(k, float("nan"))
    dv = torch.full_like(v, float("nan"))
    sb.bwd_selected(q, k, v, o, do, stats, _topk_dev(topk), cu, cu, bs, scale, mode,
                    deterministic=det, dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    return dq, dk, dv


def test_config5_nsa_selected():
    """T=4096, 16 query heads on 1 KV head, D=128 bf16, 16 blocks of 64 keys per
    token (own block always included, padding with it when fewer exist),
    causal within the selected keys; compared in full."""
    wl = synth.workload(5)
    cu = wl.cu_seqlens()
    topk = wl.topk()
    bits = {n: wl.packed_bits(tid, H) for n, tid, H in (("q", 0, wl.Hq), ("k", 1, wl.Hkv),
                                                        ("v", 2, wl.Hkv), ("do", 3, wl.Hq))}
    x = {n: synth.decode(b, wl.dtype) for n, b in bits.items()}
    t = {n: to_device(b, wl.dtype) for n, b in bits.items()}
    f = oracle.selected_forward(x["q"], x["k"], x["v"], topk, cu, cu, wl.block_size, wl.scale, 2)
    g = oracle.selected_backward(x["q"], x["k"], x["v"], x["do"], topk, cu, cu, wl.block_size, wl.scale, 2)
    o = to_device(synth.encode(f["O"], wl.dtype), wl.dtype)
    stats = (torch.tensor(f["m"], dtype=torch.float32, device="cuda"),
             torch.tensor(f["l"], dtype=torch.float32, device="cuda"))
    runs = []
    for det in (False, True):
        dq, dk, dv = _run_selected(t["q"], t["k"], t["v"], o, t["do"], stats, topk, cu, wl.block_size,
                                   wl.scale, 2, det)
        for name, got, ref in (("dq", dq, g["dq"]), ("dk", dk, g["dk"]), ("dv", dv, g["dv"])):
            assert_rel(to_f64(got), ref, wl.dtype, f"config5 {name} det={det}")
        runs.append((dq, dk, dv))
    # every kernel of this path is deterministic
    for a, b in zip(*runs):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("dtype,D,Dv", [("f16", 64, 64), ("bf16", 128, 128), ("bf16", 192, 128), ("f16", 192, 128),
                                        ("bf16", 192, 192)])
@pytest.mark.parametrize("mode", [0, 2])
@pytest.mark.parametrize("lengths,G,N2,bs,count", [
    ((256, 128), 2, 2, 64, 2),
    ((96, 160, 80), 4, 1, 16, 5),
    ((512,), 1, 1, 128, 3),
    ((384, 192), 16, 1, 64, 3),
    ((96, 192), 2, 1, 48, 2),      # block size that does not divide a 128-key chunk
    # 16 query heads per KV head: at Dqk = Dv = 128 the dQ pass reads the dS
    # the dK/dV kernel stored (two KV heads; 32-key blocks, four to a 128-key
    # chunk; 128-key blocks, two 64-key halves each)
    ((256, 384), 16, 2, 32, 4),
    ((512,), 16, 1, 128, 3),
])
def test_selected_small(dtype, D, Dv, mode, lengths, G, N2, bs, count):
    """D: head dim of Q and K, Dv: of V and dO (192/128: the page's unequal
    head dims)."""
    rng = np.random.default_rng(len(lengths) * 100 + G * 10 + bs + D + mode)
    lengths = np.array(lengths)
    cu = np.cumsum(lengths)
    T = int(cu[-1])
    topk = synth.draw_topk(lengths, N2, bs, count, config_id=31)
    if mode == 0:    # without the causal mask any block of the sequence may be chosen
        starts = np.concatenate([[0], cu[:-1]])
        for s0, s1 in zip(starts, cu):
            nb = (s1 - s0) // bs
            topk[s0:s1] = rng.integers(0, nb, size=topk[s0:s1].shape)
    Hq = G * N2
    bits = {n: synth.encode(rng.standard_normal(shape), dtype)
            for n, shape in (("q", (T, Hq, D)), ("k", (T, N2, D)), ("v", (T, N2, Dv)), ("do", (T, Hq, Dv)))}
    x = {n: synth.decode(b, dtype) for n, b in bits.items()}
    t = {n: to_device(b, dtype) for n, b in bits.items()}
    scale = 1 / math.sqrt(D)
    f = oracle.selected_forward(x["q"], x["k"], x["v"], topk, cu, cu, bs, scale, mode)
    g = oracle.selected_backward(x["q"], x["k"], x["v"], x["do"], topk, cu, cu, bs, scale, mode)
    o = to_device(synth.encode(f["O"], dtype), dtype)
    lse = torch.tensor(f["lse"], dtype=torch.float32, device="cuda")
    dq, dk, dv = _run_selected(t["q"], t["k"], t["v"], o, t["do"], lse, topk, cu, bs, scale, mode)
    for name, got, ref in (("dq", dq, g["dq"]), ("dk", dk, g["dk"]), ("dv", dv, g["dv"])):
        assert_rel(to_f64(got), ref, dtype, name)


def test_unequal_head_dims_long_sequence():
    """Dqk = 192, Dv = 128 bf16 at the NSA workload's head grouping (16 query
    heads per KV head, 16 blocks of 64 keys, causal) on a 2048-token sequence:
    early blocks are chosen by many tokens and split into several pieces, so
    the partial reduction runs with the two widths."""
    rng = np.random.default_rng(192)
    lengths = np.array([2048])
    cu = np.cumsum(lengths)
    T, G, D, Dv, bs, count, dtype = 2048, 16, 192, 128, 64, 16, "bf16"
    topk = synth.draw_topk(lengths, 1, bs, count, config_id=5)
    bits = {n: synth.encode(rng.standard_normal(shape), dtype)
            for n, shape in (("q", (T, G, D)), ("k", (T, 1, D)), ("v", (T, 1, Dv)), ("do", (T, G, Dv)))}
    x = {n: synth.decode(b, dtype) for n, b in bits.items()}
    t = {n: to_device(b, dtype) for n, b in bits.items()}
    scale = 1 / math.sqrt(D)
    f = oracle.selected_forward(x["q"], x["k"], x["v"], topk, cu, cu, bs, scale, 2)
    g = oracle.selected_backward(x["q"], x["k"], x["v"], x["do"], topk, cu, cu, bs, scale, 2)
    o = to_device(synth.encode(f["O"], dtype), dtype)
    stats = (torch.tensor(f["m"], dtype=torch.float32, device="cuda"),
             torch.tensor(f["l"], dtype=torch.float32, device="cuda"))
    dq, dk, dv = _run_selected(t["q"], t["k"], t["v"], o, t["do"], stats, topk, cu, bs, scale, 2)
    for name, got, ref in (("dq", dq, g["dq"]), ("dk", dk, g["dk"]), ("dv", dv, g["dv"])):
        assert_rel(to_f64(got), ref, dtype, name)


@pytest.mark.parametrize("mode", [0, 2])
@pytest.mark.parametrize("G,D,dtype", [(2, 64, "f16"), (16, 128, "bf16")])
def test_many_sequences(mode, G, D, dtype):
    """70 packed sequences (lengths 32..192, some below block_count blocks of
    keys) through the forward and the backward: more sequences than the kernel
    arguments hold (at 16 heads per KV head and D=128 with the stored-dS dQ
    pass)."""
    rng = np.random.default_rng(700 + mode)
    lengths = rng.integers(2, 7, size=70) * 32
    cu = np.cumsum(lengths)
    T, N2, bs, count = int(cu[-1]), 1, 32, 2
    topk = synth.draw_topk(lengths, N2, bs, count, config_id=71)
    if mode == 0:
        starts = np.concatenate([[0], cu[:-1]])
        for s0, s1 in zip(starts, cu):
            topk[s0:s1] = rng.integers(0, (s1 - s0) // bs, size=topk[s0:s1].shape)
    bits = {n: synth.encode(rng.standard_normal(shape), dtype)
            for n, shape in (("q", (T, G, D)), ("k", (T, N2, D)), ("v", (T, N2, D)), ("do", (T, G, D)))}
    x = {n: synth.decode(b, dtype) for n, b in bits.items()}
    t = {n: to_device(b, dtype) for n, b in bits.items()}
    scale = 1 / math.sqrt(D)
    f = oracle.selected_forward(x["q"], x["k"], x["v"], topk, cu, cu, bs, scale, mode)
    g = oracle.selected_backward(x["q"], x["k"], x["v"], x["do"], topk, cu, cu, bs, scale, mode)
    o, m, l = sb.fwd_selected(t["q"], t["k"], t["v"], _topk_dev(topk), cu, cu, bs, scale, mode)
    torch.cuda.synchronize()
    assert_rel(to_f64(o), f["O"], dtype, "O, 70 sequences")
    assert float(np.max(np.abs(to_f64(m) - f["m"]))) <= 1e-4
    o_ref = to_device(synth.encode(f["O"], dtype), dtype)
    stats = (torch.tensor(f["m"], dtype=torch.float32, device="cuda"),
             torch.tensor(f["l"], dtype=torch.float32, device="cuda"))
    dq, dk, dv = _run_selected(t["q"], t["k"], t["v"], o_ref, t["do"], stats, topk, cu, bs, scale, mode)
    for name, got, ref in (("dq", dq, g["dq"]), ("dk", dk, g["dk"]), ("dv", dv, g["dv"])):
        assert_rel(to_f64(got), ref, dtype, f"{name}, 70 sequences")


def test_checked_mode_rejects_out_of_range_topk(monkeypatch):
    """SDPA_BWD_CHECK=1: a top-k value outside the token's sequence's blocks
    is an SDPA_ERR_INVALID error (copied to the host and checked) instead of
    an ignored slot; valid values pass unchanged."""
    rng = np.random.default_rng(5)
    lengths = np.array([256, 128])
    cu = np.cumsum(lengths)
    T, G, bs, count, dtype = int(cu[-1]), 2, 64, 2, "bf16"
    topk = synth.draw_topk(lengths, 1, bs, count, config_id=31)
    bits = {n: synth.encode(rng.standard_normal(shape), dtype)
            for n, shape in (("q", (T, G, 128)), ("k", (T, 1, 128)), ("v", (T, 1, 128)), ("do", (T, G, 128)))}
    t = {n: to_device(b, dtype) for n, b in bits.items()}
    monkeypatch.setenv("SDPA_BWD_CHECK", "1")
    o, m, l = sb.fwd_selected(t["q"], t["k"], t["v"], _topk_dev(topk), cu, cu, bs, 0.1, 2)
    sb.bwd_selected(t["q"], t["k"], t["v"], o, t["do"], (m, l), _topk_dev(topk), cu, cu, bs, 0.1, 2)
    torch.cuda.synchronize()
    bad = topk.copy()
    bad[300, 0, 1] = 2          # token 300 is in the 128-token sequence: blocks 0 and 1 only
    for call in (lambda: sb.fwd_selected(t["q"], t["k"], t["v"], _topk_dev(bad), cu, cu, bs, 0.1, 2),
                 lambda: sb.bwd_selected(t["q"], t["k"], t["v"], o, t["do"], (m, l), _topk_dev(bad), cu, cu, bs,
                                         0.1, 2)):
        with pytest.raises(sb.SdpaError) as e:
            call()
        assert e.value.status == 2    # SDPA_ERR_INVALID
