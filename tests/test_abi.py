"""C-ABI checks that run without a GPU: the library loads, exports every
function include/sdpa_bwd.h declares, and rejects bad arguments with the
documented status before making any HIP call.  Pointers here are fake aligned
addresses; argument validation never dereferences them."""
import ctypes

import pytest
import torch

import sdpa_backward_fa2_amd as sb

OK, NULLPTR, INVALID, UNSUPPORTED, WORKSPACE, HIP = range(6)
FAKE = 0x10000


def lib():
    return sb.load()


def test_exports_every_declared_symbol():
    names = sb.declared_functions()
    assert len(names) >= 10, names
    L = lib()
    for n in names:
        assert hasattr(L, n), n
    for must in ("sdpa_fwd_stats", "sdpa_bwd", "sdpa_bwd_varlen", "sdpa_bwd_selected",
                 "sdpa_selected_build_index", "sdpa_status_string"):
        assert must in names


def test_status_strings():
    for s in range(6):
        assert lib().sdpa_status_string(s)


def t4(ptr=FAKE, strides=(16384, 8192, 64, 1)):
    return sb.Tensor4(ptr, *strides)


def dense_call(**kw):
    a = dict(dtype=0, B=1, Hq=2, Hkv=2, Sq=128, Sk=128, D=64, Dv=None, scale=0.125, causal=0, det=0, grad=None,
             q=t4(), k=t4(), v=t4(), o=t4(), do=t4(), dq=t4(), dk=t4(), dv=t4(),
             stats=sb.Stats(0, FAKE, None, 256, 128, 1), ws=FAKE, ws_bytes=1 << 30)
    a.update(kw)
    ref = lambda x: ctypes.byref(x) if x is not None else None  # noqa: E731
    grad = a["dtype"] if a["grad"] is None else a["grad"]
    dv = a["D"] if a["Dv"] is None else a["Dv"]
    return lib().sdpa_bwd(a["dtype"], a["B"], a["Hq"], a["Hkv"], a["Sq"], a["Sk"], a["D"], dv, a["scale"],
                          a["causal"], a["det"], grad, ref(a["q"]), ref(a["k"]), ref(a["v"]), ref(a["o"]),
                          ref(a["do"]), ref(a["stats"]), ref(a["dq"]), ref(a["dk"]), ref(a["dv"]),
                          a["ws"], a["ws_bytes"], None)


def test_dense_validation_order():
    assert dense_call(q=None) == NULLPTR
    assert dense_call(dv=t4(ptr=0)) == NULLPTR
    assert dense_call(stats=sb.Stats(1, FAKE, None, 256, 128, 1)) == NULLPTR   # max/sum without sum
    assert dense_call(ws=None) == NULLPTR
    assert dense_call(dtype=7) == INVALID
    assert dense_call(Hq=3, Hkv=2) == INVALID
    assert dense_call(Hkv=0) == INVALID
    assert dense_call(B=-1) == INVALID
    assert dense_call(grad=1) == INVALID          # gradients: the input dtype or fp32
    assert dense_call(grad=3) == INVALID
    assert dense_call(scale=float("nan")) == INVALID
    assert dense_call(det=3) == INVALID          # dQ mode outside 0..2
    assert dense_call(det=-1) == INVALID
    assert dense_call(stats=sb.Stats(5, FAKE, None, 256, 128, 1)) == INVALID
    assert dense_call(D=96) == UNSUPPORTED
    assert dense_call(q=t4(strides=(16384, 8192, 64, 2))) == UNSUPPORTED
    assert dense_call(k=t4(ptr=FAKE + 2)) == UNSUPPORTED
    assert dense_call(v=t4(strides=(16384, 8192, 68, 1))) == UNSUPPORTED
    assert dense_call(q=t4(strides=(16384, 8192, -64, 1))) == UNSUPPORTED     # row stride < 0
    assert dense_call(dq=t4(strides=(1 << 40, 1 << 30, 1 << 23, 1))) == UNSUPPORTED
    assert dense_call(stats=sb.Stats(0, FAKE, None, 256, 128, 1 << 23)) == UNSUPPORTED
    assert dense_call(ws_bytes=16) == WORKSPACE
    # NULL beats INVALID beats UNSUPPORTED beats WORKSPACE
    assert dense_call(q=None, dtype=7) == NULLPTR
    assert dense_call(dtype=7, D=96) == INVALID
    assert dense_call(D=96, ws_bytes=16) == UNSUPPORTED


@pytest.mark.skipif(torch.cuda.device_count() > 0, reason="would launch on fake pointers")
def test_valid_call_without_device_reports_hip_error():
    assert dense_call() == HIP
    assert lib().sdpa_last_error()
    assert dense_call(causal=1, Sk=64) == HIP     # causal with Sq != Sk (top-left) is valid
    assert dense_call(grad=2) == HIP              # fp32 gradients


def test_workspace_size_query():
    rows = 4 * 12 * 1024

    def size(D, mode):
        n = ctypes.c_size_t(0)
        assert lib().sdpa_bwd_workspace_size(0, 4, 12, 12, 1024, 1024, D, D, mode, ctypes.byref(n)) == OK
        return n.value
    # atomic-free modes: LSE and Delta rows; the atomic mode adds the fp32 dQ
    # accumulator
    for D in (64, 128):
        assert size(D, 0) == size(D, 1) >= rows * 8
        assert size(D, 2) >= size(D, 1) + rows * D * 4
    # D=192: the atomic-free modes only
    assert size(192, 0) == size(192, 1) >= rows * 8
    m = ctypes.c_size_t(0)
    assert lib().sdpa_bwd_workspace_size(0, 4, 12, 12, 1024, 1024, 192, 192, 2, ctypes.byref(m)) == UNSUPPORTED
    assert lib().sdpa_bwd_workspace_size(0, 4, 12, 12, 1024, 1024, 256, 256, 0, ctypes.byref(m)) == UNSUPPORTED
    assert lib().sdpa_bwd_workspace_size(0, 4, 12, 12, 1024, 1024, 64, 64, 3, ctypes.byref(m)) == INVALID
    assert lib().sdpa_bwd_workspace_size(0, 4, 12, 12, 1024, 1024, 80, 80, 0, ctypes.byref(m)) == UNSUPPORTED
    assert lib().sdpa_bwd_workspace_size(0, 4, 12, 12, 1024, 1024, 64, 64, 0, None) == NULLPTR


def noalloc_call(**kw):
    a = dict(dtype=0, B=1, Hq=2, Hkv=2, Sq=128, Sk=128, D=64, scale=0.125, causal=0, det=0,
             stats=sb.Stats(0, FAKE, None, 256, 128, 1))
    a.update(kw)
    ts = [t4() for _ in range(8)]
    return lib().sdpa_bwd_noalloc(a["dtype"], a["B"], a["Hq"], a["Hkv"], a["Sq"], a["Sk"], a["D"], a["D"],
                                  a["scale"],
                                  a["causal"], a["det"], a["dtype"], *[ctypes.byref(t) for t in ts[:5]],
                                  ctypes.byref(a["stats"]), *[ctypes.byref(t) for t in ts[5:]], None)


def test_noalloc_validation():
    """sdpa_bwd_noalloc validates like sdpa_bwd and refuses, before any HIP
    call, a problem whose scratch exceeds its fixed 16 MiB."""
    assert noalloc_call(stats=sb.Stats(1, FAKE, None, 256, 128, 1)) == NULLPTR
    assert noalloc_call(dtype=7) == INVALID
    assert noalloc_call(D=96) == UNSUPPORTED
    rows_limit = (16 << 20) // 8
    assert noalloc_call(Hq=64, Hkv=64, Sq=rows_limit // 64 + 64) == WORKSPACE    # 8 B per row, modes 0/1
    assert b"16777216" in lib().sdpa_last_error()
    assert noalloc_call(Hq=16, Hkv=16, Sq=4096, det=2) == WORKSPACE                # + 4*D B per row, mode 2
    n = ctypes.c_size_t(0)
    assert lib().sdpa_bwd_workspace_size(0, 1, 16, 16, 4096, 4096, 64, 64, 2, ctypes.byref(n)) == OK
    assert n.value > (16 << 20)


@pytest.mark.skipif(torch.cuda.device_count() > 0, reason="would launch on fake pointers")
def test_noalloc_valid_without_device():
    assert noalloc_call() == HIP
    assert noalloc_call(Hq=12, Hkv=12, Sq=1024, Sk=1024, det=2) == HIP   # 12.6 MB of scratch fits


def t3(ptr=FAKE, strides=(32 * 128, 128, 1)):
    return sb.Tensor3(ptr, *strides)


def varlen_call(cu_q, cu_k, **kw):
    a = dict(dtype=1, Hq=32, Hkv=32, D=128, Dv=None, scale=0.088, causal=1, det=0, grad=1, ws_bytes=1 << 34)
    a.update(kw)
    aq = (ctypes.c_int64 * len(cu_q))(*cu_q)
    ak = (ctypes.c_int64 * len(cu_k))(*cu_k)
    st = sb.Stats(1, FAKE, FAKE, 0, 1, 32)
    ts = [t3() for _ in range(8)]
    dv = a["D"] if a["Dv"] is None else a["Dv"]
    return lib().sdpa_bwd_varlen(a["dtype"], len(cu_q), aq, ak, a["Hq"], a["Hkv"], a["D"], dv, a["scale"],
                                 a["causal"], a["det"], a["grad"], *[ctypes.byref(t) for t in ts[:5]],
                                 ctypes.byref(st), *[ctypes.byref(t) for t in ts[5:]], FAKE,
                                 a["ws_bytes"], None)


def test_varlen_validation():
    assert varlen_call([100, 50], [100, 50]) == INVALID           # non-monotone
    assert varlen_call([100, 300], [100, 300], grad=0) == INVALID  # bf16 inputs, fp16 gradients
    assert varlen_call([100, 300], [100, 300], Hq=3, Hkv=2) == INVALID
    assert varlen_call([100, 300], [100, 300], D=96) == UNSUPPORTED
    assert varlen_call([100, 300], [100, 300], D=192, det=2) == UNSUPPORTED   # no atomic dQ at D=192
    assert varlen_call([100, 300], [100, 300], ws_bytes=8) == WORKSPACE
    n = ctypes.c_size_t(0)
    cu = (ctypes.c_int64 * 2)(100, 300)
    assert lib().sdpa_bwd_varlen_workspace_size(1, 2, cu, cu, 32, 32, 128, 128, 0, ctypes.byref(n)) == OK
    assert n.value >= 300 * 32 * 8                      # LSE and Delta per (token, head)
    assert lib().sdpa_bwd_varlen_workspace_size(1, 2, cu, cu, 32, 32, 128, 128, 2, ctypes.byref(n)) == OK
    assert n.value >= 300 * 32 * (8 + 128 * 4)         # plus the fp32 dQ accumulator
    assert varlen_call([100, 300], [100, 300], det=5) == INVALID
    # (sequence, query head) of a chunk of sequences must fit grid y (65535)
    assert varlen_call([100, 300], [100, 300], Hq=40000, Hkv=40000) == UNSUPPORTED
    big = sb.Tensor3(FAKE, 1 << 23, 128, 1)                          # token stride 2^23
    cu = (ctypes.c_int64 * 2)(100, 300)
    st = sb.Stats(1, FAKE, FAKE, 0, 1, 32)
    ts = [t3() for _ in range(8)]
    ts[2] = big
    assert lib().sdpa_bwd_varlen(1, 2, cu, cu, 32, 32, 128, 128, 0.088, 1, 0, 1,
                                 *[ctypes.byref(t) for t in ts[:5]], ctypes.byref(st),
                                 *[ctypes.byref(t) for t in ts[5:]], FAKE, 1 << 34, None) == UNSUPPORTED


@pytest.mark.skipif(torch.cuda.device_count() > 0, reason="would launch on fake pointers")
def test_varlen_valid_without_device():
    assert varlen_call([100, 300], [100, 300]) == HIP
    assert varlen_call([100, 300], [100, 200]) == HIP             # causal, unequal lengths
    assert varlen_call([100, 300], [100, 300], grad=2) == HIP     # fp32 gradients


def fwd_call(**kw):
    a = dict(dtype=0, B=1, Hq=2, Hkv=1, Sq=64, Sk=64, D=64, Dv=None, scale=0.1, causal=1)
    a.update(kw)
    so = sb.StatsOut(FAKE, 128, 64, 1)
    dv = a["D"] if a["Dv"] is None else a["Dv"]
    return lib().sdpa_fwd_stats(a["dtype"], a["B"], a["Hq"], a["Hkv"], a["Sq"], a["Sk"], a["D"], dv,
                                a["scale"], a["causal"], ctypes.byref(t4()), ctypes.byref(t4()),
                                ctypes.byref(t4()), ctypes.byref(t4()), ctypes.byref(so), None)


def test_fwd_validation():
    assert fwd_call(Hq=3, Hkv=2) == INVALID
    assert fwd_call(D=256) == UNSUPPORTED
    assert fwd_call(dtype=2) == INVALID


def fwd_varlen_call(cu_q, cu_k, **kw):
    a = dict(dtype=1, Hq=4, Hkv=2, D=128, Dv=None, scale=0.088, causal=1, lse=FAKE)
    a.update(kw)
    aq = (ctypes.c_int64 * len(cu_q))(*cu_q)
    ak = (ctypes.c_int64 * len(cu_k))(*cu_k)
    so = sb.StatsOut(a["lse"], 0, 1, 4)
    ts = [t3() for _ in range(4)]
    dv = a["D"] if a["Dv"] is None else a["Dv"]
    return lib().sdpa_fwd_stats_varlen(a["dtype"], len(cu_q), aq, ak, a["Hq"], a["Hkv"], a["D"], dv, a["scale"],
                                       a["causal"], *[ctypes.byref(t) for t in ts], ctypes.byref(so), None)


def test_fwd_varlen_validation():
    assert fwd_varlen_call([100, 300], [100, 300], lse=None) == NULLPTR
    assert fwd_varlen_call([100, 50], [100, 50]) == INVALID           # non-monotone
    assert fwd_varlen_call([100, 300], [100, 300], Hq=3) == INVALID   # heads not grouped
    assert fwd_varlen_call([100, 300], [100, 300], dtype=4) == INVALID
    assert fwd_varlen_call([100, 300], [100, 300], D=96) == UNSUPPORTED


@pytest.mark.skipif(torch.cuda.device_count() > 0, reason="would launch on fake pointers")
def test_fwd_varlen_valid_without_device():
    assert fwd_varlen_call([100, 300], [100, 200], causal=0) == HIP
    assert fwd_varlen_call([100, 300], [100, 200]) == HIP             # causal, unequal lengths
    assert fwd_call(causal=1, Sk=32) == HIP                           # dense causal, Sq != Sk


def fwd_selected_call(**kw):
    a = dict(dtype=1, cu=[512], Hq=16, Hkv=1, D=128, bs=64, count=4, mode=2, m=FAKE, l=FAKE,
             mask=None, mask_stride=0)
    a.update(kw)
    a.setdefault("Dv", a["D"])
    cu = (ctypes.c_int64 * len(a["cu"]))(*a["cu"])
    ts = [t3() for _ in range(4)]
    return lib().sdpa_fwd_selected(a["dtype"], len(a["cu"]), cu, cu, a["Hq"], a["Hkv"], a["D"], a["Dv"], 0.088,
                                   a["mode"], a["mask"], a["mask_stride"],
                                   FAKE, 4 * a["count"], a["count"], 1, a["bs"], a["count"],
                                   *[ctypes.byref(t) for t in ts], a["m"], a["l"], 16, 1, None)


def test_fwd_selected_validation():
    assert fwd_selected_call(m=None) == NULLPTR
    assert fwd_selected_call(dtype=3) == INVALID
    assert fwd_selected_call(bs=40) == INVALID          # not a multiple of 16
    assert fwd_selected_call(cu=[500]) == INVALID       # KV length not a multiple of block_size
    assert fwd_selected_call(mode=1) == INVALID
    assert fwd_selected_call(Hq=64) == INVALID          # more than 32 query heads per KV head
    assert fwd_selected_call(D=96) == UNSUPPORTED
    big = sb.Tensor3(FAKE, 128, 1 << 23, 1)                  # head stride 2^23
    cu = (ctypes.c_int64 * 1)(512)
    ts = [t3() for _ in range(4)]
    ts[1] = big
    assert lib().sdpa_fwd_selected(1, 1, cu, cu, 16, 1, 128, 128, 0.088, 2, None, 0, FAKE, 64, 16, 1, 64, 4,
                                   *[ctypes.byref(t) for t in ts], FAKE, FAKE, 16, 1, None) == UNSUPPORTED
    # user attention mask: a row must cover the longest KV sequence (INVALID),
    # base and stride 16-byte multiples (UNSUPPORTED)
    assert fwd_selected_call(mask=FAKE, mask_stride=496) == INVALID
    assert fwd_selected_call(mask=FAKE, mask_stride=520) == UNSUPPORTED
    assert fwd_selected_call(mask=FAKE + 8, mask_stride=512) == UNSUPPORTED
    assert fwd_selected_call(mask=FAKE, mask_stride=496, D=96) == INVALID     # INVALID before UNSUPPORTED


def bwd_selected_call(**kw):
    a = dict(dtype=1, grad=1, det=0, D=128, Dv=128, mask=None, mask_stride=0)
    a.update(kw)
    cu = (ctypes.c_int64 * 1)(512)
    st = sb.Stats(1, FAKE, FAKE, 0, 1, 16)
    ts = [t3() for _ in range(8)]
    return lib().sdpa_bwd_selected(a["dtype"], 1, cu, cu, 16, 1, a["D"], a["Dv"], 0.088, 2,
                                   a["mask"], a["mask_stride"], FAKE, 16, 4, 1, 64, 4,
                                   a["det"], a["grad"], *[ctypes.byref(t) for t in ts[:5]], ctypes.byref(st),
                                   *[ctypes.byref(t) for t in ts[5:]], FAKE, 1 << 34, None)


def test_bwd_selected_validation():
    assert bwd_selected_call(grad=0) == INVALID       # bf16 inputs, fp16 gradients
    assert bwd_selected_call(grad=7) == INVALID
    assert bwd_selected_call(det=3) == INVALID
    assert bwd_selected_call(Dv=0) == INVALID
    assert bwd_selected_call(D=64, Dv=128) == UNSUPPORTED     # kernels: equal 64/128/192, and (192,128)
    assert bwd_selected_call(D=128, Dv=64) == UNSUPPORTED
    assert bwd_selected_call(mask=FAKE, mask_stride=256) == INVALID     # row shorter than the KV length
    assert bwd_selected_call(mask=FAKE, mask_stride=1 << 31) == UNSUPPORTED
    cu = (ctypes.c_int64 * 1)(512)

    def ws(Hq, D, Dv):
        n = ctypes.c_size_t(0)
        assert lib().sdpa_bwd_selected_workspace_size(1, 1, cu, cu, Hq, 1, D, Dv, 64, 4, 0, ctypes.byref(n)) == OK
        return n.value
    assert ws(16, 192, 192) > ws(16, 192, 128)          # wider dV partials, same pieces
    # 16 query heads per KV head: the dK/dV kernel stores dS for the dQ pass,
    # one 16-bit 16-head x 64-key tile per (token, slot) entry
    stored_ds = 512 * 4 * 16 * 64 * 2
    assert min(ws(16, 64, 64), ws(16, 128, 128), ws(16, 192, 128)) >= stored_ds
    assert ws(8, 128, 128) < stored_ds
    assert fwd_selected_call(D=128, Dv=192) == UNSUPPORTED


@pytest.mark.skipif(torch.cuda.device_count() > 0, reason="would launch on fake pointers")
def test_bwd_selected_valid_without_device():
    assert bwd_selected_call() == HIP
    assert bwd_selected_call(grad=2) == HIP           # fp32 gradients
    assert bwd_selected_call(D=192, Dv=128) == HIP    # unequal head dims
    assert bwd_selected_call(D=192, Dv=192) == HIP
    assert bwd_selected_call(mask=FAKE, mask_stride=512) == HIP   # with a user mask


@pytest.mark.skipif(torch.cuda.device_count() > 0, reason="would launch on fake pointers")
def test_fwd_selected_valid_without_device():
    assert fwd_selected_call() == HIP
    assert fwd_selected_call(cu=[256 * (i + 1) for i in range(70)]) == HIP   # 70 sequences
    assert fwd_selected_call(D=192, Dv=128) == HIP
