"""Python binding of libsdpa_bwd (SDPA backward for MI355X / gfx950).

Argument marshalling only: torch tensors are turned into pointers and element
strides, outputs and workspaces are allocated with torch, and every step of the
computation runs in the HIP kernels of ``libsdpa_bwd.so``.  There is no
fallback: if the library is missing or fails to load, every call raises.

torch is imported before the library is loaded so that the library binds to
the HIP runtime torch already mapped (both carry the soname libamdhip64.so.7);
two runtimes in one process would not share streams or memory.
"""
from __future__ import annotations

import ctypes
import os
import re

import torch

__all__ = [
    "SdpaError", "load", "library_path", "fwd_stats", "bwd", "bwd_noalloc", "bwd_varlen", "bwd_selected",
    "selected_build_index", "bwd_workspace_size", "bwd_varlen_workspace_size",
    "bwd_selected_workspace_size", "STATUS",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libsdpa_bwd.so")
HEADER = os.path.join(os.path.dirname(_HERE), "include", "sdpa_bwd.h")

STATUS = {0: "SDPA_OK", 1: "SDPA_ERR_NULLPTR", 2: "SDPA_ERR_INVALID", 3: "SDPA_ERR_UNSUPPORTED",
          4: "SDPA_ERR_WORKSPACE", 5: "SDPA_ERR_HIP"}
F16, BF16, F32 = 0, 1, 2
STATS_LSE, STATS_MAX_SUM = 0, 1

c_i64 = ctypes.c_int64
c_int = ctypes.c_int
c_vp = ctypes.c_void_p
c_dbl = ctypes.c_double
c_size = ctypes.c_size_t


class Tensor4(ctypes.Structure):
    _fields_ = [("data", c_vp), ("stride_b", c_i64), ("stride_h", c_i64), ("stride_s", c_i64),
                ("stride_d", c_i64)]


class Tensor3(ctypes.Structure):
    _fields_ = [("data", c_vp), ("stride_t", c_i64), ("stride_n", c_i64), ("stride_d", c_i64)]


class Stats(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("lse_or_max", c_vp), ("sum", c_vp),
                ("stride_b", c_i64), ("stride_h", c_i64), ("stride_s", c_i64)]


class StatsOut(ctypes.Structure):
    _fields_ = [("lse", c_vp), ("stride_b", c_i64), ("stride_h", c_i64), ("stride_s", c_i64)]


class SdpaError(RuntimeError):
    def __init__(self, status: int, fn: str, msg: str):
        super().__init__(f"{fn} failed: {STATUS.get(status, status)} ({msg})")
        self.status = status


_lib = None

P4, P3, PS = ctypes.POINTER(Tensor4), ctypes.POINTER(Tensor3), ctypes.POINTER(Stats)
PI64 = ctypes.POINTER(c_i64)

_SIGS = {
    "sdpa_status_string": (ctypes.c_char_p, [c_int]),
    "sdpa_last_error": (ctypes.c_char_p, []),
    "sdpa_fwd_stats": (c_int, [c_int, c_i64, c_i64, c_i64, c_i64, c_i64, c_i64, c_i64, c_dbl, c_int,
                               P4, P4, P4, P4, ctypes.POINTER(StatsOut), c_vp]),
    "sdpa_fwd_stats_varlen": (c_int, [c_int, c_i64, PI64, PI64, c_i64, c_i64, c_i64, c_i64, c_dbl, c_int,
                                      P3, P3, P3, P3, ctypes.POINTER(StatsOut), c_vp]),
    "sdpa_bwd_workspace_size": (c_int, [c_int, c_i64, c_i64, c_i64, c_i64, c_i64, c_i64, c_i64, c_int,
                                        ctypes.POINTER(c_size)]),
    "sdpa_bwd": (c_int, [c_int, c_i64, c_i64, c_i64, c_i64, c_i64, c_i64, c_i64, c_dbl, c_int, c_int, c_int,
                         P4, P4, P4, P4, P4, PS, P4, P4, P4, c_vp, c_size, c_vp]),
    "sdpa_bwd_noalloc": (c_int, [c_int, c_i64, c_i64, c_i64, c_i64, c_i64, c_i64, c_i64, c_dbl, c_int, c_int, c_int,
                                 P4, P4, P4, P4, P4, PS, P4, P4, P4, c_vp]),
    "sdpa_bwd_varlen_workspace_size": (c_int, [c_int, c_i64, PI64, PI64, c_i64, c_i64, c_i64, c_i64, c_int,
                                               ctypes.POINTER(c_size)]),
    "sdpa_bwd_varlen": (c_int, [c_int, c_i64, PI64, PI64, c_i64, c_i64, c_i64, c_i64, c_dbl, c_int, c_int, c_int,
                                P3, P3, P3, P3, P3, PS, P3, P3, P3, c_vp, c_size, c_vp]),
    "sdpa_bwd_selected_workspace_size": (c_int, [c_int, c_i64, PI64, PI64, c_i64, c_i64, c_i64, c_i64,
                                                 c_i64, c_i64, c_int, ctypes.POINTER(c_size)]),
    "sdpa_bwd_selected": (c_int, [c_int, c_i64, PI64, PI64, c_i64, c_i64, c_i64, c_i64, c_dbl, c_int,
                                  c_vp, c_i64, c_vp, c_i64, c_i64, c_i64, c_i64, c_i64, c_int, c_int,
                                  P3, P3, P3, P3, P3, PS, P3, P3, P3, c_vp, c_size, c_vp]),
    "sdpa_fwd_selected": (c_int, [c_int, c_i64, PI64, PI64, c_i64, c_i64, c_i64, c_i64, c_dbl, c_int,
                                  c_vp, c_i64, c_vp, c_i64, c_i64, c_i64, c_i64, c_i64,
                                  P3, P3, P3, P3, c_vp, c_vp, c_i64, c_i64, c_vp]),
    "sdpa_profile_begin": (c_int, []),
    "sdpa_profile_end": (c_int, [c_int, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(c_i64)]),
    "sdpa_kernel_name": (ctypes.c_char_p, [c_int]),
    "sdpa_selected_build_index": (c_int, [c_i64, PI64, PI64, c_i64, c_vp, c_i64, c_i64, c_i64,
                                          c_i64, c_i64, c_vp, c_vp, c_vp, c_size, c_vp]),
}


N_KERNEL_IDS = 11


class KernelTimer:
    """Context manager: per-kernel HIP-event timing of every library launch
    inside the block.  After exit, ``result[name] = (total_ms, launches)``."""

    def __enter__(self):
        _check(load().sdpa_profile_begin(), "sdpa_profile_begin")
        self.result = {}
        return self

    def __exit__(self, *exc):
        ms = (ctypes.c_double * N_KERNEL_IDS)()
        n = (c_i64 * N_KERNEL_IDS)()
        _check(load().sdpa_profile_end(N_KERNEL_IDS, ms, n), "sdpa_profile_end")
        for i in range(N_KERNEL_IDS):
            if n[i]:
                self.result[load().sdpa_kernel_name(i).decode()] = (ms[i], n[i])
        return False


def library_path() -> str:
    return _LIB_PATH


def _hip_runtimes_mapped() -> set[str]:
    found = set()
    try:
        with open("/proc/self/maps") as fh:
            for line in fh:
                m = re.search(r"(\S*libamdhip64\.so\S*)$", line.strip())
                if m:
                    found.add(os.path.realpath(m.group(1)))
    except OSError:
        pass
    return found


def load() -> ctypes.CDLL:
    """Load libsdpa_bwd.so (raises if it is missing: there is no fallback)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(f"{_LIB_PATH} not built; run `python -m sdpa_backward_fa2_amd.build`")
    lib = ctypes.CDLL(_LIB_PATH, mode=ctypes.RTLD_GLOBAL)
    for name, (res, args) in _SIGS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    runtimes = _hip_runtimes_mapped()
    if len(runtimes) > 1:
        raise RuntimeError(f"more than one HIP runtime mapped in this process: {sorted(runtimes)}")
    _lib = lib
    return lib


def declared_functions() -> list[str]:
    """Names of the functions include/sdpa_bwd.h declares."""
    with open(HEADER) as fh:
        text = fh.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"^\s*(?:const\s+)?(?:int|size_t|char\s*\*|void)\s*\*?\s*(sdpa_\w+)\s*\(",
                      text, flags=re.M)


def _check(status: int, fn: str):
    if status != 0:
        msg = load().sdpa_status_string(status)
        raise SdpaError(status, fn, msg.decode() if msg else "")


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float16:
        return F16
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError(f"expected float16 or bfloat16, got {t.dtype}")


def _grads(q, k, v, dq, dk, dv, grad_dtype):
    """The gradient tensors (allocated like q, k, v when not given, in
    grad_dtype or the input dtype) and their element-type code: the input
    type or fp32, the same for all three."""
    want = q.dtype if grad_dtype is None else grad_dtype
    dq = torch.empty_like(q, dtype=want) if dq is None else dq
    dk = torch.empty_like(k, dtype=want) if dk is None else dk
    dv = torch.empty_like(v, dtype=want) if dv is None else dv
    if not (dq.dtype == dk.dtype == dv.dtype):
        raise TypeError(f"gradients differ in dtype: {dq.dtype}, {dk.dtype}, {dv.dtype}")
    if dq.dtype == torch.float32:
        return dq, dk, dv, F32
    if dq.dtype != q.dtype:
        raise TypeError(f"gradients must be {q.dtype} or float32, got {dq.dtype}")
    return dq, dk, dv, _dtype_code(q)


def _stream_ptr(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _t4(x: torch.Tensor) -> Tensor4:
    assert x.dim() == 4
    return Tensor4(x.data_ptr(), *x.stride())


def _t3(x: torch.Tensor) -> Tensor3:
    assert x.dim() == 3
    return Tensor3(x.data_ptr(), *x.stride())


def _squeeze_stats(x: torch.Tensor) -> torch.Tensor:
    """Accept (B, H, S) or the sample's (B, H, S, 1) statistics."""
    if x.dim() == 4 and x.shape[-1] == 1:
        return x[..., 0]
    return x


def _workspace(nbytes: int, device, workspace: torch.Tensor | None) -> torch.Tensor:
    if workspace is not None and workspace.numel() * workspace.element_size() >= nbytes:
        return workspace
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)


# ----------------------------------------------------------------------------
# Forward statistics
# ----------------------------------------------------------------------------

def fwd_stats(q, k, v, scale: float, causal: bool, o=None, lse=None):
    """O and the natural-log LSE (B, Hq, Sq) fp32 for dense (B, H, S, D) inputs
    (v and O may have their own head dim Dv)."""
    lib = load()
    B, Hq, Sq, D = q.shape
    Hkv, Sk, Dv = k.shape[1], k.shape[2], v.shape[3]
    if o is None:
        o = torch.empty_like(q) if Dv == D else q.new_empty((B, Hq, Sq, Dv))
    if lse is None:
        lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=q.device)
    l3 = _squeeze_stats(lse)
    so = StatsOut(l3.data_ptr(), *l3.stride())
    st = lib.sdpa_fwd_stats(_dtype_code(q), B, Hq, Hkv, Sq, Sk, D, Dv, float(scale), int(causal),
                            _t4(q), _t4(k), _t4(v), _t4(o), ctypes.byref(so), _stream_ptr(q.device))
    _check(st, "sdpa_fwd_stats")
    return o, lse


def fwd_stats_varlen(q, k, v, cu_q, cu_kv, scale: float, causal: bool, o=None, lse=None):
    """O and the natural-log LSE (Tq, Hq) fp32 for a packed (T, N, D) batch;
    cu_q / cu_kv: host sequences of inclusive end offsets."""
    lib = load()
    Hq, D = q.shape[1], q.shape[2]
    Hkv, Dv = k.shape[1], v.shape[2]
    if o is None:
        o = torch.empty_like(q) if Dv == D else q.new_empty((q.shape[0], Hq, Dv))
    if lse is None:
        lse = torch.empty((q.shape[0], Hq), dtype=torch.float32, device=q.device)
    so = StatsOut(lse.data_ptr(), 0, lse.stride(1), lse.stride(0))
    aq, n = _cu_host(cu_q)
    ak, _ = _cu_host(cu_kv)
    st = lib.sdpa_fwd_stats_varlen(_dtype_code(q), n, aq, ak, Hq, Hkv, D, Dv, float(scale), int(causal),
                                   _t3(q), _t3(k), _t3(v), _t3(o), ctypes.byref(so), _stream_ptr(q.device))
    _check(st, "sdpa_fwd_stats_varlen")
    return o, lse


# ----------------------------------------------------------------------------
# Dense backward
# ----------------------------------------------------------------------------

# dQ modes (the `deterministic` argument of the backward entry points)
DQ_FASTEST = 0          # the library's fastest method (atomic-free today)
DQ_DETERMINISTIC = 1    # bitwise reproducible
DQ_ATOMIC = 2           # fp32 atomic accumulation (FA2's method)


def bwd_workspace_size(dtype: int, B, Hq, Hkv, Sq, Sk, D, deterministic: int, Dv=None) -> int:
    n = c_size(0)
    _check(load().sdpa_bwd_workspace_size(dtype, B, Hq, Hkv, Sq, Sk, D, D if Dv is None else Dv, int(deterministic),
                                          ctypes.byref(n)), "sdpa_bwd_workspace_size")
    return n.value


def _stats_arg(stats, packed: bool) -> Stats:
    """stats: an LSE tensor, or a (max, sum) pair."""
    if isinstance(stats, (tuple, list)):
        m, s = stats
        m = m if packed else _squeeze_stats(m)
        s = s if packed else _squeeze_stats(s)
        if m.stride() != s.stride():
            raise ValueError("max and sum statistics must share strides")
        kind, a, b, ref = STATS_MAX_SUM, m.data_ptr(), s.data_ptr(), m
    else:
        ref = stats if packed else _squeeze_stats(stats)
        kind, a, b = STATS_LSE, ref.data_ptr(), None
    if packed:   # (T, N[, k]) -> stride_s = token stride, stride_h = head stride
        return Stats(kind, a, b, 0, ref.stride(1), ref.stride(0))
    return Stats(kind, a, b, *ref.stride()[:3])


def prepare_bwd(q, k, v, o, dout, stats, scale: float, causal: bool, deterministic: int = DQ_FASTEST,
                dq=None, dk=None, dv=None, workspace=None, grad_dtype=None):
    """Marshal the arguments of one dense backward once; returns (call, (dq, dk, dv))
    where call() enqueues the backward on the stream that was current when it
    was prepared (prepare inside a capture stream to graph it).  The tensors must
    stay alive and unmoved while call is used.  Gradients are q's dtype or
    float32 (given tensors, else grad_dtype)."""
    lib = load()
    B, Hq, Sq, D = q.shape
    Hkv, Sk, Dv = k.shape[1], k.shape[2], v.shape[3]
    dt = _dtype_code(q)
    dq, dk, dv, gdt = _grads(q, k, v, dq, dk, dv, grad_dtype)
    nbytes = bwd_workspace_size(dt, B, Hq, Hkv, Sq, Sk, D, deterministic, Dv)
    ws = _workspace(nbytes, q.device, workspace)
    sa = _stats_arg(stats, packed=False)
    structs = [_t4(x) for x in (q, k, v, o, dout, dq, dk, dv)]
    args = (dt, B, Hq, Hkv, Sq, Sk, D, Dv, float(scale), int(causal), int(deterministic), gdt,
            *[ctypes.byref(x) for x in structs[:5]], ctypes.byref(sa),
            *[ctypes.byref(x) for x in structs[5:]], ws.data_ptr(), ws.numel(),
            _stream_ptr(q.device))
    fn = lib.sdpa_bwd
    keep = (structs, sa, ws, stats)

    def call():
        _check(fn(*args), "sdpa_bwd")

    call.keep = keep
    return call, (dq, dk, dv)


def bwd(q, k, v, o, dout, stats, scale: float, causal: bool, deterministic: int = DQ_FASTEST,
        dq=None, dk=None, dv=None, workspace=None, grad_dtype=None):
    """dQ, dK, dV of dense attention.  stats: LSE (B, Hq, Sq[, 1]) or (max, sum).
    deterministic: DQ_FASTEST (0), DQ_DETERMINISTIC (1) or DQ_ATOMIC (2); a
    bool is read as 0 or 1.  grad_dtype: torch.float32 for fp32 gradients
    (default: q's dtype, or that of the given dq, dk, dv)."""
    call, outs = prepare_bwd(q, k, v, o, dout, stats, scale, causal, deterministic, dq, dk, dv,
                             workspace, grad_dtype)
    call()
    return outs


def bwd_noalloc(q, k, v, o, dout, stats, scale: float, causal: bool, deterministic: int = DQ_FASTEST,
                dq=None, dk=None, dv=None, grad_dtype=None):
    """The dense backward through sdpa_bwd_noalloc: no workspace, the library's
    fixed per-GPU scratch instead (16 MiB; larger problems raise
    SDPA_ERR_WORKSPACE).  Outputs as bwd; given dq, dk, dv are written in place."""
    lib = load()
    B, Hq, Sq, D = q.shape
    Hkv, Sk, Dv = k.shape[1], k.shape[2], v.shape[3]
    dq, dk, dv, gdt = _grads(q, k, v, dq, dk, dv, grad_dtype)
    sa = _stats_arg(stats, packed=False)
    structs = [_t4(x) for x in (q, k, v, o, dout, dq, dk, dv)]
    _check(lib.sdpa_bwd_noalloc(_dtype_code(q), B, Hq, Hkv, Sq, Sk, D, Dv, float(scale), int(causal),
                                int(deterministic), gdt, *[ctypes.byref(x) for x in structs[:5]],
                                ctypes.byref(sa), *[ctypes.byref(x) for x in structs[5:]],
                                _stream_ptr(q.device)), "sdpa_bwd_noalloc")
    return dq, dk, dv


# ----------------------------------------------------------------------------
# Packed variable-length backward
# ----------------------------------------------------------------------------

def _cu_host(cu):
    arr = (c_i64 * len(cu))(*[int(x) for x in cu])
    return arr, len(cu)


def bwd_varlen_workspace_size(dtype, cu_q, cu_kv, Hq, Hkv, D, deterministic, Dv=None) -> int:
    aq, n = _cu_host(cu_q)
    ak, _ = _cu_host(cu_kv)
    out = c_size(0)
    _check(load().sdpa_bwd_varlen_workspace_size(dtype, n, aq, ak, Hq, Hkv, D, D if Dv is None else Dv,
                                                 int(deterministic),
                                                 ctypes.byref(out)), "sdpa_bwd_varlen_workspace_size")
    return out.value


def prepare_varlen(q, k, v, o, dout, stats, cu_q, cu_kv, scale: float, causal: bool,
                   deterministic: int = DQ_FASTEST, dq=None, dk=None, dv=None, workspace=None,
                   grad_dtype=None):
    """Marshal one packed (T, N, D) backward once; returns (call, (dq, dk, dv)).
    cu_q / cu_kv: host sequences of inclusive end offsets; stats: LSE (T, Hq)
    or a (max, sum) pair of (T, Hq[, 8]) tensors."""
    lib = load()
    Hq, D = q.shape[1], q.shape[2]
    Hkv, Dv = k.shape[1], v.shape[2]
    dt = _dtype_code(q)
    dq, dk, dv, gdt = _grads(q, k, v, dq, dk, dv, grad_dtype)
    aq, n = _cu_host(cu_q)
    ak, _ = _cu_host(cu_kv)
    nbytes = bwd_varlen_workspace_size(dt, cu_q, cu_kv, Hq, Hkv, D, deterministic, Dv)
    ws = _workspace(nbytes, q.device, workspace)
    sa = _stats_arg(stats, packed=True)
    structs = [_t3(x) for x in (q, k, v, o, dout, dq, dk, dv)]
    args = (dt, n, aq, ak, Hq, Hkv, D, Dv, float(scale), int(causal), int(deterministic), gdt,
            *structs[:5], ctypes.byref(sa), *structs[5:], ws.data_ptr(), ws.numel(),
            _stream_ptr(q.device))
    fn = lib.sdpa_bwd_varlen
    keep = (structs, sa, ws, stats, aq, ak)

    def call():
        _check(fn(*args), "sdpa_bwd_varlen")

    call.keep = keep
    return call, (dq, dk, dv)


def bwd_varlen(q, k, v, o, dout, stats, cu_q, cu_kv, scale: float, causal: bool,
               deterministic: int = DQ_FASTEST, dq=None, dk=None, dv=None, workspace=None,
               grad_dtype=None):
    """Packed (T, N, D) backward; cu_q / cu_kv: host sequences of inclusive end
    offsets; stats: LSE (T, Hq) or a (max, sum) pair of (T, Hq[, 8]) tensors."""
    call, outs = prepare_varlen(q, k, v, o, dout, stats, cu_q, cu_kv, scale, causal, deterministic,
                                dq, dk, dv, workspace, grad_dtype)
    call()
    return outs


# ----------------------------------------------------------------------------
# NSA selected attention
# ----------------------------------------------------------------------------

def bwd_selected_workspace_size(dtype, cu_q, cu_kv, Hq, Hkv, D, block_size, block_count,
                                deterministic, Dv=None) -> int:
    """Bytes of workspace for the selected backward; D: q/k head dim, Dv: v's
    (default D)."""
    aq, n = _cu_host(cu_q)
    ak, _ = _cu_host(cu_kv)
    out = c_size(0)
    Dv = D if Dv is None else Dv
    _check(load().sdpa_bwd_selected_workspace_size(dtype, n, aq, ak, Hq, Hkv, D, Dv, block_size,
                                                   block_count, int(deterministic), ctypes.byref(out)),
           "sdpa_bwd_selected_workspace_size")
    return out.value


def _mask_arg(atten_mask):
    """(pointer, row stride) of an optional 2-D bool/uint8 device mask."""
    if atten_mask is None:
        return None, 0
    if atten_mask.dim() != 2 or atten_mask.dtype not in (torch.bool, torch.uint8) or atten_mask.stride(1) != 1:
        raise ValueError("atten_mask: a 2-D bool or uint8 device tensor with unit column stride")
    return atten_mask.data_ptr(), atten_mask.stride(0)


def prepare_selected(q, k, v, o, dout, stats, topk, cu_q, cu_kv, block_size: int, scale: float,
                     sparse_mode: int, deterministic: int = DQ_FASTEST, dq=None, dk=None, dv=None,
                     workspace=None, grad_dtype=None, atten_mask=None):
    """Marshal one NSA selected-attention backward once; returns (call, (dq, dk, dv)).
    topk: int32 (T, Hkv, count) on the device; atten_mask: optional (Sq, Sk)
    bool/uint8 device tensor, True = masked out (sequence-local positions)."""
    lib = load()
    Hq, D = q.shape[1], q.shape[2]
    Hkv, Dv = k.shape[1], v.shape[2]
    count = topk.shape[2]
    dt = _dtype_code(q)
    dq, dk, dv, gdt = _grads(q, k, v, dq, dk, dv, grad_dtype)
    aq, n = _cu_host(cu_q)
    ak, _ = _cu_host(cu_kv)
    nbytes = bwd_selected_workspace_size(dt, cu_q, cu_kv, Hq, Hkv, D, block_size, count, deterministic, Dv)
    ws = _workspace(nbytes, q.device, workspace)
    sa = _stats_arg(stats, packed=True)
    structs = [_t3(x) for x in (q, k, v, o, dout, dq, dk, dv)]
    mp, ms = _mask_arg(atten_mask)
    args = (dt, n, aq, ak, Hq, Hkv, D, Dv, float(scale), int(sparse_mode), mp, ms,
            topk.data_ptr(), *topk.stride(), block_size, count, int(deterministic), gdt,
            *structs[:5], ctypes.byref(sa), *structs[5:], ws.data_ptr(), ws.numel(),
            _stream_ptr(q.device))
    fn = lib.sdpa_bwd_selected
    keep = (structs, sa, ws, stats, topk, aq, ak, atten_mask)

    def call():
        _check(fn(*args), "sdpa_bwd_selected")

    call.keep = keep
    return call, (dq, dk, dv)


def bwd_selected(q, k, v, o, dout, stats, topk, cu_q, cu_kv, block_size: int, scale: float,
                 sparse_mode: int, deterministic: int = DQ_FASTEST, dq=None, dk=None, dv=None,
                 workspace=None, grad_dtype=None, atten_mask=None):
    """NSA selected-attention backward; topk: int32 (T, Hkv, count) on the device;
    gradients in q's dtype or float32 (grad_dtype, or the given tensors');
    atten_mask as prepare_selected."""
    call, outs = prepare_selected(q, k, v, o, dout, stats, topk, cu_q, cu_kv, block_size, scale,
                                  sparse_mode, deterministic, dq, dk, dv, workspace, grad_dtype, atten_mask)
    call()
    return outs


def fwd_selected(q, k, v, topk, cu_q, cu_kv, block_size: int, scale: float, sparse_mode: int,
                 o=None, m=None, l=None, atten_mask=None):
    """NSA selected-attention forward: O and the (max, sum) statistics (T, Hq)
    fp32 over each token's gathered keys; topk: int32 (T, Hkv, count) on the device.
    O has v's head dim."""
    lib = load()
    Hq, D = q.shape[1], q.shape[2]
    Hkv, Dv = k.shape[1], v.shape[2]
    count = topk.shape[2]
    if o is None:
        o = torch.empty((q.shape[0], Hq, Dv), dtype=q.dtype, device=q.device)
    if m is None:
        m = torch.empty((q.shape[0], Hq), dtype=torch.float32, device=q.device)
    if l is None:
        l = torch.empty_like(m)
    assert m.stride() == l.stride()
    aq, n = _cu_host(cu_q)
    ak, _ = _cu_host(cu_kv)
    mp, ms = _mask_arg(atten_mask)
    st = lib.sdpa_fwd_selected(_dtype_code(q), n, aq, ak, Hq, Hkv, D, Dv, float(scale), int(sparse_mode),
                               mp, ms, topk.data_ptr(), *topk.stride(), int(block_size), count,
                               _t3(q), _t3(k), _t3(v), _t3(o), m.data_ptr(), l.data_ptr(),
                               m.stride(0), m.stride(1), _stream_ptr(q.device))
    _check(st, "sdpa_fwd_selected")
    return o, m, l


def selected_build_index(topk, cu_q, cu_kv, block_size: int, workspace=None):
    """CSR inverse of the top-k choice: (offsets int32 [Hkv*NB+1], entries int32)."""
    lib = load()
    T, Hkv, count = topk.shape
    NB = int(cu_kv[-1]) // block_size
    offsets = torch.empty(Hkv * NB + 1, dtype=torch.int32, device=topk.device)
    entries = torch.empty(max(T * Hkv * count, 1), dtype=torch.int32, device=topk.device)
    aq, n = _cu_host(cu_q)
    ak, _ = _cu_host(cu_kv)
    nbytes = bwd_selected_workspace_size(F16, cu_q, cu_kv, Hkv, Hkv, 128, block_size, count, False)
    ws = _workspace(nbytes, topk.device, workspace)
    st = lib.sdpa_selected_build_index(n, aq, ak, Hkv, topk.data_ptr(), *topk.stride(), block_size,
                                       count, offsets.data_ptr(), entries.data_ptr(), ws.data_ptr(),
                                       ws.numel(), _stream_ptr(topk.device))
    _check(st, "sdpa_selected_build_index")
    return offsets, entries[:T * Hkv * count]
