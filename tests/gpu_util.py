"""Helpers shared by the GPU parity tests: moving synth's bit patterns onto the
device and measuring errors against the oracle.  No attention arithmetic."""
import os

import numpy as np
import torch

import synth

TORCH_DTYPE = {"f16": torch.float16, "bf16": torch.bfloat16}
# max|err| / max|ref| bounds per I/O type for dQ, dK, dV
REL_TOL = {"f16": 5e-3, "bf16": 2e-2}
STATS_ABS_TOL = 1e-4


def to_device(bits: np.ndarray, dtype: str, device="cuda") -> torch.Tensor:
    """uint16 bit patterns (any strides) -> device tensor with the same logical
    shape.  Physical order is the numpy array's memory order if contiguous in
    some permutation; callers pass the physical array and permute afterwards."""
    arr = np.ascontiguousarray(bits).view(np.int16)
    return torch.from_numpy(arr).to(device).view(TORCH_DTYPE[dtype])


def dense_input(wl: synth.Workload, tensor_id: int, heads: int, device="cuda"):
    """(device tensor in the workload's physical layout viewed as (B,H,S,D),
    fp64 numpy copy in logical order)."""
    phys = synth.normal_bits(wl.dense_physical_shape(heads), wl.dtype, wl.config_id, tensor_id)
    t = to_device(phys, wl.dtype, device)
    x = synth.decode(phys, wl.dtype)
    if wl.layout == "bshd":
        t = t.permute(0, 2, 1, 3)
        x = x.transpose(0, 2, 1, 3)
    return t, x


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().double().numpy()


def rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    denom = float(np.max(np.abs(ref)))
    return float(np.max(np.abs(got - ref))) / (denom if denom > 0 else 1.0)


# (test id, what, dtype, error, bound) of every assert_rel in this session;
# conftest writes them out at the end of a GPU run so the margin under each
# bound is on record, not only pass or fail
MARGINS = []


def assert_rel(got, ref, dtype: str, what: str):
    e = rel_err(got, ref)
    test = os.environ.get("PYTEST_CURRENT_TEST", "").split(" ")[0]
    MARGINS.append((test, what, dtype, e, REL_TOL[dtype]))
    assert e <= REL_TOL[dtype], f"{what}: max|err|/max|ref| = {e:.3e} > {REL_TOL[dtype]:.0e}"
    return e


def empty_like_layout(t: torch.Tensor) -> torch.Tensor:
    """Uninitialised tensor with t's strides (outputs keep the input's layout)."""
    return torch.empty_strided(t.shape, t.stride(), dtype=t.dtype, device=t.device)
