"""Seeded synthetic inputs for the SDPA-backward workloads.

This module only draws random numbers and rounds them to the 16-bit I/O types.
It holds none of the attention arithmetic, so both the fp64 oracle (through the
tests) and the HIP library (through the tests and the benchmark) can take their
inputs from it without sharing any of the method.

Conventions
-----------
* Every tensor is drawn from ``numpy.random.default_rng([42, config_id, tensor_id])``
  with tensor ids Q=0, K=1, V=2, dO=3, lengths=4, topk=5.  The base seed 42 is
  the one the cuDNN SDPA-backward sample notebook sets before drawing its
  inputs (cudnn-frontend notebook, "Problem sizes" cell).
* Values are N(0, 1) in fp64, then rounded to nearest-even to fp16 or bf16.
  16-bit tensors are returned as ``uint16`` bit patterns so that the exact same
  bytes reach the GPU (as a torch tensor view) and the oracle (upcast exactly).
* Dense tensors are drawn as one flat buffer in their *physical* order and then
  viewed in the logical (B, H, S, D) order, the way the notebook builds its
  BSHD-physical / BHSD-logical tensors (cudnn-frontend notebook, tensor-creation
  cell).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace

import numpy as np

BASE_SEED = 42
TID_Q, TID_K, TID_V, TID_DO, TID_LEN, TID_TOPK = 0, 1, 2, 3, 4, 5

IO_DTYPES = ("f16", "bf16")


def rng(config_id: int, tensor_id: int) -> np.random.Generator:
    return np.random.default_rng([BASE_SEED, int(config_id), int(tensor_id)])


# ----------------------------------------------------------------------------
# 16-bit encodings (round to nearest, ties to even) and exact decodes
# ----------------------------------------------------------------------------

def encode(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round fp64/fp32 values to fp16 or bf16; return the uint16 bit patterns."""
    x = np.asarray(x)
    if dtype == "f16":
        # numpy converts double -> half with a single correctly rounded step.
        return x.astype(np.float16).view(np.uint16)
    if dtype == "bf16":
        # Correct rounding straight from fp64: bf16 keeps the top 8 mantissa
        # bits of fp32, so round the fp64 value to fp32 with round-to-odd
        # first (exact sticky bit), then to bf16 with ties-to-even.
        x64 = x.astype(np.float64)
        f32 = x64.astype(np.float32)
        u = f32.view(np.uint32).astype(np.uint64)
        back = f32.astype(np.float64)
        inexact = (back != x64) & np.isfinite(x64)
        # round-to-odd: if the fp32 rounding was inexact, force the last bit
        # to 1 on the truncated-towards-zero value
        trunc_mag_gt = np.abs(back) > np.abs(x64)
        u_trunc = np.where(inexact & trunc_mag_gt, u - 1, u)
        u_odd = np.where(inexact, u_trunc | 1, u_trunc)
        lsb = (u_odd >> 16) & 1
        r = (u_odd + 0x7FFF + lsb) >> 16
        nan = np.isnan(x64)
        r = np.where(nan, 0x7FC0, r)
        return r.astype(np.uint16)
    raise ValueError(f"unknown 16-bit dtype {dtype!r}")


def decode(bits: np.ndarray, dtype: str) -> np.ndarray:
    """Exact fp64 value of fp16/bf16 bit patterns."""
    bits = np.asarray(bits, dtype=np.uint16)
    if dtype == "f16":
        return bits.view(np.float16).astype(np.float64)
    if dtype == "bf16":
        return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    raise ValueError(f"unknown 16-bit dtype {dtype!r}")


def normal_bits(shape, dtype: str, config_id: int, tensor_id: int) -> np.ndarray:
    """N(0,1) draws in the given (physical) shape, rounded to the 16-bit type."""
    n = int(np.prod(shape))
    x = rng(config_id, tensor_id).standard_normal(n)
    return encode(x, dtype).reshape(shape)


# ----------------------------------------------------------------------------
# Packed variable-length batches
# ----------------------------------------------------------------------------

def draw_lengths(n: int, lo: int, hi: int, config_id: int) -> np.ndarray:
    """n sequence lengths uniform over the integers lo..hi inclusive."""
    return rng(config_id, TID_LEN).integers(lo, hi, size=n, endpoint=True).astype(np.int64)


def inclusive_offsets(lengths) -> np.ndarray:
    """The cumulative-length array in the Ascend form: B inclusive end offsets
    (no leading zero), int64 (aclnnNsaSelectedAttentionGrad, parameter table,
    actualSeqQLenOptional / actualSeqKvLenOptional)."""
    return np.cumsum(np.asarray(lengths, dtype=np.int64)).astype(np.int64)


# ----------------------------------------------------------------------------
# NSA top-k block choices
# ----------------------------------------------------------------------------

def draw_topk(seq_lengths, n_kv_heads: int, block_size: int, block_count: int,
              config_id: int) -> np.ndarray:
    """int32 [T, N2, count] block choices, relative to each sequence's start.

    For a token at local position t its own block is b = t // block_size.  When
    b >= count-1 the row is {b} plus count-1 distinct blocks drawn without
    replacement from 0..b-1; otherwise it is 0..b padded with copies of b.
    Distinct blocks come sorted, padding last.
    """
    g = rng(config_id, TID_TOPK)
    rows = []
    for L in seq_lengths:
        for t in range(int(L)):
            for _h in range(n_kv_heads):
                b = t // block_size
                if b + 1 >= block_count:
                    others = g.choice(b, size=block_count - 1, replace=False) if block_count > 1 else []
                    row = sorted([b, *map(int, others)])
                else:
                    row = list(range(b + 1)) + [b] * (block_count - b - 1)
                rows.append(row)
    T = int(np.sum(seq_lengths))
    return np.asarray(rows, dtype=np.int32).reshape(T, n_kv_heads, block_count)


# ----------------------------------------------------------------------------
# The five workloads
# ----------------------------------------------------------------------------

@dataclass
class Workload:
    """Description of one synthetic problem; arrays are drawn lazily."""
    config_id: int
    name: str
    kind: str                 # "dense" | "varlen" | "selected"
    dtype: str                # "f16" | "bf16"
    causal: bool
    scale: float
    D: int
    Hq: int
    Hkv: int
    # dense
    B: int = 0
    S: int = 0
    layout: str = "bhsd"      # physical layout for dense: "bhsd" or "bshd"
    # varlen / selected
    lengths: np.ndarray | None = None
    block_size: int = 0
    block_count: int = 0
    stats_source: str = "oracle"   # who produces O and the stats
    extra: dict = field(default_factory=dict)
    Dv_: int = 0              # head dim of V, O and dO when it differs from D

    @property
    def Dv(self) -> int:
        return self.Dv_ or self.D

    # -- dense helpers -------------------------------------------------------
    def dense_physical_shape(self, heads: int) -> tuple:
        if self.layout == "bshd":
            return (self.B, self.S, heads, self.D)
        return (self.B, heads, self.S, self.D)

    def dense_bits(self, tensor_id: int, heads: int) -> np.ndarray:
        """Logical (B, H, S, D) view of a physically laid out draw."""
        phys = normal_bits(self.dense_physical_shape(heads), self.dtype, self.config_id, tensor_id)
        if self.layout == "bshd":
            return phys.transpose(0, 2, 1, 3)
        return phys

    # -- packed helpers ------------------------------------------------------
    @property
    def T(self) -> int:
        return int(np.sum(self.lengths)) if self.lengths is not None else self.B * self.S

    def packed_bits(self, tensor_id: int, heads: int) -> np.ndarray:
        """(T, heads, dim): Q and K take D, V and dO take Dv."""
        dim = self.Dv if tensor_id in (TID_V, TID_DO) else self.D
        return normal_bits((self.T, heads, dim), self.dtype, self.config_id, tensor_id)

    def cu_seqlens(self) -> np.ndarray:
        return inclusive_offsets(self.lengths)

    def topk(self) -> np.ndarray:
        return draw_topk(self.lengths, self.Hkv, self.block_size, self.block_count, self.config_id)

    # -- work counting (for reports) -----------------------------------------
    def counted_flops(self) -> float:
        """5 matmuls of 2*Sq*Sk*D per query head; halved when causal; over the
        selected keys only for the block-sparse variant."""
        if self.kind == "dense":
            f = 5 * 2.0 * self.S * self.S * self.D * self.B * self.Hq
            return f / 2 if self.causal else f
        if self.kind == "varlen":
            f = sum(5 * 2.0 * int(L) * int(L) * self.D * self.Hq for L in self.lengths)
            return f / 2 if self.causal else f
        if self.kind == "selected":
            # S, dQ and dK contract or produce D columns, dP and dV Dv columns
            return 2.0 * self.T * self.Hq * self.block_count * self.block_size * (3 * self.D + 2 * self.Dv)
        raise ValueError(self.kind)


def workload(config_id: int) -> Workload:
    if config_id == 1:
        return Workload(1, "tiny dense B1 H2 S128 D64 fp16 non-causal", "dense", "f16",
                        False, 1.0 / math.sqrt(64), 64, 2, 2, B=1, S=128, layout="bhsd",
                        stats_source="oracle")
    if config_id == 2:
        return Workload(2, "GPT-2 shape B4 H12 S1024 D64 fp16 causal", "dense", "f16",
                        True, 1.0 / 8.0, 64, 12, 12, B=4, S=1024, layout="bshd",
                        stats_source="gpu")
    if config_id == 3:
        return Workload(3, "long context B2 H16 S4096 D128 bf16 causal", "dense", "bf16",
                        True, 1.0 / math.sqrt(128), 128, 16, 16, B=2, S=4096, layout="bshd",
                        stats_source="gpu")
    if config_id == 4:
        return Workload(4, "packed varlen 8 seqs L~U[256,2048] H32 D128 bf16 causal", "varlen",
                        "bf16", True, 1.0 / math.sqrt(128), 128, 32, 32,
                        lengths=draw_lengths(8, 256, 2048, 4), stats_source="oracle")
    if config_id == 5:
        return Workload(5, "NSA selected T4096 Hq16 Hkv1 D128 bf16 bs64x16 causal", "selected",
                        "bf16", True, 1.0 / math.sqrt(128), 128, 16, 1,
                        lengths=np.array([4096], dtype=np.int64), block_size=64,
                        block_count=16, stats_source="oracle")
    raise ValueError(f"no workload {config_id}")


def with_head_dims(wl: Workload, D: int, Dv: int) -> Workload:
    """The same workload with query/key head dim D and value head dim Dv (the
    NSA page allows D of 192 or 128, unequal for K and V); scale 1/sqrt(D)."""
    return replace(wl, name=wl.name.replace(f"D{wl.D}", f"Dqk{D} Dv{Dv}"), D=D, Dv_=0 if Dv == D else Dv,
                   scale=1.0 / math.sqrt(D))


ALL_CONFIGS = (1, 2, 3, 4, 5)
