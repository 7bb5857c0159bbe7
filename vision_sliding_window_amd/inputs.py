"""Seeded synthetic inputs and the workload shapes (no attention arithmetic here).

This module is the one piece shared by the GPU path's tests/bench and the fp64
oracle's tests: it draws random numbers and rounds them to the storage type,
nothing else.

Recipe (one ``numpy.random.default_rng(seed)`` per workload): draw Q, K, V in
that order as standard normals in float64 with shape [B, heads, H, W, d], then
the relative-position-bias table [heads, 2k-1, 2k-1] as standard normals times
``rpb_std`` (0.02 by default: the "N(0, 0.02)" of the workloads read as a
standard deviation).  Q, K, V are rounded once to the storage dtype with
round-to-nearest-even (torch's cast); the table is rounded to float32.  The
"exact" float64 copies returned beside them are those rounded values widened
back, which is what the GPU receives.

The shapes are those of the Neighborhood Attention Transformer's NAT-Tiny
stages (CSDN translation of the paper, section 3.3: feature maps at h/4 ...
h/32 of a 224x224 input, i.e. 56, 28, 14 and 7) and of the layer benchmark up
to 448x448 (Fig. 4 of the same page).
"""
from __future__ import annotations

import dataclasses

import numpy as np
import torch

DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}
DTYPE_CODE = {"f32": 0, "f16": 1, "bf16": 2}


@dataclasses.dataclass(frozen=True)
class Workload:
    """One benchmark / parity configuration.  `op` is the operation: "na2d"
    (the default), "na1d" (a sequence of length W: H = depth = 1), "na3d" (a
    depth x H x W volume, cubic window) or "sasa2d" (centred windows over a
    zero-padded map)."""
    name: str
    B: int
    heads: int
    H: int
    W: int
    d: int
    k: int
    dtype: str
    op: str = "na2d"
    depth: int = 1

    @property
    def queries(self) -> int:
        return self.B * self.heads * self.depth * self.H * self.W

    @property
    def shape(self):
        if self.op == "na1d":
            return (self.B, self.heads, self.W, self.d)
        if self.op == "na3d":
            return (self.B, self.heads, self.depth, self.H, self.W, self.d)
        return (self.B, self.heads, self.H, self.W, self.d)

    @property
    def rpb_shape(self):
        return rpb_shape(self.op, self.heads, self.k)

    @property
    def keys_per_query(self) -> int:
        return self.k ** {"na1d": 1, "na2d": 2, "sasa2d": 2, "na3d": 3}[self.op]


def rpb_shape(op: str, heads: int, k: int):
    n = 2 * k - 1
    return {"na1d": (heads, n), "na3d": (heads, n, n, n)}.get(op, (heads, n, n))


# The five workloads (tiny parity case, NAT-Tiny stage 1, all four NAT-Tiny
# stages, a 448x448 map, the large-kernel sweep).
WORKLOADS = {
    "tiny_14x14_k7_f32": Workload("tiny_14x14_k7_f32", 1, 1, 14, 14, 32, 7, "f32"),
    "tiny_sa_7x7_k7_f32": Workload("tiny_sa_7x7_k7_f32", 1, 1, 7, 7, 32, 7, "f32"),
    "nat_tiny_stage1_f16": Workload("nat_tiny_stage1_f16", 32, 2, 56, 56, 32, 7, "f16"),
    "nat_tiny_stage1_bf16": Workload("nat_tiny_stage1_bf16", 32, 2, 56, 56, 32, 7, "bf16"),
    "nat_tiny_stage2_bf16": Workload("nat_tiny_stage2_bf16", 32, 4, 28, 28, 32, 7, "bf16"),
    "nat_tiny_stage3_bf16": Workload("nat_tiny_stage3_bf16", 32, 8, 14, 14, 32, 7, "bf16"),
    "nat_tiny_stage4_bf16": Workload("nat_tiny_stage4_bf16", 32, 16, 7, 7, 32, 7, "bf16"),
    "hires_448_f16": Workload("hires_448_f16", 1, 4, 448, 448, 32, 7, "f16"),
    "large_kernel_k13_bf16": Workload("large_kernel_k13_bf16", 8, 4, 128, 128, 32, 13, "bf16"),
    "large_kernel_k21_bf16": Workload("large_kernel_k21_bf16", 8, 4, 128, 128, 32, 21, "bf16"),
    # beyond the 2D forward: a sequence with the same queries and keys per query
    # as NAT-Tiny stage 1 (56 x 56 = 3136 positions, 49 keys), SASA windows on
    # the stage-1 map, and a 16 x 56 x 56 volume with 5 x 5 x 5 windows
    "na1d_L3136_k49_f16": Workload("na1d_L3136_k49_f16", 32, 2, 1, 3136, 32, 49, "f16", "na1d"),
    "sasa2d_stage1_f16": Workload("sasa2d_stage1_f16", 32, 2, 56, 56, 32, 7, "f16", "sasa2d"),
    "na3d_16x56x56_k5_f16": Workload("na3d_16x56x56_k5_f16", 2, 2, 56, 56, 32, 5, "f16", "na3d",
                                     16),
}

BENCH_WORKLOAD = "nat_tiny_stage1_f16"


@dataclasses.dataclass
class Inputs:
    q: torch.Tensor      # storage dtype, CPU
    k: torch.Tensor
    v: torch.Tensor
    rpb: torch.Tensor    # float32, CPU
    q64: np.ndarray      # the same values widened to float64
    k64: np.ndarray
    v64: np.ndarray
    rpb64: np.ndarray


def _round(a: np.ndarray, dtype: str):
    t = torch.from_numpy(a).to(DTYPES[dtype])
    return t, t.to(torch.float64).numpy()


def make_inputs(shape, ksize: int, dtype: str, seed: int = 0, rpb_std: float = 0.02,
                q_scale: float = 1.0, op: str = "na2d") -> Inputs:
    """Draw Q, K, V ~ N(0, 1) (Q optionally times q_scale) and RPB ~ N(0, rpb_std).
    `shape` is [B, heads, ..., d]; the bias table is [heads, 2k-1] per axis of `op`."""
    heads = shape[1]
    rng = np.random.default_rng(seed)
    q = rng.standard_normal(shape)
    k = rng.standard_normal(shape)
    v = rng.standard_normal(shape)
    rpb = rng.standard_normal(rpb_shape(op, heads, ksize)) * rpb_std
    if q_scale != 1.0:
        q = q * q_scale
    qt, q64 = _round(q, dtype)
    kt, k64 = _round(k, dtype)
    vt, v64 = _round(v, dtype)
    rt, r64 = _round(rpb, "f32")
    return Inputs(qt, kt, vt, rt, q64, k64, v64, r64)


def workload_inputs(w: Workload, seed: int = 0, **kw) -> Inputs:
    return make_inputs(w.shape, w.k, w.dtype, seed=seed, op=w.op, **kw)
