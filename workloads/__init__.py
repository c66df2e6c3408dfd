"""Seeded synthetic inputs of the causal-dot-product workloads.

Shared by the tests, the benchmark and the smoke check, on both sides of a
parity comparison.  It holds no arithmetic of the method itself: it draws
normal variates, shapes them into the input distributions of the workloads
and rounds them to the I/O precision.

Input recipe (the same for every workload):
  * ``numpy.random.default_rng(seed)`` (PCG64) draws, in this order and in
    float64, x_Q, x_K (N*H*L*E each), V, then dO (N*H*L*M each) from
    N(0, 1); V and dO are then scaled by their standard deviation.
  * For the causal-product workloads the queries and keys are the positive
    values elu(x) + 1 (elu with alpha = 1), formed here in float64 as part of
    the input distribution; the linear-attention workload passes the raw x
    and its feature map is applied inside the operation.
  * Every tensor is rounded to fp32 and, for bf16 workloads, further to bf16
    with round-to-nearest-even.  The arrays returned are float32 whose values
    are exactly the values the device receives.
"""
from __future__ import annotations

from dataclasses import dataclass, replace

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    op: str            # "fwd", "fwd+bwd" or "linattn"
    dtype: str         # "f32", "bf16" or "f16"
    N: int
    H: int
    L: int
    E: int
    M: int
    seed: int
    qk: str = "elu1"   # "elu1": Q, K = elu(x) + 1;  "raw": Q, K = x
    v_std: float = 1.0
    do_std: float = 1.0

    @property
    def slices(self) -> int:
        return self.N * self.H

    @property
    def token_heads(self) -> int:
        return self.N * self.H * self.L

    def with_shape(self, **kw) -> "Workload":
        return replace(self, **kw)


# The workloads: a tiny fp32 forward, an fp32 forward, the bf16
# forward+backward at L=4096 E=M=64 (the headline), bf16 normalised linear
# attention at L=16384 E=M=128, an fp32 forward+backward with E != M, and the
# normalised form's forward+backward in bf16 at the headline shape; the
# headline shape in fp16 and with 80-wide heads; the forward+backward of the
# causal product and of the normalised form at the normalised workload's
# few-slice long-row shape.
WORKLOADS = {
    w.name: w
    for w in (
        Workload("fwd_f32_l64_e16", "fwd", "f32", 1, 1, 64, 16, 16, seed=0),
        Workload("fwd_f32_l1024_e64", "fwd", "f32", 4, 8, 1024, 64, 64, seed=1),
        Workload("fwdbwd_bf16_l4096_e64", "fwd+bwd", "bf16", 8, 16, 4096, 64, 64, seed=2),
        Workload("linattn_bf16_l16384_e128", "linattn", "bf16", 2, 8, 16384, 128, 128, seed=3,
                 qk="raw"),
        Workload("fwdbwd_f32_l2048_e32_m128", "fwd+bwd", "f32", 16, 12, 2048, 32, 128, seed=4,
                 v_std=0.5, do_std=0.5),
        # the normalised form's forward and backward at the headline shape
        Workload("linattn_fwdbwd_bf16_l4096_e64", "linattn+bwd", "bf16", 8, 16, 4096, 64, 64, seed=5,
                 qk="raw"),
        # the headline shape in fp16, and with 80-wide heads (run on 128-wide tiles)
        Workload("fwdbwd_f16_l4096_e64", "fwd+bwd", "f16", 8, 16, 4096, 64, 64, seed=6),
        Workload("fwdbwd_bf16_l4096_e80", "fwd+bwd", "bf16", 8, 16, 4096, 80, 80, seed=7),
        # few slices over long rows (16 slices of 16384 rows, 128-wide heads):
        # forward and backward both run over sequence segments
        Workload("fwdbwd_bf16_l16384_e128", "fwd+bwd", "bf16", 2, 8, 16384, 128, 128, seed=8),
        Workload("linattn_fwdbwd_bf16_l16384_e128", "linattn+bwd", "bf16", 2, 8, 16384, 128, 128, seed=9,
                 qk="raw"),
    )
}
HEADLINE = "fwdbwd_bf16_l4096_e64"


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even); returns float32
    holding exactly those bf16 values.  NaN stays NaN."""
    a = np.ascontiguousarray(x, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    bias = np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))
    r = ((u + bias) & np.uint64(0xFFFF0000)).astype(np.uint32)
    out = r.view(np.float32).copy()
    nan = np.isnan(a)
    if nan.any():
        out[nan] = np.nan
    return out


def to_io(x64: np.ndarray, dtype: str) -> np.ndarray:
    """float64 -> float32, then to bf16 values when dtype == "bf16", or to IEEE
    half values when dtype == "f16" (numpy's round to nearest even)."""
    x = np.asarray(x64, dtype=np.float64).astype(np.float32)
    if dtype == "bf16":
        return round_bf16(x)
    if dtype == "f16":
        return x.astype(np.float16).astype(np.float32)
    if dtype != "f32":
        raise ValueError(f"unknown dtype {dtype!r}")
    return x


def _elu1(x: np.ndarray) -> np.ndarray:
    return np.where(x > 0.0, x + 1.0, np.exp(np.minimum(x, 0.0)))


def generate(w: Workload, need_do: bool | None = None) -> dict:
    """Draw the inputs of workload ``w``.  Returns float32 arrays ``Q``, ``K``
    ([N,H,L,E]), ``V`` and, for backward workloads (or ``need_do``), ``dO``
    ([N,H,L,M])."""
    rng = np.random.default_rng(w.seed)
    qk_shape = (w.N, w.H, w.L, w.E)
    v_shape = (w.N, w.H, w.L, w.M)
    xq = rng.standard_normal(qk_shape)
    xk = rng.standard_normal(qk_shape)
    v = rng.standard_normal(v_shape) * w.v_std
    if w.qk == "elu1":
        xq, xk = _elu1(xq), _elu1(xk)
    elif w.qk != "raw":
        raise ValueError(f"unknown qk recipe {w.qk!r}")
    out = {"Q": to_io(xq, w.dtype), "K": to_io(xk, w.dtype), "V": to_io(v, w.dtype)}
    del xq, xk, v
    if need_do if need_do is not None else w.op.endswith("bwd"):
        out["dO"] = to_io(rng.standard_normal(v_shape) * w.do_std, w.dtype)
    return out


def integer_inputs(N, H, L, E, M, seed=0, lo=0, hi=2, need_do=True) -> dict:
    """Small non-negative integers drawn uniformly from [lo, hi]; with small
    L, E, M every partial sum is an integer well inside the exact range of
    fp32 and every value of moderate size is exact in bf16."""
    rng = np.random.default_rng(seed)
    d = {
        "Q": rng.integers(lo, hi + 1, size=(N, H, L, E)).astype(np.float32),
        "K": rng.integers(lo, hi + 1, size=(N, H, L, E)).astype(np.float32),
        "V": rng.integers(lo, hi + 1, size=(N, H, L, M)).astype(np.float32),
    }
    if need_do:
        d["dO"] = rng.integers(lo, hi + 1, size=(N, H, L, M)).astype(np.float32)
    return d


def onehot_inputs(N, H, L, E, M, seed=0, need_do=True) -> dict:
    """Q and K rows with a single 1 at a random feature, V (and dO) in {0, 1}.
    Every state entry counts the rows that hit one feature (about L / E of
    them), so long sequences keep states, scores and every partial sum small
    integers: exact in fp32 and, as operands, in bf16."""
    rng = np.random.default_rng(seed)

    def onehot(n):
        x = np.zeros((N, H, L, n), dtype=np.float32)
        np.put_along_axis(x, rng.integers(0, n, size=(N, H, L, 1)), 1.0, axis=-1)
        return x

    d = {"Q": onehot(E), "K": onehot(E), "V": rng.integers(0, 2, size=(N, H, L, M)).astype(np.float32)}
    if need_do:
        d["dO"] = rng.integers(0, 2, size=(N, H, L, M)).astype(np.float32)
    return d
