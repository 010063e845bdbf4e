"""Seeded synthetic inputs for the log-linear attention forward and decode.

This module only draws random numbers and lays them out.  It contains none of
the method's arithmetic (no decays, no levels, no Fenwick logic), so both the
fp64 oracle under ``oracle/`` and the HIP path can take their inputs from it.

Distributions follow the workload descriptions used throughout the project:

* q, v ~ N(0, 1); k ~ N(0, 1) then L2-normalised per token (in fp64, before
  any cast);
* log-decay a_t = -softplus(x_t) * scale with x_t ~ N(0, 1) and
  softplus(x) = max(x, 0) + log1p(exp(-|x|)); scale is 0.05, or 0.01 for the
  long-context workload so that far levels still carry mass;
* per-level weights lambda_t[l] ~ U[0, 1).

Draw order per workload is fixed: q, k, v, x_a, lambda.  Standard-normal draws
are fp64; they are cast to fp32, and bf16 tensors are the round-to-nearest-even
cast of the fp32 values (torch ``.to(torch.bfloat16)``).  a and lambda always
stay fp32.  Layout is [B, H, T, .] contiguous.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch


def num_levels(T: int) -> int:
    """Number of lambda entries per token: 1 + ceil(log2 T) (1 for T <= 1).

    This is a shape rule (how wide the lambda tensor is), the same rule the
    library's ``loglinear_num_levels`` documents.
    """
    if T <= 1:
        return 1
    return 1 + (T - 1).bit_length()


@dataclass(frozen=True)
class FwdConfig:
    name: str
    B: int
    H: int
    T: int
    dk: int
    dv: int
    chunk: int
    dtype: str  # "f32" or "bf16"
    a_scale: float = 0.05
    seed: int = 0

    @property
    def L(self) -> int:
        return num_levels(self.T)

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16


@dataclass(frozen=True)
class DecodeConfig:
    name: str
    S: int
    H: int
    dk: int
    dv: int
    Lcap: int
    max_pos: int
    dtype: str = "bf16"
    a_scale: float = 0.05
    seed: int = 0

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16


# The five workloads: a tiny fp32 case, the 2K/16K/64K bf16 forwards and the
# batched decode.  Seeds are 1000 + index.
WORKLOADS = {
    "tiny_f32_T256": FwdConfig("tiny_f32_T256", 1, 1, 256, 16, 16, 16, "f32", 0.05, 1000),
    "fwd_bf16_T2K": FwdConfig("fwd_bf16_T2K", 2, 8, 2048, 128, 64, 64, "bf16", 0.05, 1001),
    "fwd_bf16_T16K": FwdConfig("fwd_bf16_T16K", 1, 16, 16384, 128, 64, 64, "bf16", 0.05, 1002),
    # Log-Linear Gated DeltaNet forward at the same shape, float32
    "gdn_f32_T16K": FwdConfig("gdn_f32_T16K", 1, 16, 16384, 128, 64, 64, "f32", 0.05, 1005),
    "fwd_bf16_T64K": FwdConfig("fwd_bf16_T64K", 1, 8, 65536, 128, 64, 64, "bf16", 0.01, 1003),
    "decode_bf16_S64": DecodeConfig("decode_bf16_S64", 64, 16, 128, 64, 17, 32768, "bf16", 0.05, 1004),
}


def _softplus(x: np.ndarray) -> np.ndarray:
    return np.maximum(x, 0.0) + np.log1p(np.exp(-np.abs(x)))


def _cast(x64: np.ndarray, dtype: str) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(x64.astype(np.float32)))
    if dtype == "bf16":
        t = t.to(torch.bfloat16)
    return t.contiguous()


def _unit_rows(x: np.ndarray) -> np.ndarray:
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
    n[n == 0.0] = 1.0
    return x / n


def make_fwd_inputs(cfg: FwdConfig, T: int | None = None, seed: int | None = None):
    """Return dict(q, k, v, a, lam) as CPU torch tensors in device dtypes.

    ``T`` overrides the sequence length (used by prefix and ragged-tail tests);
    the number of lambda levels follows the overridden T.
    """
    T = cfg.T if T is None else T
    seed = cfg.seed if seed is None else seed
    B, H, dk, dv = cfg.B, cfg.H, cfg.dk, cfg.dv
    L = num_levels(T)
    rng = np.random.Generator(np.random.PCG64(seed))
    q = rng.standard_normal((B, H, T, dk))
    k = _unit_rows(rng.standard_normal((B, H, T, dk)))
    v = rng.standard_normal((B, H, T, dv))
    xa = rng.standard_normal((B, H, T))
    lam = rng.random((B, H, T, L))
    a = -_softplus(xa) * cfg.a_scale
    return {
        "q": _cast(q, cfg.dtype),
        "k": _cast(k, cfg.dtype),
        "v": _cast(v, cfg.dtype),
        "a": torch.from_numpy(a.astype(np.float32)).contiguous(),
        "lam": torch.from_numpy(lam.astype(np.float32)).contiguous(),
    }


def make_gdn_inputs(cfg: FwdConfig, T: int | None = None, seed: int | None = None):
    """Inputs of the Log-Linear Gated DeltaNet forward, float32 CPU tensors:
    q and k unit-norm rows (Gated DeltaNet normalises both), v ~ N(0, 1),
    beta = sigmoid(N(0, 1)), a = -softplus(N(0, 1)) * a_scale,
    lambda ~ U[0, 1).  Returns dict(q, k, v, a, beta, lam)."""
    T = cfg.T if T is None else T
    seed = cfg.seed if seed is None else seed
    B, H, dk, dv = cfg.B, cfg.H, cfg.dk, cfg.dv
    L = num_levels(T)
    rng = np.random.Generator(np.random.PCG64(seed))
    q = _unit_rows(rng.standard_normal((B, H, T, dk)))
    k = _unit_rows(rng.standard_normal((B, H, T, dk)))
    v = rng.standard_normal((B, H, T, dv))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((B, H, T))))
    a = -_softplus(rng.standard_normal((B, H, T))) * cfg.a_scale
    lam = rng.random((B, H, T, L))
    f = lambda x: torch.from_numpy(x.astype(np.float32)).contiguous()
    return {"q": f(q), "k": f(k), "v": f(v), "a": f(a), "beta": f(beta), "lam": f(lam)}


def make_decode_inputs(cfg: DecodeConfig, seed: int | None = None, positions=None):
    """Return dict(q, k, v, a, lam, state, logscale, pos) for one decode step.

    Positions (0-indexed position of the new token) are drawn from
    U{1..max_pos} unless given.  Every one of the Lcap stack slots of every
    (sequence, head) is filled with a seeded sum of m decayed rank-one terms
    sum_j exp(-0.04 j) k_j v_j^T (k_j unit-norm, v_j ~ N(0,1)), with m = 1 for
    slot 0 and m = min(2^(slot-1), 64) above; computed in fp64, stored fp32.
    Which slots a step reads is the kernel's business, not the generator's.
    logscale starts at 0.
    """
    seed = cfg.seed if seed is None else seed
    S, H, dk, dv, Lc = cfg.S, cfg.H, cfg.dk, cfg.dv, cfg.Lcap
    rng = np.random.Generator(np.random.PCG64(seed))
    if positions is None:
        pos = rng.integers(1, cfg.max_pos + 1, size=S, dtype=np.int64)
    else:
        pos = np.asarray(positions, dtype=np.int64).reshape(S)
    q = rng.standard_normal((S, H, dk))
    k = _unit_rows(rng.standard_normal((S, H, dk)))
    v = rng.standard_normal((S, H, dv))
    xa = rng.standard_normal((S, H))
    lam = rng.random((S, H, Lc))
    a = -_softplus(xa) * cfg.a_scale
    state = np.empty((S, H, Lc, dk, dv), dtype=np.float32)
    for slot in range(Lc):
        m = 1 if slot == 0 else min(2 ** (slot - 1), 64)
        w = np.exp(-0.04 * np.arange(m))
        kk = _unit_rows(rng.standard_normal((S, H, m, dk)))
        vv = rng.standard_normal((S, H, m, dv))
        state[:, :, slot] = np.matmul(np.swapaxes(kk * w[None, None, :, None], -1, -2), vv).astype(np.float32)
    return {
        "q": _cast(q, cfg.dtype),
        "k": _cast(k, cfg.dtype),
        "v": _cast(v, cfg.dtype),
        "a": torch.from_numpy(a.astype(np.float32)).contiguous(),
        "lam": torch.from_numpy(lam.astype(np.float32)).contiguous(),
        "state": torch.from_numpy(state).contiguous(),
        "logscale": torch.zeros((S, H, Lc), dtype=torch.float32),
        "pos": torch.from_numpy(pos).contiguous(),
    }


def sample_rows(B: int, H: int, T: int, chunk: int, per_head: int, seed: int):
    """Seeded row sample for full-size parity: per (b, h), ``per_head`` random
    positions plus every row of the first, one middle and the last chunk.
    Returns an int64 array of shape [n, 2] holding (b*H + h, t)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    n_chunks = (T + chunk - 1) // chunk
    fixed = set()
    for c in (0, n_chunks // 2, n_chunks - 1):
        for t in range(c * chunk, min(T, (c + 1) * chunk)):
            fixed.add(t)
    out = []
    for bh in range(B * H):
        rows = set(fixed)
        rows.update(int(x) for x in rng.integers(0, T, size=per_head))
        out.extend((bh, t) for t in sorted(rows))
    return np.asarray(out, dtype=np.int64)


def to_f64(t: torch.Tensor) -> np.ndarray:
    """Exact upcast of a device-dtype CPU tensor (fp32 or bf16) to fp64."""
    return t.detach().to(torch.float64).cpu().numpy()
