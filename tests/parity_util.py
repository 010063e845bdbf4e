"""Helpers for GPU parity tests: device placement, error metrics, tolerances.

Tolerances (relative L2 error, fp64, over the whole output and per head):
  float32 inputs, float32 accumulation:  1e-4
  bfloat16 inputs, float32 accumulation: 2e-2
"""

import numpy as np
import torch

TOL = {"f32": 1e-4, "bf16": 2e-2}


def to_dev(d: dict) -> dict:
    return {k: v.cuda() for k, v in d.items()}


def rel_l2(x: np.ndarray, ref: np.ndarray) -> float:
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref.ravel())
    num = np.linalg.norm((x - ref).ravel())
    return float(num / den) if den > 0 else float(num)


def per_head_max(x: np.ndarray, ref: np.ndarray) -> float:
    """Max over (b, h) of the relative L2 error; x, ref are [B,H,...]."""
    B, H = ref.shape[:2]
    return max(rel_l2(x[b, h], ref[b, h]) for b in range(B) for h in range(H))


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to(torch.float64).cpu().numpy()


def announce(msg: str) -> None:
    print(f"[case] {msg}", flush=True)
