"""Helpers shared by the GPU parity tests: device upload in the storage type and
the per-row relative error used as the parity gate."""
from __future__ import annotations

import numpy as np
import torch

from linear_rnn_layers_amd import inputs

TOL = {inputs.F32: 1e-4, inputs.BF16: 2e-2}  # the stated parity tolerances
TORCH_DT = {inputs.F32: torch.float32, inputs.BF16: torch.bfloat16}


def dev(x: np.ndarray, dtype: str = inputs.F32) -> torch.Tensor:
    """Upload float32 values (exactly representable in `dtype`) as `dtype`."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to("cuda")
    return t.to(TORCH_DT[dtype]).contiguous()


def dev32(x) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to("cuda")


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def rowerr(x, y, row_axis_len: bool = True, row_floor=None) -> float:
    """max over rows r of ||x_r - y_r||_inf / max(||y_r||_inf, 1e-3 * max_{r' in same (b,h)} ||y_r'||_inf).

    A row is the last axis (one token's vector, one state row); for arrays
    whose rows are scalars (den) pass row_axis_len=False.  The floor only
    neutralises rows that are exactly zero by construction.  `row_floor`, if
    given (one value per row), raises each row's denominator further; it is
    used for rows that are a cancellation of larger terms."""
    x = np.asarray(x, dtype=np.float64)
    y = np.asarray(y, dtype=np.float64)
    if not row_axis_len:
        x = x[..., None]
        y = y[..., None]
    if x.shape != y.shape:
        raise ValueError(f"shape mismatch {x.shape} vs {y.shape}")
    if y.size == 0:
        return 0.0
    if not np.all(np.isfinite(x)):
        return float("inf")
    diff = np.abs(x - y).max(axis=-1)
    ynorm = np.abs(y).max(axis=-1)
    B, H = y.shape[:2]
    floor = 1e-3 * ynorm.reshape(B, H, -1).max(axis=-1)
    floor = floor.reshape((B, H) + (1,) * (ynorm.ndim - 2))
    denom = np.maximum(ynorm, floor)
    if row_floor is not None:
        denom = np.maximum(denom, np.asarray(row_floor, dtype=np.float64).reshape(denom.shape))
    ratio = np.where(denom > 0, diff / np.where(denom > 0, denom, 1.0), diff)
    return float(ratio.max())
