"""Helpers shared by the GPU parity tests, the smoke check and the bench:
moving stored inputs to the device and the row-scaled parity metric.

Tolerance (per output element (b, h, i, c)):
    err = |y_gpu - y_ref| / scale,
    scale = (sum_j |w_ij| |vop_jc| + |y_ic| sum_j |w_ij|) / |den_i|   (oracle),
and a run passes if the maximum over all elements is <= tol (1e-4 for fp32
inputs, 2e-2 for bf16 inputs with fp32 accumulation).  scale is the
first-order rounding-error bound of the quotient y = num / den divided by the
unit roundoff, so eps-accurate sums give err ~ eps on every row, including the
order-1 rows whose normaliser nearly cancels (there |y| and sum|w|/|den| are
both large).  At order 2 all weights are >= 0 and scale is the weighted mean of
|vop| plus |y|, i.e. a relative error on every row.

The decode step evaluates the state form of Algorithm 6, y = phi(q)^T S /
phi(q)^T z, whose sums run over the feature products; its tests use the
oracle's scale_state, the same bound with (sum_a |q_ia||k_ja|)^p in place of
|q_i . k_j|^p (equal to scale when no feature product cancels).
"""
from __future__ import annotations

import numpy as np

from mamba_ssd_sequence_amd import inputs as I

TOL = {I.F32: 1e-4, I.BF16: 2e-2}


def to_dev_qkv(x: np.ndarray, dtype: str, device="cuda"):
    import torch
    if dtype == I.BF16:
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(device)


def to_dev_f32(x: np.ndarray, device="cuda"):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(device)


def row_error(y_gpu: np.ndarray, y_ref: np.ndarray, scale: np.ndarray) -> float:
    """max over elements of |y_gpu - y_ref| / scale (NaN anywhere -> inf)."""
    d = np.abs(np.asarray(y_gpu, np.float64) - y_ref) / scale
    if not np.all(np.isfinite(d)):
        return float("inf")
    return float(d.max()) if d.size else 0.0


def sample_rows(N: int, n_random: int, rng: np.random.Generator, block: int = 64,
                boundaries: bool = True) -> np.ndarray:
    """First and last `block` rows, every block boundary +-1 over the whole
    sequence (if `boundaries`), and `n_random` random rows."""
    s = set(range(min(N, block))) | set(range(max(0, N - block), N))
    if boundaries:
        for b in range(block, N, block):
            s.update((b - 1, b, b + 1))
    s.update(rng.integers(0, N, size=n_random).tolist())
    return np.array(sorted(x for x in s if 0 <= x < N), dtype=np.int64)


def worst(y_gpu: np.ndarray, y_ref: np.ndarray, scale: np.ndarray, rows=None) -> str:
    """Where the largest scaled error sits: (b, h, token, column) and its value."""
    d = np.abs(np.asarray(y_gpu, np.float64) - y_ref) / scale
    if d.size == 0:
        return "empty"
    d = np.where(np.isfinite(d), d, np.inf)
    b, h, r, c = np.unravel_index(int(np.argmax(d)), d.shape)
    tok = r if rows is None else int(rows[r])
    return f"max err {d[b, h, r, c]:.3e} at (b={b}, h={h}, token={tok}, col={c})"
