"""Seeded random tensors, stored as bf16 bit patterns (numpy uint16).

Recipe for a tensor of shape (R, C) (a vector is one row):
  * rows are drawn in blocks of ``rows_per_block(C)`` rows; block ``b`` comes
    from its own numpy sub-stream ``default_rng([seed, tensor_id, b])`` as fp32
    standard normals, so any block can be regenerated alone and blocks can be
    drawn in parallel;
  * scale and offset are applied in fp32;
  * outliers, if asked for, are exactly floor(frac * R * C) distinct flat
    positions drawn without replacement from the sub-stream
    ``default_rng([seed, tensor_id, OUTLIER_STREAM])``; their fp32 sample is
    multiplied by the outlier factor;
  * the result is rounded to bf16 exactly once (torch's CPU cast, round to
    nearest even).
"""

from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

OUTLIER_STREAM = 0x0F17
BLOCK_ELEMS = 1 << 20


def rows_per_block(cols: int) -> int:
    return max(1, BLOCK_ELEMS // max(1, int(cols)))


def bf16_bits_from_f32(a: np.ndarray) -> np.ndarray:
    """fp32 array -> bf16 bit patterns (uint16), rounded by torch's CPU cast."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _outlier_positions(n: int, seed: int, tensor_id: int, frac: float) -> np.ndarray:
    k = int(math.floor(frac * n))
    if k <= 0:
        return np.zeros(0, dtype=np.int64)
    rng = np.random.default_rng([int(seed), int(tensor_id), OUTLIER_STREAM])
    return np.sort(rng.choice(n, size=k, replace=False).astype(np.int64))


def normal_bf16(shape, seed: int, tensor_id: int, mean: float = 0.0,
                std: float = 1.0, outlier_frac: float = 0.0,
                outlier_mult: float = 50.0, rows=None) -> np.ndarray:
    """bf16 tensor ~ mean + std * N(0, 1), with optional outliers.

    ``rows`` (optional, sorted or not) selects a subset of rows to return, in
    the given order; only the blocks holding them are drawn.  The values are
    the same as in the full tensor.
    """
    shape = tuple(int(s) for s in shape)
    if len(shape) == 1:
        R, C = 1, shape[0]
    elif len(shape) == 2:
        R, C = shape
    else:
        raise ValueError("1-D or 2-D shapes only")
    rpb = rows_per_block(C)
    sel = np.arange(R, dtype=np.int64) if rows is None else np.asarray(rows, dtype=np.int64)
    out = np.empty((len(sel), C), dtype=np.float32)
    blocks = np.unique(sel // rpb) if len(sel) else np.zeros(0, dtype=np.int64)

    def draw(b):
        r0 = int(b) * rpb
        r1 = min(R, r0 + rpb)
        rng = np.random.default_rng([int(seed), int(tensor_id), int(b)])
        blk = rng.standard_normal((r1 - r0) * C, dtype=np.float32).reshape(r1 - r0, C)
        m = (sel >= r0) & (sel < r1)
        out[m] = blk[sel[m] - r0]

    if len(blocks) > 1:
        with ThreadPoolExecutor(_workers()) as ex:
            list(ex.map(draw, blocks))
    else:
        for b in blocks:
            draw(b)
    if std != 1.0:
        out *= np.float32(std)
    if mean != 0.0:
        out += np.float32(mean)
    if outlier_frac > 0.0:
        pos = _outlier_positions(R * C, seed, tensor_id, outlier_frac)
        prow, pcol = pos // C, pos % C
        if rows is None:
            out[prow, pcol] *= np.float32(outlier_mult)
        else:
            for i, r in enumerate(sel):
                lo, hi = np.searchsorted(prow, [r, r + 1])
                if hi > lo:
                    out[i, pcol[lo:hi]] *= np.float32(outlier_mult)
    res = bf16_bits_from_f32(out)
    if rows is None and len(shape) == 1:
        return res.reshape(shape)
    return res.reshape((len(sel), C)) if rows is not None else res.reshape(shape)


def uniform_f32(shape, seed: int, tensor_id: int, low: float, high: float) -> np.ndarray:
    """fp32 tensor ~ U[low, high) from its own sub-stream (used for scales)."""
    rng = np.random.default_rng([int(seed), int(tensor_id)])
    return rng.uniform(low, high, size=tuple(shape)).astype(np.float32)
