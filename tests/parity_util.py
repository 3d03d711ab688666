"""Shared helpers of the GPU parity tests: tolerances and comparisons, and
oracle evaluations restricted to selected rows (built from the oracle's own
functions, for full-size workloads where a whole document would be slow)."""
from __future__ import annotations

import math
from typing import Sequence

import numpy as np
import torch

import oracle as O

# Attention-output tolerances: max-abs bar per dtype, plus a per-row
# relative check ||o - o_ref|| / ||o_ref|| so that long rows with tiny
# outputs keep teeth.
TOL = {"bf16": (2e-2, 1e-2), "f32": (1e-5, 1e-5)}


def np32(t: torch.Tensor) -> np.ndarray:
    return t.detach().to(torch.float32).cpu().numpy()


def assert_close(got: np.ndarray, ref: np.ndarray, dtype: str, what: str) -> None:
    atol, rel = TOL[dtype]
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite values"
    err = np.abs(got - ref)
    mx = float(err.max()) if err.size else 0.0
    assert mx <= atol, f"{what}: max abs err {mx:.3e} > {atol}"
    num = np.linalg.norm((got - ref).reshape(-1, ref.shape[-1]), axis=1)
    den = np.linalg.norm(ref.reshape(-1, ref.shape[-1]), axis=1)
    r = num / np.maximum(den, 1e-30)
    assert float(r.max()) <= rel, f"{what}: row-relative err {float(r.max()):.3e} > {rel}"


def assert_lse_close(got: np.ndarray, ref: np.ndarray, dtype: str, what: str) -> None:
    tol = 2e-2 if dtype == "bf16" else 2e-5
    err = np.abs(np.asarray(got, np.float64) - np.asarray(ref, np.float64))
    assert float(err.max()) <= tol, f"{what}: lse max abs err {float(err.max()):.3e}"


def bf16_ulp_diff(a: np.ndarray, b: np.ndarray) -> int:
    """Largest distance in bf16 units in the last place between two arrays
    of bf16-representable fp32 values (ordered-integer metric)."""
    def key(x):
        u = np.ascontiguousarray(x, dtype=np.float32).view(np.int32).astype(np.int64) >> 16
        return np.where(u < 0, -(u & 0x7FFF), u)
    return int(np.abs(key(a) - key(b)).max()) if a.size else 0


def assert_rotated_close(got: np.ndarray, ref: np.ndarray, pre: np.ndarray, dtype: str, what: str) -> None:
    """Composed/appended keys against the oracle.  Both sides rotate the same
    fp32 angle, but their cos/sin may differ by a few fp32 ulp, and the
    rotation x_i c - x_{i+d/2} s can cancel; so the fp32 results may differ by
    up to (|x_i| + |x_{i+d/2}|) 2^-21 (four ulp of 1 per factor, with rounding
    of the products), and after rounding to bf16 by that plus one bf16 ulp of
    the larger result."""
    got = np.asarray(got, np.float32)
    ref = np.asarray(ref, np.float32)
    d = pre.shape[-1]
    h = d // 2
    b = np.abs(pre[..., :h]).astype(np.float64) + np.abs(pre[..., h:])
    bound = np.concatenate([b, b], axis=-1) * 2.0 ** -21
    if dtype == "bf16":
        mag = np.maximum(np.abs(got), np.abs(ref)).astype(np.float64)
        e = np.floor(np.log2(np.maximum(mag, 1e-38)))
        bound = bound + 2.0 ** (e - 7)
    err = np.abs(got.astype(np.float64) - ref)
    bad = err > bound + 1e-30
    assert not bad.any(), (f"{what}: {int(bad.sum())} of {bad.size} elements outside the rotation bound; "
                           f"max err {float(err.max()):.3e}; max bf16-ulp distance {bf16_ulp_diff(got, ref)}")


def oracle_extract_rows(q, k, v, n: int, ratio_k: int, sink, theta: float, rows: Sequence[int],
                        anchor: bool = False):
    """Oracle extraction outputs of selected packed rows of ONE document
    (q/k/v: that document's packed [n | m] rows as numpy).  Uses the oracle's
    rotation, structured mask (the anchor ablation's with anchor=True) and
    attention on the selected query rows."""
    pos = O.extraction_positions(n, ratio_k)
    rows = np.asarray(rows)
    qr = O.rope_rotate(np.asarray(q[rows], np.float32), pos[rows], theta)
    kr = O.rope_rotate(np.asarray(k, np.float32), pos, theta)
    M = O.structured_mask(n, ratio_k, sink, anchor)[rows]
    return O.attention(qr, kr, np.asarray(v, np.float64), M)
