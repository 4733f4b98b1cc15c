"""Parity metrics between a result and the oracle -- TEST INFRASTRUCTURE ONLY.

The bar: per element |got - ref| <= 2e-3 + 1e-2 * |ref|, and the cosine
similarity of every token's row >= 0.999995, for h and for y.  (The blog
post, "Hardware efficiency", reports a minimum cosine above 0.999996 and a
maximum absolute difference of 0.001953 against its reference
implementation; the bar here is a per-element bound of that size plus a
relative term for large values.)
"""
from __future__ import annotations

import numpy as np

ATOL = 2e-3
RTOL = 1e-2
MIN_COS = 0.999995


def bf16_to_f64(bits):
    u = np.asarray(bits).astype(np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def parity(got_bits, ref_bits, rows: int):
    """Compare two bf16 tensors (bit patterns) reshaped to [rows, -1].

    Returns a dict with max |diff|, the worst bound ratio (<= 1 passes), min
    per-row cosine, count of differing elements and NaN counts."""
    g = bf16_to_f64(got_bits).reshape(rows, -1)
    r = bf16_to_f64(ref_bits).reshape(rows, -1)
    nan_g, nan_r = int(np.isnan(g).sum()), int(np.isnan(r).sum())
    d = np.abs(g - r)
    ratio = d / (ATOL + RTOL * np.abs(r))
    num = (g * r).sum(1)
    den = np.sqrt((g * g).sum(1) * (r * r).sum(1))
    cos = np.where(den > 0, num / np.where(den > 0, den, 1), np.where((g == r).all(1), 1.0, 0.0))
    return dict(
        max_abs=float(np.nanmax(d)) if d.size else 0.0,
        worst_ratio=float(np.nanmax(ratio)) if d.size else 0.0,
        min_cos=float(cos.min()) if cos.size else 1.0,
        n_diff=int((np.asarray(got_bits) != np.asarray(ref_bits)).sum()),
        n=int(g.size),
        nan_got=nan_g,
        nan_ref=nan_r,
    )


def passes(p) -> bool:
    return p["nan_got"] == p["nan_ref"] == 0 and p["worst_ratio"] <= 1.0 and p["min_cos"] >= MIN_COS
