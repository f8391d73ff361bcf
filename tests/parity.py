"""Parity gate between a GPU bf16 result and the fp64 oracle.

Gate (the reading of "max-abs 2e-2 and max-rel 1e-2" used throughout):
  * every value is finite;
  * max over all elements |g - r| <= 2e-2;
  * for every output row (one (token, q head) vector of D values)
        max_d |g - r| <= 1e-2 * max_d |r|;
  * rows whose oracle value is exactly zero are exactly zero.
The row-relative bound keeps the gate meaningful where outputs are small (long contexts average
many values toward zero, so an absolute bound alone would accept an all-zero answer).
"""
import numpy as np
import torch

ATOL = 2e-2
ROW_RTOL = 1e-2


def to_f64(x) -> np.ndarray:
    if isinstance(x, torch.Tensor):
        return x.detach().to("cpu").to(torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def parity_stats(got, ref) -> dict:
    g = to_f64(got)
    r = to_f64(ref)
    assert g.shape == r.shape, (g.shape, r.shape)
    D = g.shape[-1]
    g2, r2 = g.reshape(-1, D), r.reshape(-1, D)
    err = np.abs(g2 - r2)
    row_err = err.max(axis=1) if err.size else np.zeros(0)
    row_scale = np.abs(r2).max(axis=1) if r2.size else np.zeros(0)
    zero_rows = row_scale == 0
    nz = ~zero_rows
    rel = row_err[nz] / row_scale[nz] if nz.any() else np.zeros(0)
    dot = (g2 * r2).sum(1)
    cos = dot[nz] / (np.linalg.norm(g2[nz], axis=1) * np.linalg.norm(r2[nz], axis=1) + 1e-300) if nz.any() else np.ones(1)
    return {
        "finite": bool(np.isfinite(g).all()),
        "max_abs": float(err.max()) if err.size else 0.0,
        "max_row_rel": float(rel.max()) if rel.size else 0.0,
        "zero_rows_exact": bool((g2[zero_rows] == 0).all()),
        "worst_row_cos": float(cos.min()) if cos.size else 1.0,
        "elem_rel_floor": float((err / (np.abs(r2) + 1e-3)).max()) if err.size else 0.0,
        "rows": int(g2.shape[0]),
    }


def assert_parity(got, ref, what: str = "") -> dict:
    s = parity_stats(got, ref)
    msg = f"{what}: {s}"
    assert s["finite"], msg
    assert s["max_abs"] <= ATOL, msg
    assert s["max_row_rel"] <= ROW_RTOL, msg
    assert s["zero_rows_exact"], msg
    return s
