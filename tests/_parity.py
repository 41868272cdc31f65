"""Parity metric between the HIP path and the float64 oracle.

An element passes iff |g - o| <= rtol * s + ulp_T(o) / 2, where
  * o is the oracle value and s >= |o| the oracle's magnitude ("scale") of the
    same element: the same loops run on absolute values, so s measures the
    size of the terms whose rounding a correct float32 kernel is exposed to;
  * rtol is 1e-5 for float32 I/O and 3e-3 for float16 / bfloat16 I/O;
  * ulp_T(o) / 2 is the rounding of the stored result to its own dtype T
    (one bfloat16 rounding alone can exceed 3e-3 relative).
NaN or inf on either side fails.  Also reports the largest error relative to
|o| over elements with |o| > 1e-3 max|o| and the normwise error.
"""
from __future__ import annotations

import numpy as np

RTOL = {"f32": 1e-5, "f16": 3e-3, "bf16": 3e-3}
# every check's statistics, in order (written out at the end of a test session
# when SSM_PARITY_STATS names a file; see tests/conftest.py)
RECORD = []
_MANT_EMIN = {"f32": (23, -126), "f16": (10, -14), "bf16": (7, -126)}


def to_f64(a):
    import torch

    if isinstance(a, torch.Tensor):
        a = a.detach().cpu()
        if a.dtype in (torch.float16, torch.bfloat16):
            a = a.to(torch.float32)
        return a.numpy().astype(np.float64)
    return np.asarray(a, dtype=np.float64)


def half_ulp(o, dtype: str) -> np.ndarray:
    mant, emin = _MANT_EMIN[dtype]
    a = np.abs(np.asarray(o, dtype=np.float64))
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(e, emin)
    return 0.5 * np.exp2(e - mant)


def check(got, want, scale, rtol: float, dtype: str, what: str) -> dict:
    g = to_f64(got)
    o = np.asarray(want, dtype=np.float64)
    s = np.asarray(scale, dtype=np.float64)
    if g.shape != o.shape:
        g = g.reshape(o.shape)
    err = np.abs(g - o)
    tol = rtol * s + half_ulp(o, dtype)
    ok = np.isfinite(g) & np.isfinite(o) & (err <= tol)
    mx = np.max(np.abs(o)) if o.size else 0.0
    big = np.abs(o) > 1e-3 * mx
    stats = {
        "n": int(o.size),
        "max_err_over_tol": float(np.max(np.where(np.isfinite(err), err / np.maximum(tol, 1e-300), np.inf)))
        if o.size else 0.0,
        "max_rel": float(np.max(err[big] / np.abs(o[big]))) if big.any() else 0.0,
        "normwise": float(np.linalg.norm(g - o) / max(np.linalg.norm(o), 1e-300)) if o.size else 0.0,
    }
    RECORD.append({"what": what, "dtype": dtype, "rtol": rtol, **stats})
    if not ok.all():
        bad = np.argwhere(~ok)
        lines = []
        for ix in bad[:8]:
            ix = tuple(int(i) for i in ix)
            lines.append(f"  at {ix}: got {g[ix]!r} want {o[ix]!r} scale {s[ix]:.3e} tol {tol[ix]:.3e}")
        raise AssertionError(
            f"{what}: {len(bad)}/{o.size} elements outside |g-o| <= {rtol:g}*s + ulp_{dtype}/2 "
            f"(stats {stats})\n" + "\n".join(lines))
    return stats
