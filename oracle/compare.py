"""Parity comparators (oracle side).

TEST INFRASTRUCTURE ONLY -- see the package docstring.

* Expert ids: exact, except at routing near-ties, where either expert may be
  picked when their logits are within 1e-5 of the top-k boundary.  [Reading:
  a device selection is accepted when every chosen expert's float64 logit is
  >= tau - 1e-5 and every expert left out has a logit <= tau + 1e-5, tau
  being the oracle's k-th largest logit, and the chosen list is in
  non-increasing logit order up to 1e-5.]
* Floating-point outputs: per element |y - yref| / max(|yref|, rms_t(yref)),
  rms over the token's row, against the relative tolerance 1e-2.  [Reading:
  a plain element-wise relative error is undefined at cancellation zeros.]
* Any NaN or infinity where the reference is finite is a failure.
"""
from __future__ import annotations

import numpy as np

TIE_TOL = 1e-5


def valid_selection(sel: np.ndarray, logits64: np.ndarray, k: int, tol: float = TIE_TOL) -> bool:
    """Is ``sel`` (k expert ids, in the device's order) a valid top-k of
    ``logits64`` (one token) under the tie rule?"""
    sel = np.asarray(sel, dtype=np.int64)
    E = logits64.size
    if sel.size != k or np.any(sel < 0) or np.any(sel >= E) or np.unique(sel).size != k:
        return False
    tau = np.sort(logits64)[::-1][k - 1]
    chosen = np.zeros(E, dtype=bool)
    chosen[sel] = True
    if np.any(logits64[chosen] < tau - tol):
        return False
    if np.any(logits64[~chosen] > tau + tol):
        return False
    ls = logits64[sel]
    return bool(np.all(ls[1:] <= ls[:-1] + tol))


def compare_ids(dev_ids: np.ndarray, ref_ids: np.ndarray, logits64: np.ndarray):
    """Returns (n_exact, n_tie_accepted, bad_tokens)."""
    dev_ids = np.asarray(dev_ids, dtype=np.int64)
    ref_ids = np.asarray(ref_ids, dtype=np.int64)
    T, k = ref_ids.shape
    exact = 0
    ties = 0
    bad = []
    for t in range(T):
        if np.array_equal(dev_ids[t], ref_ids[t]):
            exact += 1
        elif valid_selection(dev_ids[t], logits64[t], k):
            ties += 1
        else:
            bad.append(t)
    return exact, ties, bad


def rowwise_rel_error(y: np.ndarray, yref: np.ndarray) -> np.ndarray:
    """Per-element error |y - yref| / max(|yref|, rms of yref's row).
    Non-finite device values where the reference is finite give +inf."""
    y = np.asarray(y, dtype=np.float64)
    yref = np.asarray(yref, dtype=np.float64)
    yref2 = yref.reshape(-1, yref.shape[-1])
    y2 = y.reshape(yref2.shape)
    rms = np.sqrt(np.mean(yref2 * yref2, axis=1, keepdims=True))
    denom = np.maximum(np.abs(yref2), rms)
    with np.errstate(invalid="ignore", divide="ignore"):
        err = np.abs(y2 - yref2) / denom
    bad = ~np.isfinite(y2) & np.isfinite(yref2)
    err = np.where(bad, np.inf, err)
    err = np.where(np.isnan(err), np.inf, err)
    err = np.where((denom == 0) & (y2 == 0), 0.0, err)
    return err.reshape(yref.shape)


def max_rel_error(y, yref) -> float:
    e = rowwise_rel_error(y, yref)
    return float(e.max()) if e.size else 0.0


def normwise_rel_error(y, yref) -> float:
    y = np.asarray(y, dtype=np.float64)
    yref = np.asarray(yref, dtype=np.float64)
    if not np.all(np.isfinite(y)):
        return float("inf")
    n = np.linalg.norm(yref)
    return float(np.linalg.norm(y - yref) / n) if n else float(np.linalg.norm(y))


def bf16_bits_equal(a, b) -> bool:
    """Bit equality of BF16 arrays, except that any NaN matches any NaN."""
    a = np.asarray(a, dtype=np.uint16)
    b = np.asarray(b, dtype=np.uint16)
    if a.shape != b.shape:
        return False
    nan_a = ((a & 0x7F80) == 0x7F80) & ((a & 0x7F) != 0)
    nan_b = ((b & 0x7F80) == 0x7F80) & ((b & 0x7F) != 0)
    if not np.array_equal(nan_a, nan_b):
        return False
    return bool(np.array_equal(a[~nan_a], b[~nan_b]))
