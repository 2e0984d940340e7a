"""Shared test helpers: the oracle view of a seeded workload, golden fixtures,
and the parity metrics and bound used by every fold comparison."""
from __future__ import annotations

import json
import math
import os

import numpy as np

from oracle.case import OracleView, oracle_addr, to_f64  # noqa: F401

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")

# Tolerance for the bf16-in / fp32-accumulate fold against the fp64 oracle.
REL_L2_TOL = 2e-3
MAX_ABS_TOL = 3e-2

# Arithmetic model of the fold's evaluation error (the max-abs reading):
U32 = 2.0 ** -24    # fp32 unit roundoff
HILO = 2.0 ** -18   # relative error of scale*H carried as bf16 hi + lo halves
LAMBDA = 10.0       # probabilistic rounding-error bound parameter (see eval_margin)


def golden_lines(name):
    out = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                out.append(line)
    return out


def golden_json(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def rel_l2(got: np.ndarray, ref: np.ndarray) -> float:
    den = float(np.linalg.norm(ref))
    num = float(np.linalg.norm(got - ref))
    return num / den if den > 0 else num


def max_abs(got: np.ndarray, ref: np.ndarray) -> float:
    return float(np.max(np.abs(got - ref))) if got.size else 0.0


def ulp(v: np.ndarray, dtype: str) -> np.ndarray:
    """Spacing of the output format at |v| (bf16: 8 significant bits, fp32: 24)."""
    bits = 8 if dtype == "bf16" else 24
    _, e = np.frexp(np.abs(v))  # |v| = m * 2**e, m in [0.5, 1)
    e = np.maximum(e, -125)
    return np.ldexp(1.0, e - bits)


def eval_margin(mag: np.ndarray, ref: np.ndarray, k_in: int, max_rank: int) -> np.ndarray:
    """Bound on the evaluation error of one output element before its final
    rounding to the output format, for a bf16-in / fp32-accumulate fold.

    The products are exact in fp32 (bf16 x bf16 has 16 significant bits).
    The shrink sums k_in of them, the expand 2 * max_rank (hi and lo halves of
    scale * H, which together carry H to within 2**-18 relatively), and the
    base add is one more fp32 rounding. For a sum of n products the fp32 error
    is at most gamma(n) times the sum of the products' absolute values; with
    the probabilistic bound of Higham and Mary ("A new approach to
    probabilistic rounding error analysis", SIAM J. Sci. Comput. 41(5), 2019)
    gamma(n) <= LAMBDA * sqrt(n) * u, which fails with probability at most
    2n exp(-LAMBDA**2 / 2) per element (below 1e-18 here) instead of the
    deterministic n * u, which no summation of this size comes near.
    ``mag`` is that sum of absolute values per element (oracle magnitude
    fold); the last term covers the base add and the fp32 value's own
    rounding before the output rounding."""
    gam = LAMBDA * (math.sqrt(k_in) + math.sqrt(2 * max_rank)) * U32
    return (gam + HILO + 2 * U32) * mag + 2 * U32 * np.abs(ref)


def max_abs_limit(ref: np.ndarray, eps: np.ndarray, dtype: str) -> np.ndarray:
    """Per element: max(3e-2, half an output ulp at |ref| + eps, plus eps).

    Reading of the max-abs bound: a correctly rounded bf16 output is off from
    the exact result by up to half an ulp, which exceeds 3e-2 once |ref| >= 8
    (gate/up outputs reach |ref| ~ 10); a device result is rounded from an
    fp32 value within eps of the exact one, so it may be off by half an ulp of
    that value plus eps."""
    return np.maximum(MAX_ABS_TOL, 0.5 * ulp(np.abs(ref) + eps, dtype) + eps)


def max_abs_excess(got: np.ndarray, ref: np.ndarray, dtype: str, eps: np.ndarray) -> float:
    """Largest ratio |got - ref| / max_abs_limit(ref, eps); <= 1 passes."""
    if not got.size:
        return 0.0
    return float(np.max(np.abs(got - ref) / max_abs_limit(ref, eps, dtype)))


def view_margin(view, ref: np.ndarray, windows=None) -> np.ndarray:
    """eval_margin for an OracleView's case (its magnitude fold, which does not
    depend on the base and is kept on the view)."""
    c = view.case
    key = "_mag" if windows is None else None
    mag = getattr(view, key, None) if key else None
    if mag is None:
        mag = view.magnitude(windows=windows)
        if key:
            setattr(view, key, mag)
    return eval_margin(mag, ref, c.k_in, c.max_rank)


# Observed parity figures of this process: (label, rel_l2, max_abs,
# max_abs / limit). conftest writes them out when MLORA_PARITY_LOG is set.
PARITY_LOG = []


def parity_figures(view, got_f64: np.ndarray, ref: np.ndarray, label: str, windows=None):
    """(rel_l2, max_abs, max_abs / limit) of one comparison, recorded."""
    eps = view_margin(view, ref, windows)
    rel, mx = rel_l2(got_f64, ref), max_abs(got_f64, ref)
    ex = max_abs_excess(got_f64, ref, view.case.dtype, eps)
    PARITY_LOG.append((label, rel, mx, ex))
    return rel, mx, ex
