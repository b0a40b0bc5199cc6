"""Error reporting shared by the GPU parity tests.

Every comparison against the oracle goes through ``report``: it prints the case name,
the max abs error, the max |ref| and their ratio (an off-by-one band shifts outputs by
a fraction of their own size, so the ratio is the figure that shows it), and appends
the same figures as one JSON line to the file named by $LF_PARITY_REPORT when that
variable is set.
"""
from __future__ import annotations

import json
import os

import numpy as np


def report(case: str, got, ref, tol) -> float:
    """Print and record the error of ``got`` against ``ref``; returns the max abs error."""
    g = np.asarray(got, np.float64)
    r = np.asarray(ref, np.float64)
    err = np.abs(g - r)
    max_abs = float(err.max()) if err.size else 0.0
    max_ref = float(np.abs(r).max()) if r.size else 0.0
    ratio = max_abs / max_ref if max_ref > 0 else 0.0
    tol_s = tol if isinstance(tol, str) else (f"{float(tol):.3g}" if np.ndim(tol) == 0
                                              else "per-element")
    print(f"[parity] {case}: max_abs={max_abs:.3e} max_ref={max_ref:.3e} "
          f"abs/ref={ratio:.3e} elements={err.size} tol={tol_s}", flush=True)
    path = os.environ.get("LF_PARITY_REPORT")
    if path:
        with open(path, "a") as f:
            f.write(json.dumps({"case": case, "max_abs": max_abs, "max_ref": max_ref,
                                "abs_over_ref": ratio, "elements": int(err.size),
                                "tol": tol_s}) + "\n")
    return max_abs
