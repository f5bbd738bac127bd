"""Max-abs errors of the GPU parity checks, printed at the end of the run.

Every floating-point comparison of a HIP result with the oracle goes through
``within``, which records the test, what was compared, the measured max-abs
error and the tolerance; conftest prints the table (with the margin, the
tolerance over the error) in pytest's terminal summary.
"""

from __future__ import annotations

import os

import numpy as np

RECORDS: list[tuple[str, str, str, float, float]] = []


def within(got, want, tol, dtype="", what=""):
    """Asserts max|got - want| <= tol (0 for empty arrays), records it and
    returns the error."""
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, (got.shape, want.shape)
    err = float(np.abs(got - want).max()) if got.size else 0.0
    test = os.environ.get("PYTEST_CURRENT_TEST", "?").rsplit(" (", 1)[0]
    RECORDS.append((test, what, dtype, err, float(tol)))
    assert err <= tol, f"{what} max|err| {err:.3e} > {tol:.1e}"
    return err


def summary_lines():
    if not RECORDS:
        return []
    lines = [f"{'max|err|':>10} {'tol':>8} {'margin':>8}  dtype  test [what]"]
    worst: dict[str, float] = {}
    for test, what, dtype, err, tol in RECORDS:
        margin = tol / err if err > 0 else float("inf")
        lines.append(f"{err:10.3e} {tol:8.1e} {margin:8.1f}  {dtype:5}  {test}"
                     + (f" [{what}]" if what else ""))
        if dtype:
            worst[dtype] = max(worst.get(dtype, 0.0), err / tol)
    for dtype, r in sorted(worst.items()):
        lines.append(f"worst {dtype}: max|err| = {r:.3f} x tol (margin {1 / r if r else float('inf'):.1f})")
    return lines
