"""Error metric of the parity checks — oracle, test infrastructure only.

rel_F(a, ref) = ||a - ref||_F / ||ref||_F in fp64; where ||ref|| = 0 the check is
that a is exactly zero (returned as 0.0 if so, inf otherwise).
"""
from __future__ import annotations

import numpy as np


def rel_f(a, ref) -> float:
    a = np.asarray(a, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    nr = np.linalg.norm(ref.ravel())
    if nr == 0.0:
        return 0.0 if not np.any(a) else float("inf")
    return float(np.linalg.norm((a - ref).ravel()) / nr)
