"""Bound on the requests a parity check may leave uncompared.

The oracle flags a request whose outcome sits within a rounding band of a boundary (an
acceptance test, an inverse-CDF breakpoint, a nucleus cut, a fuzzy threshold); parity skips
those requests.  A flag that fired too often would silently empty a parity test, so every check
asserts that at most max(1, B / 1000) requests were flagged (or the bound a test states for
inputs built to sit on boundaries), and that at least one request was compared.
"""
import numpy as np


def bound_flagged(flags, label, allow=None):
    flags = np.asarray(flags)
    B = int(flags.size)
    n = int((flags != 0).sum())
    lim = max(1, B // 1000) if allow is None else int(allow)
    print(f"[flags] {label}: oracle flagged {n} of {B} (bound {lim})", flush=True)
    assert n <= lim, f"{label}: {n} of {B} requests flagged, more than {lim}"
    assert n < B, f"{label}: every request flagged, nothing compared"
    return n
