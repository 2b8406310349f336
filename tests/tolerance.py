"""Output tolerances for comparing GPU results with the oracle's y_exact.

Integer results (codes, scales, zero points, int32 accumulators) are compared
bit for bit elsewhere; this module covers the floating-point epilogues.

  fp32 outputs:       |y - y_exact| <= 1e-5 |y_exact|
  bf16 / fp16 outputs:|y - y_exact| <= 1 ulp of the output format at y_exact
A result that sums terms of both signs in binary32 (the group sums of W4A8
and W4A16) may lose relative accuracy near zero; such an output also passes if
  |y - y_exact| <= ulp_out(y_exact) + n * 2^-24 * B,
with B the sum of the magnitudes of the terms and n the number of binary32
roundings that can touch the sum (derived per kernel in the test).

For fp32 outputs the floor is the working bar whenever |y_exact| is below
about n / 168 of B (1e-5 is 168 units of 2^-24): that is what binary32
summation can promise near cancellation.  Over seeded random layers it decides
about 0.2% of the fp32 outputs, so a check of at least FLOOR_MIN_OUTPUTS
outputs may pass at most FLOOR_FRAC_32 of them through it alone (smaller
checks, a few dozen outputs, at most FLOOR_FRAC_SMALL).  For bf16 / fp16
outputs one ulp is 2^-8 / 2^-11 relative, so the floor should decide only
outputs near zero: at most FLOOR_FRAC_16 of them.  Every check is logged in
FLOOR_LOG, and the test session prints the counts at its end
(tests/conftest.py).
"""
from __future__ import annotations

import numpy as np

_FMT = {"bf16": (8, -126), "f16": (11, -14)}
FLOOR_FRAC_16 = 0.01   # bf16 / fp16 outputs that may pass through the floor alone
FLOOR_FRAC_32 = 0.02   # fp32 outputs, checks of at least FLOOR_MIN_OUTPUTS outputs
FLOOR_FRAC_SMALL = 0.25
FLOOR_MIN_OUTPUTS = 4096
FLOOR_LOG = []         # (what, fmt, outputs passing only via the floor, outputs checked)


def ulp(y_exact: np.ndarray, fmt: str) -> np.ndarray:
    """Spacing of `fmt` values at |y_exact| (the subnormal spacing near 0)."""
    p, emin = _FMT[fmt]
    a = np.abs(np.asarray(y_exact, np.float64))
    _, e = np.frexp(a)                    # a = m 2^e, m in [0.5, 1)
    e = np.maximum(e - 1, emin)
    return np.ldexp(1.0, e - (p - 1))


def check(y, y_exact, fmt: str, floor=None):
    """Return (ok mask, number of outputs that pass only through the floor)."""
    y = np.asarray(y, np.float64)
    ye = np.asarray(y_exact, np.float64)
    d = np.abs(y - ye)
    if fmt == "f32":
        base = d <= 1e-5 * np.abs(ye)
        bound = 1e-5 * np.abs(ye)
    else:
        bound = ulp(ye, fmt)
        base = d <= bound
    if floor is None:
        return base, 0
    ok = base | (d <= bound + floor)
    return ok, int(np.count_nonzero(ok & ~base))


def assert_close(y, y_exact, fmt: str, floor=None, what: str = "", max_floor_frac=None):
    ok, via_floor = check(y, y_exact, fmt, floor)
    if floor is not None:
        FLOOR_LOG.append((what, fmt, via_floor, int(np.size(y_exact))))
        if max_floor_frac is not None:
            lim = max_floor_frac
        elif fmt != "f32":
            lim = FLOOR_FRAC_16
        else:
            lim = FLOOR_FRAC_32 if np.size(y_exact) >= FLOOR_MIN_OUTPUTS else FLOOR_FRAC_SMALL
        if lim is not None and via_floor > lim * np.size(y_exact):
            raise AssertionError(f"{what}: {via_floor} of {np.size(y_exact)} {fmt} outputs pass only "
                                 f"through the cancellation floor (limit {lim:.2%})")
    if not ok.all():
        idx = np.argwhere(~ok)[:5]
        yy = np.asarray(y, np.float64)
        ye = np.asarray(y_exact, np.float64)
        rows = [(tuple(i), float(yy[tuple(i)]), float(ye[tuple(i)])) for i in idx]
        raise AssertionError(f"{what}: {np.count_nonzero(~ok)} of {ok.size} outputs out of "
                             f"tolerance ({fmt}); first: {rows}")
    return via_floor
