"""Pins of the oracle's acceptance function (CPU only).

Every GPU parity test decides pass or fail through oracle.within_tolerance,
so it is pinned here to values worked out by hand from the stated bound
|y - y_ref| <= 1e-3 * s + 1e-5 (s = sum |w_i x_i|, inclusive) and from the
rule that non-finite results must match in class: NaN where the oracle has
NaN, and the infinity of the same sign where it has one. Plausible
mistakes are planted in copies of the function and each must be caught by
at least one case.
"""
import numpy as np

import oracle.qmm_oracle as O

INF, NAN = np.inf, np.nan
UP = np.nextafter(1e-5, 1.0)  # one double above 1e-5

# (y, y_ref, s, accepted). Bounds worked out by hand:
#   s = 0     -> bound 1e-5 (the absolute term alone, exactly the double 1e-5)
#   s = 1000  -> bound 1.00001
#   s = 4000  -> bound 4.00001
#   s = 1e6   -> bound 1000.00001
CASES = [
    (0.0, 0.0, 0.0, True),
    (1e-5, 0.0, 0.0, True),           # exactly at the bound: inclusive
    (-1e-5, 0.0, 0.0, True),
    (UP, 0.0, 0.0, False),            # one double over
    (-UP, 0.0, 0.0, False),
    (5e-6, 0.0, 0.0, True),           # inside the absolute term only
    (1.000009, 0.0, 1000.0, True),    # relative term: 1e-3 * 1000 = 1
    (1.000011, 0.0, 1000.0, False),
    (2.000009, 1.0, 1000.0, True),
    (-0.000011, 1.0, 1000.0, False),
    (1.0, -3.0, 4000.0, True),        # |1 - (-3)| = 4 <= 4.00001
    (1.0001, -3.0, 4000.0, False),
    (-7.000009, -3.0, 4000.0, True),
    (-7.0002, -3.0, 4000.0, False),
    (3.0, -3.0, 4000.0, False),       # right magnitude, wrong sign
    (1999.0, 1000.0, 1e6, True),      # |999| <= 1000.00001
    (2001.0, 1000.0, 1e6, False),
    # non-finite classes
    (NAN, NAN, NAN, True),
    (NAN, NAN, 1.0, True),
    (INF, NAN, INF, False),
    (-INF, NAN, INF, False),
    (0.0, NAN, INF, False),
    (INF, INF, INF, True),
    (-INF, -INF, INF, True),
    (-INF, INF, INF, False),
    (INF, -INF, INF, False),
    (NAN, INF, INF, False),
    (3.4e38, INF, INF, False),
    (NAN, 0.0, 0.0, False),
    (INF, 0.0, 0.0, False),
    (-INF, 1.0, 1000.0, False),
]


def _verdicts(fn):
    y = np.array([c[0] for c in CASES])
    ref = np.array([c[1] for c in CASES])
    s = np.array([c[2] for c in CASES])
    return np.asarray(fn(y, ref, s), dtype=bool)


WANT = np.array([c[3] for c in CASES])


def test_hand_worked_cases():
    got = _verdicts(O.within_tolerance)
    bad = [CASES[i] for i in np.flatnonzero(got != WANT)]
    assert not bad, f"wrong verdicts: {bad}"


def test_elementwise_shapes_and_fp32_results():
    # fp32 results (what the kernels return) widen exactly; 2-D arrays keep their shape
    y = np.array([[1e-5, 2e-5], [0.5, np.nan]], np.float32)
    ref = np.array([[0.0, 0.0], [0.5, np.nan]])
    s = np.zeros((2, 2))
    got = O.within_tolerance(y, ref, s)
    assert got.shape == (2, 2)
    # float32(1e-5) lies just below the double 1e-5 (inside the bound at s = 0),
    # float32(2e-5) about twice it (outside)
    assert float(np.float32(1e-5)) < 1e-5 < float(np.float32(2e-5))
    assert got.tolist() == [[True, False], [True, True]]


# ------------------------------------------------------------- planted mistakes
def _rel_1e2(y, r, s):
    return O.within_tolerance(y, r, s, rel=1e-2)


def _no_abs(y, r, s):
    return O.within_tolerance(y, r, s, abs_=0.0)


def _strict(y, r, s):
    with np.errstate(invalid="ignore"):
        ok = np.abs(y - r) < 1e-3 * s + 1e-5
    return np.where(np.isnan(r), np.isnan(y), np.where(np.isinf(r), y == r, ok & np.isfinite(y)))


def _any_nonfinite(y, r, s):
    # the earlier acceptance: non-finite where the oracle is, whatever the class
    fin_ref = np.isfinite(r) & np.isfinite(s)
    with np.errstate(invalid="ignore"):
        close = np.abs(y - r) <= 1e-3 * s + 1e-5
    return (np.isfinite(y) == fin_ref) & (close | ~fin_ref)


def _sign_blind_inf(y, r, s):
    with np.errstate(invalid="ignore"):
        close = np.isfinite(y) & (np.abs(y - r) <= 1e-3 * s + 1e-5)
    return np.where(np.isnan(r), np.isnan(y), np.where(np.isinf(r), np.isinf(y), close))


def _magnitude_only(y, r, s):
    with np.errstate(invalid="ignore"):
        close = np.isfinite(y) & (np.abs(np.abs(y) - np.abs(r)) <= 1e-3 * s + 1e-5)
    return np.where(np.isnan(r), np.isnan(y), np.where(np.isinf(r), y == r, close))


def _nan_unchecked(y, r, s):
    with np.errstate(invalid="ignore"):
        close = np.isfinite(y) & (np.abs(y - r) <= 1e-3 * s + 1e-5)
    return np.where(np.isnan(r), True, np.where(np.isinf(r), y == r, close))


def _relative_to_ref(y, r, s):
    # bound scaled by |y_ref| instead of sum |w x|
    with np.errstate(invalid="ignore"):
        close = np.isfinite(y) & (np.abs(y - r) <= 1e-3 * np.abs(r) + 1e-5)
    return np.where(np.isnan(r), np.isnan(y), np.where(np.isinf(r), y == r, close))


def test_planted_mistakes_are_caught():
    for bad in (_rel_1e2, _no_abs, _strict, _any_nonfinite, _sign_blind_inf, _magnitude_only, _nan_unchecked,
                _relative_to_ref):
        assert (_verdicts(bad) != WANT).any(), bad.__name__
