"""CPU checks of the exact-rational selection counts (tests/_exact.py) that
the full-size GPU tests use as the exact-arithmetic pin of the selection."""

from fractions import Fraction

import numpy as np
import pytest

import oracle
from tests import _exact


def _fraction_count(x, tau):
    """The selection count as a plain loop over Fractions."""
    vals = sorted((Fraction(float(v)) for v in x), reverse=True)
    if tau >= 1.0:
        return len(vals)
    tot, t = Fraction(0), Fraction(tau)
    for k, val in enumerate(vals, 1):
        tot += val
        if tot >= t:
            return k
    return len(vals)


def test_scaled_ints_are_exact():
    vals = np.array([0.0, 1.4e-45, 2.9e-39, 1.1754942e-38, 1.1754944e-38, 2.0 ** -30, 1e-7,
                     0.1, 0.5, 0.99, 1.0, 3.4e38], np.float32)
    ints = _exact.scaled_ints(vals)
    for v, i in zip(vals, ints):
        assert Fraction(i, 2 ** 149) == Fraction(float(v)), v
    with pytest.raises(ValueError):
        _exact.scaled_ints(np.array([-1.0], np.float32))
    with pytest.raises(ValueError):
        _exact.scaled_ints(np.array([np.inf], np.float32))


@pytest.mark.parametrize("nb", [1, 5, 64, 300])
def test_exact_counts_match_fraction_loop(nb):
    rng = np.random.default_rng(nb)
    rows = []
    for kind in range(6):
        x = rng.dirichlet(np.full(nb, (0.05, 0.5, 5.0, 1.0, 0.2, 0.5)[kind]))
        if kind == 3:
            x[:] = 1.0 / nb
        if kind == 4:
            x[rng.integers(0, nb, max(1, nb // 3))] = 0.0
        if kind == 5:
            x[rng.integers(0, nb, max(1, nb // 3))] = 1e-40   # float32 denormals
        rows.append(x.astype(np.float32))
    mass = np.stack(rows)
    for tau in (0.3, 0.9, 0.99, 0.999, 1.0, 1.5):
        got = _exact.exact_counts(mass, tau, chunk=4)
        want = [_fraction_count(r, tau) for r in mass]
        assert got.tolist() == want, tau


def test_exact_counts_at_the_cut():
    # a prefix that equals tau exactly in rationals reaches it; one ulp
    # below does not
    x = np.array([0.5, 0.25, 0.125, 0.125], np.float32)
    assert _exact.exact_counts(x[None], 0.75).tolist() == [2]
    assert _exact.exact_counts(x[None], np.nextafter(0.75, 1.0)).tolist() == [3]
    assert _exact.exact_counts(x[None], np.nextafter(0.75, 0.0)).tolist() == [2]


def test_oracle_float64_decisions_are_exact():
    # the oracle accumulates in float64; for float32 masses >= 2^-30 its
    # prefixes below 1 are exact, so its counts equal the exact ones
    rng = np.random.default_rng(11)
    mass = np.stack([rng.dirichlet(np.full(512, a)) for a in (0.05, 0.3, 3.0) * 20])
    mass = np.maximum(mass, 2.0 ** -30).astype(np.float32)
    for tau in (0.9, 0.99, 0.999):
        _, cnt = oracle.select(mass, tau)
        assert np.array_equal(cnt, _exact.exact_counts(mass, tau))
