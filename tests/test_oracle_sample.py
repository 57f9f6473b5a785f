"""Pins of the sampler oracle against facts that do not come from it.

* Exactness of the inverse CDF: over the fine uniform grid u = (k + 1/2) / N the fraction of u
  mapped to each token equals p(x) = scipy's softmax(z / T)(x) within 1/N (for any weights the
  map sends an interval of length p(x) to x).
* A chi-square test of the tokens drawn with random uniforms against scipy's softmax.
* numpy's searchsorted on the cumulative sum, and the zero-probability tokens never drawn.
* Mutation checks: plausible mistakes planted in the oracle make a pin fail.
"""

import numpy as np
import pytest
from scipy import stats
from scipy.special import softmax as sp_softmax

from oracle import chain as OC
from oracle import sample as OS


def _grid_fractions_match(seed=5, N=20000):
    rng = np.random.default_rng(seed)
    for V, T in ((2, 1.0), (7, 0.6), (40, 1.7)):
        z = rng.normal(0, 2, size=V)
        z[rng.integers(0, V)] = -np.inf if V > 2 else z[0]
        p = sp_softmax(z / T)
        counts = np.zeros(V)
        for k in range(N):
            counts[OS.sample_row(z, T, (k + 0.5) / N)["token"]] += 1
        if not np.all(np.abs(counts / N - p) <= 1.0 / N + 1e-12):
            return False
    return True


def test_inverse_cdf_grid_exactness():
    assert _grid_fractions_match()


def _chi_square_passes(seed=6, N=20000):
    rng = np.random.default_rng(seed)
    V, T = 12, 0.8
    z = rng.normal(0, 1.5, size=V)
    u = rng.integers(0, 1 << 24, size=N) / float(1 << 24)
    toks = [OS.sample_row(z, T, x)["token"] for x in u]
    obs = np.bincount(toks, minlength=V)
    return stats.chisquare(obs, sp_softmax(z / T) * N).pvalue > 1e-3


def test_chi_square_against_softmax():
    assert _chi_square_passes()


def _searchsorted_agrees(trials=200):
    """Token-id order: the draw equals searchsorted on the cumulative softmax, and prob = p(y)."""
    rng = np.random.default_rng(7)
    for _ in range(trials):
        V = int(rng.integers(1, 30))
        T = float(rng.uniform(0.2, 3.0))
        z = rng.normal(0, 3, size=V)
        u = float(rng.random())
        r = OS.sample_row(z, T, u)
        p = sp_softmax(z / T)
        c = np.cumsum(p)
        if r["token"] != int(np.searchsorted(c, u * c[-1], side="right")):
            return False
        if not np.isclose(r["prob"], p[r["token"]], rtol=1e-12):
            return False
    return True


def test_matches_searchsorted_and_prob():
    assert _searchsorted_agrees()


def test_zero_probability_never_drawn_and_flags():
    z = np.array([-np.inf, 0.0, -np.inf, 1.0])
    for u in (0.0, 0.3, 0.999999):
        assert OS.sample_row(z, 1.0, u)["token"] in (1, 3)
    assert OS.sample_row(z, 0.0, 0.5)["status"] == OC.ROW_BAD_TEMPERATURE
    assert OS.sample_row(z, 1.0, 1.0)["status"] == OC.ROW_BAD_UNIFORM
    r = OS.sample_row(np.array([0.0, np.nan]), 1.0, 0.5)
    assert r["status"] == OC.ROW_NONFINITE and r["token"] == 0


MUTATIONS = {
    "temperature_ignored": ("softmax_fp64", lambda z, T: sp_softmax(z)),
    "reversed_cdf": ("inverse_cdf", lambda w, u: (len(w) - 1 - OC.inverse_cdf(w[::-1], u)[0], 1.0)),
    "cdf_off_by_one": ("inverse_cdf", lambda w, u: (min(len(w) - 1, OC.inverse_cdf(w, u)[0] + 1), 1.0)),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistakes_fail_a_pin(name, monkeypatch):
    attr, bad = MUTATIONS[name]
    monkeypatch.setattr(OS, attr, bad)
    ok = _searchsorted_agrees() and _grid_fractions_match(N=4000) and _chi_square_passes(N=8000)
    assert not ok, f"mutation {name} went undetected"
