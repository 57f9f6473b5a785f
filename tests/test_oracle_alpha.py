"""Pins of the acceptance-rate oracle against facts that do not come from it.

* Closed forms: V = 2 with p = (a, 1-a), q = (b, 1-b) gives alpha = 1 - |a - b|; p uniform on
  n tokens and q uniform on n tokens shifted by s gives alpha = (n - s) / n; p == q gives 1 and
  disjoint supports give 0.
* The identity sum_x min(p, q) = 1 - sum_x max(0, p - q) against scipy's softmax.
* Monte Carlo through the chain oracle (pinned by Theorem 1 and the expected-tokens law): the
  fraction of sequences whose first drafted token is accepted estimates alpha_0.
* Mutation checks: plausible mistakes planted in the oracle make a pin fail.
"""

import numpy as np
import pytest
from scipy.special import softmax as sp_softmax

from oracle import alpha as OA
from oracle import chain as OC


def _closed_forms_hold():
    for a, b in ((0.6, 0.3), (0.1, 0.9), (0.5, 0.5), (0.999, 0.001)):
        zt = np.log(np.array([[a, 1 - a]] * 3))
        zd = np.log(np.array([[b, 1 - b]] * 2))
        al, st = OA.acceptance_rates_seq(zt, zd, 1.0)
        if not (np.allclose(al, 1 - abs(a - b), rtol=1e-12, atol=1e-15) and not st.any()):
            return False
    for n, s in ((8, 2), (10, 7), (16, 0)):
        V = n + s
        zt = np.full((2, V), -np.inf)
        zd = np.full((1, V), -np.inf)
        zt[:, :n] = 0.0
        zd[:, s:s + n] = 0.0
        al, _ = OA.acceptance_rates_seq(zt, zd, 0.7)
        if not np.isclose(al[0], (n - s) / n, rtol=1e-12, atol=1e-15):
            return False
    return True


def test_closed_forms():
    assert _closed_forms_hold()


def _temperature_closed_form_holds():
    # Two tokens with logit gaps g_t and g_d: p = sigmoid(g_t / T), q = sigmoid(g_d / T).
    for T in (0.5, 2.0):
        zt = np.array([[1.3, 0.0], [0.0, 0.0]])
        zd = np.array([[-0.4, 0.0]])
        al, _ = OA.acceptance_rates_seq(zt, zd, T)
        a = 1 / (1 + np.exp(-1.3 / T))
        b = 1 / (1 + np.exp(0.4 / T))
        if not np.isclose(al[0], 1 - abs(a - b), rtol=1e-12):
            return False
    return True


def test_temperature_closed_form():
    assert _temperature_closed_form_holds()


def test_identity_with_residual_mass_and_symmetry():
    rng = np.random.default_rng(8)
    for _ in range(50):
        V = int(rng.integers(2, 40))
        T = float(rng.uniform(0.3, 2.0))
        zt = rng.normal(0, 2, size=(2, V))
        zd = rng.normal(0, 2, size=(1, V))
        al, _ = OA.acceptance_rates_seq(zt, zd, T)
        p, q = sp_softmax(zt[0] / T), sp_softmax(zd[0] / T)
        assert np.isclose(al[0], np.minimum(p, q).sum(), rtol=1e-12)
        assert np.isclose(al[0], 1 - np.maximum(0, p - q).sum(), rtol=1e-9, atol=1e-12)
        back, _ = OA.acceptance_rates_seq(zd, zt[:1], T)
        assert np.isclose(al[0], back[0], rtol=1e-12)


def _monte_carlo_agrees(seed=9, N=6000):
    rng = np.random.default_rng(seed)
    V, T = 6, 0.9
    zt = rng.normal(0, 1.5, size=(2, V))
    zd = zt[:1] + rng.normal(0, 1.0, size=(1, V))
    al, _ = OA.acceptance_rates_seq(zt, zd, T)
    acc = 0
    for _ in range(N):
        x = np.argmax(zd / T + rng.gumbel(size=zd.shape), axis=1)
        u = rng.integers(0, 1 << 24, 2) / float(1 << 24)
        acc += OC.verify_chain_seq(zt, zd, x, u, T)["k"] >= 1
    est = acc / N
    se = np.sqrt(al[0] * (1 - al[0]) / N)
    return abs(est - al[0]) < 4 * se


def test_monte_carlo_first_position():
    assert _monte_carlo_agrees()


def test_special_cases_and_flags():
    z = np.random.default_rng(3).normal(size=(3, 9))
    al, st = OA.acceptance_rates_seq(z, z[:2], 1.3)
    assert np.allclose(al, 1.0) and not st.any()
    zt = np.array([[0.0, -np.inf], [0.0, 0.0]])
    zd = np.array([[-np.inf, 0.0]])
    al, _ = OA.acceptance_rates_seq(zt, zd, 1.0)
    assert al[0] == 0.0
    zt = np.array([[0.0, np.nan], [0.0, 0.0], [0.0, 0.0]])
    zd = np.zeros((2, 2))
    al, st = OA.acceptance_rates_seq(zt, zd, -1.0)
    assert np.isnan(al[0]) and st[0] == OC.ROW_NONFINITE | OC.ROW_BAD_TEMPERATURE
    assert al[1] == 1.0 and st[1] == OC.ROW_BAD_TEMPERATURE


MUTATIONS = {
    "max_instead_of_min": lambda p, q: float(sum(qx * max(1.0, px / qx) for px, qx in zip(p, q) if qx > 0)),
    "ratio_transposed": lambda p, q: float(sum(qx * min(1.0, qx / px) for px, qx in zip(p, q) if px > 0)),
    "weighted_by_p": lambda p, q: float(sum(px * min(1.0, px / qx) for px, qx in zip(p, q) if qx > 0)),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistakes_fail_a_pin(name, monkeypatch):
    monkeypatch.setattr(OA, "acceptance_rate", MUTATIONS[name])
    ok = _closed_forms_hold() and _temperature_closed_form_holds() and _monte_carlo_agrees(N=3000)
    assert not ok, f"mutation {name} went undetected"


def test_planted_temperature_ignored_fails(monkeypatch):
    monkeypatch.setattr(OA, "softmax_fp64", lambda z, T: sp_softmax(z))
    assert not _temperature_closed_form_holds()
