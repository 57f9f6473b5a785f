"""Pins of the oracle's parity bands: the accept-test flag, the inverse-CDF edge distance and the
set of tokens a draw inside the band may return (oracle.chain.draw_band).

The bands decide which GPU results count as correct, so they are pinned against values that do
not come from the oracle: hand-computed literals on small integer-weight rows whose total is a
power of two (every bucket edge and every u * W is then a dyadic rational, exact in fp64), and
exact rational arithmetic (fractions.Fraction) on random rows of that kind, with u * W placed on
an edge, just inside the band and just outside it.  Planted mistakes in the edge distance and
the band set each fail a pin.

Sources: the Speculative Sampling explainer (0h-n0.github.io), Step 3 (ステップ3, the accept test
u < min(1, p/q)) and modified rejection sampling (修正付き棄却サンプリング, the draw); the band
width 1e-6 is the parity tolerance of the build's statement of the problem.
"""

from fractions import Fraction

import numpy as np
import pytest

from oracle import chain as OC
from parity import allowed_outcomes

EPS24 = 2.0 ** -24  # one step of the uniforms' 2^-24 grid
EPS19 = 2.0 ** -19  # 1.9e-6: a relative distance just outside the 1e-6 band

# w = [3, 0, 5, 2, 0, 6], W = 16: buckets token 0 [0, 3), token 2 [3, 8), token 3 [8, 10),
# token 5 [10, 16); tokens 1 and 4 have none.
W6 = np.array([3.0, 0.0, 5.0, 2.0, 0.0, 6.0])
# (u, drawn token, edge distance / W, band set), worked out by hand.
HAND = [
    (0.0, 0, 0.0, {0}),                          # on the left end: no neighbour below
    (3 / 16, 2, 0.0, {0, 2}),                    # exactly on the edge C(0) = C(1) = 3
    (3 / 16 + EPS24, 2, EPS24, {0, 2}),          # 2^-24 above it: inside the band
    (3 / 16 + EPS19, 2, EPS19, {2}),             # 2^-19 above it: outside
    (0.25, 2, 1 / 16, {2}),                      # mid-bucket
    (0.5 - EPS24, 2, EPS24, {2, 3}),             # just below the edge C(2) = 8
    (0.5, 3, 0.0, {2, 3}),                       # on it
    (0.5 + EPS19, 3, EPS19, {3}),                # outside the band above it
    (10 / 16, 5, 0.0, {3, 5}),                   # on C(3) = C(4) = 10: skips zero-weight 4
    (10 / 16 - EPS24, 3, EPS24, {3, 5}),         # just below it
    (1.0 - EPS24, 5, EPS24, {5}),                # near the right end: no neighbour above
]

# A bucket narrower than the band: w = [2^20, 1, 2^20 - 1], W = 2^21; token 1's bucket
# [2^20, 2^20 + 1) is 4.8e-7 W wide, so a draw near it may land one token further.
W_TINY = np.array([2.0 ** 20, 1.0, 2.0 ** 20 - 1.0])
HAND_TINY = [
    (0.5, 1, 0.0, {0, 1, 2}),
    (0.5 + EPS24, 1, 2.0 ** -3 / 2.0 ** 21, {0, 1, 2}),
    (0.25, 0, 0.25, {0}),
    (0.75, 2, 0.25 - 1 / 2.0 ** 21, {2}),
]


@pytest.mark.parametrize("w, case", [(W6, c) for c in HAND] + [(W_TINY, c) for c in HAND_TINY])
def test_draw_hand_values(w, case):
    u, y_want, edge_want, band_want = case
    y, edge = OC.inverse_cdf(w, u)
    assert y == y_want
    assert edge == pytest.approx(edge_want, rel=0, abs=1e-15)
    assert OC.draw_band(w, u) == band_want
    assert (edge < OC.BAND) == (len(band_want) > 1 or edge_want < 1e-6)


def exact_draw(wi, u):
    """Inverse CDF in exact rational arithmetic: (y, edge / W, band set) for integer weights wi
    and a uniform u (a float, taken at its exact binary value)."""
    total = sum(wi)
    tau = Fraction(u) * total
    b = Fraction(OC.BAND) * total
    c, run = [], 0
    for x in wi:
        run += x
        c.append(run)
    y = next(i for i, ci in enumerate(c) if ci > tau)
    lower = c[y - 1] if y > 0 else 0
    edge = min(tau - lower, c[y] - tau) / total
    band = set()
    for i, x in enumerate(wi):
        lo = c[i - 1] if i > 0 else 0
        if x > 0 and lo <= tau + b and c[i] > tau - b:
            band.add(i)
    return y, edge, band


def random_rows(seed, n):
    """Rows of 2..40 non-negative integer weights (about a third zero) scaled to a power-of-two
    total, each with uniforms on the 2^-24 grid and at, just inside and just outside the band
    around a random positive-weight bucket edge."""
    rng = np.random.default_rng(seed)
    for _ in range(n):
        V = int(rng.integers(2, 41))
        wi = rng.integers(1, 1000, V) * (rng.random(V) > 0.33)
        if wi.sum() == 0:
            wi[rng.integers(V)] = 1
        k = int(np.ceil(np.log2(wi.sum())))
        wi[int(np.flatnonzero(wi)[-1])] += (1 << k) - int(wi.sum())  # total 2^k
        total = 1 << k
        edges = np.cumsum(wi)[wi > 0][:-1]
        us = list(rng.integers(0, 1 << 24, 4) / float(1 << 24))
        if len(edges):
            e = float(rng.choice(edges)) / total
            us += [e, e + EPS24, e - EPS24, e + EPS19, e - EPS19, e + 2 * EPS24]
        yield [int(x) for x in wi], [u for u in us if 0.0 <= u < 1.0]


def test_draw_matches_exact_rationals():
    n = 0
    flagged = 0
    for wi, us in random_rows(7, 400):
        w = np.array(wi, dtype=np.float64)
        for u in us:
            y_ex, edge_ex, band_ex = exact_draw(wi, u)
            y, edge = OC.inverse_cdf(w, u)
            assert y == y_ex, (wi, u)
            # fp64 is exact on these rows except for the final division by W (a power of two:
            # also exact), so the edge distance agrees to the last bit.
            assert Fraction(edge) == edge_ex, (wi, u, edge, float(edge_ex))
            assert OC.draw_band(w, u) == band_ex, (wi, u)
            assert y in band_ex and all(wi[x] > 0 for x in band_ex)
            n += 1
            flagged += edge < OC.BAND
    assert n > 2000 and flagged > 500


def _mut_lower_only(w, u):
    c = np.cumsum(w)
    tau = u * c[-1]
    y = int(np.argmax(c > tau))
    return y, float((tau - (c[y - 1] if y > 0 else 0.0)) / c[-1])


def _mut_over_cy(w, u):
    c = np.cumsum(w)
    tau = u * c[-1]
    y = int(np.argmax(c > tau))
    return y, float(min(tau - (c[y - 1] if y > 0 else 0.0), c[y] - tau) / c[y])


def _mut_both_neighbours(w, u):
    y, edge = OC.inverse_cdf(w, u)
    out = {y}
    if edge < OC.BAND:
        pos = np.flatnonzero(np.asarray(w) > 0)
        out |= {int(x) for x in pos[pos < y][-1:]} | {int(x) for x in pos[pos > y][:1]}
    return out


def _band_pins_pass():
    try:
        for w, cases in ((W6, HAND), (W_TINY, HAND_TINY)):
            for u, y_want, edge_want, band_want in cases:
                y, edge = OC.inverse_cdf(w, u)
                if y != y_want or abs(edge - edge_want) > 1e-15 or OC.draw_band(w, u) != band_want:
                    return False
        return True
    except Exception:
        return False


def test_band_pins_pass_on_unmutated_oracle():
    assert _band_pins_pass()


@pytest.mark.parametrize("attr, bad", [("inverse_cdf", _mut_lower_only),
                                       ("inverse_cdf", _mut_over_cy),
                                       ("draw_band", _mut_both_neighbours),
                                       ("draw_band", lambda w, u: {OC.inverse_cdf(w, u)[0]})])
def test_planted_band_mistakes_fail_a_pin(attr, bad, monkeypatch):
    monkeypatch.setattr(OC, attr, bad)
    assert not _band_pins_pass()


# ----------------------------------------------------------------------------- accept band

ZT = np.log(np.array([[0.3, 0.7], [0.5, 0.5]]))
ZD = np.log(np.array([[0.6, 0.4]]))  # token 0: p/q = 0.5


@pytest.mark.parametrize("u0, flagged, k", [
    (0.5 - EPS24, True, 1),   # inside the band, below the threshold: accepted
    (0.5 + EPS24, True, 0),   # inside, above: rejected
    (0.5, True, 0),           # on the threshold: the strict test rejects
    (0.5 - EPS19, False, 1),  # 1.9e-6 below: outside the band
    (0.5 + EPS19, False, 0),  # 1.9e-6 above
    (0.25, False, 1),
])
def test_accept_flag_inside_and_outside(u0, flagged, k):
    r = OC.verify_chain_seq(ZT, ZD, [0], [u0, 0.5], 1.0)
    assert r["flag_accept"] == ([0] if flagged else [])
    assert r["k"] == k


def test_accept_flag_threshold_one_and_zero_probability():
    # p(x) >= q(x): the threshold is 1, so u just below 1 is inside the band (and accepted).
    zt = np.log(np.array([[0.6, 0.4], [0.5, 0.5]]))
    zd = np.log(np.array([[0.3, 0.7]]))
    r = OC.verify_chain_seq(zt, zd, [0], [1.0 - EPS24, 0.5], 1.0)
    assert r["flag_accept"] == [0] and r["k"] == 1
    r = OC.verify_chain_seq(zt, zd, [0], [1.0 - EPS19, 0.5], 1.0)
    assert r["flag_accept"] == [] and r["k"] == 1
    # p(x) = q(x) = 0 defines no threshold: rejected, never flagged, whatever u is.
    zt = np.array([[-np.inf, 0.0], [0.0, 0.0]])
    zd = np.array([[-np.inf, 0.0]])
    for u0 in (0.0, EPS24, 0.5):
        r = OC.verify_chain_seq(zt, zd, [0], [u0, 0.5], 1.0)
        assert r["flag_accept"] == [] and r["k"] == 0


def test_flags_only_positions_tested():
    # Position 1 sits in the band but is never tested once position 0 rejects.
    zt = np.log(np.array([[0.3, 0.7], [0.3, 0.7], [0.5, 0.5]]))
    zd = np.log(np.array([[0.6, 0.4], [0.6, 0.4]]))
    r = OC.verify_chain_seq(zt, zd, [0, 0], [0.9, 0.5 - EPS24, 0.5], 1.0)
    assert r["k"] == 0 and r["flag_accept"] == []
    r = OC.verify_chain_seq(zt, zd, [0, 0], [0.1, 0.5 - EPS24, 0.5], 1.0)
    assert r["k"] == 2 and r["flag_accept"] == [1]


# ----------------------------------------------------------------------------- allowed outcomes

def test_allowed_outcomes_edge_band_bonus_draw():
    # Every draft accepted (u = 0), then a bonus draw from p_1 = W6 / 16 with u' on the edge
    # C(0) = 3: the GPU may return token 0 or token 2, nothing else.
    with np.errstate(divide="ignore"):
        zt = np.vstack([np.log([0.5, 0.1, 0.1, 0.1, 0.1, 0.1]), np.log(W6 / 16.0)])
    zd = np.log(np.array([[0.5, 0.1, 0.1, 0.1, 0.1, 0.1]]))
    uni = np.array([0.0, 3 / 16])
    res = OC.verify_chain_seq(zt, zd, [0], uni, 1.0)
    assert res["k"] == 1 and res["edge"] < OC.BAND
    allowed, kind = allowed_outcomes(zt, zd, [0], uni, 1.0, res)
    assert kind == "edge_band"
    assert allowed == {(1, (0, 0)), (1, (0, 2))}
    uni = np.array([0.0, 0.25])
    res = OC.verify_chain_seq(zt, zd, [0], uni, 1.0)
    allowed, kind = allowed_outcomes(zt, zd, [0], uni, 1.0, res)
    assert kind == "exact" and allowed == {(1, (0, 2))}


def test_allowed_outcomes_accept_band_replays_both_decisions():
    uni = np.array([0.5 - EPS24, 0.3])
    res = OC.verify_chain_seq(ZT, ZD, [0], uni, 1.0)
    allowed, kind = allowed_outcomes(ZT, ZD, [0], uni, 1.0, res)
    assert kind == "accept_band"
    # Accepted: bonus draw from p_1 = (0.5, 0.5) at u' = 0.3 -> token 0.  Rejected: residual
    # max(0, p_0 - q_0) = (0, 0.3) -> token 1.
    assert allowed == {(1, (0, 0)), (0, (1,))}
