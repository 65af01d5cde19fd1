"""Pins of the oracle's analytics (Leviathan blog, section 方法细节 and the FAQ on choosing
gamma) against independent computations: the acceptance rate against exact enumeration of
the accept event and against the total-variation distance, the wall-clock factor at gamma = 1
against the page's closed form (1 + alpha) / (1 + c) and its "gain iff alpha > c" statement,
and the optimal gamma against its stated behaviour (larger c, smaller gamma; c = 0, the
largest gamma allowed)."""

import numpy as np
import pytest

import oracle.spec_verify_oracle as O


@pytest.mark.parametrize("seed", range(8))
def test_acceptance_rate_by_enumeration(seed):
    rng = np.random.default_rng(seed)
    V = 12
    q = rng.dirichlet(np.full(V, 0.5))
    p = rng.dirichlet(np.full(V, 0.5))
    for lenience in (1.0, 0.5, 0.1):
        # P(accept) = sum over drafts x of p(x) * P(u < a(x)), a from the oracle's own rule
        enum = sum(p[x] * O.accept_probability(q[x], p[x], lenience) for x in range(V))
        assert abs(O.acceptance_rate(q, p, lenience) - enum) < 1e-12
    tv = 0.5 * float(np.abs(p - q).sum())
    assert abs(O.acceptance_rate(q, p) - (1.0 - tv)) < 1e-12


def test_acceptance_rate_special_cases():
    q = np.array([0.2, 0.3, 0.5])
    assert abs(O.acceptance_rate(q, q) - 1.0) < 1e-15
    assert O.acceptance_rate(np.array([1.0, 0, 0]), np.array([0, 0.5, 0.5])) == 0.0


@pytest.mark.parametrize("alpha,c", [(0.3, 0.0), (0.6, 0.1), (0.9, 0.05), (0.5, 0.5),
                                     (0.2, 0.4)])
def test_gamma_one_closed_form_and_gain(alpha, c):
    v = O.walltime_speedup(alpha, 1, c)
    assert abs(v - (1 + alpha) / (1 + c)) < 1e-12
    assert (v > 1) == (alpha > c)


def test_optimal_gamma_behaviour():
    for alpha in (0.6, 0.8, 0.95):  # (at small alpha the factor saturates in float64)
        assert O.optimal_gamma(alpha, 0.0, 40) == 40  # free draft: longer is always better
        gs = [O.optimal_gamma(alpha, c, 40) for c in (0.01, 0.05, 0.1, 0.2, 0.4)]
        assert all(a >= b for a, b in zip(gs, gs[1:]))  # larger c, smaller gamma
        # the chosen gamma beats its neighbours
        for c in (0.01, 0.05, 0.2):
            g = O.optimal_gamma(alpha, c, 40)
            v = O.walltime_speedup(alpha, g, c)
            if g > 1:
                assert v >= O.walltime_speedup(alpha, g - 1, c)
            if g < 40:
                assert v >= O.walltime_speedup(alpha, g + 1, c)
