"""The library's host-side analytics (spec_expected_tokens, spec_walltime_speedup,
spec_ops_factor, spec_optimal_gamma; no GPU work) against the pinned oracle formulas."""

import math

import numpy as np
import pytest

import oracle.spec_verify_oracle as O


@pytest.fixture(scope="module")
def svl():
    from speculative_sampling_verification_amd import _lib
    return _lib


def test_formulas_match_the_oracle(svl):
    rng = np.random.default_rng(0)
    for _ in range(400):
        alpha = float(rng.choice([0.0, 1.0, rng.uniform(0, 1)]))
        gamma = int(rng.integers(0, 30))
        c = float(rng.choice([0.0, rng.uniform(0, 1)]))
        assert math.isclose(svl.expected_tokens(alpha, gamma),
                            O.expected_tokens_per_call(alpha, gamma), rel_tol=1e-14)
        assert math.isclose(svl.walltime_speedup(alpha, gamma, c),
                            O.walltime_speedup(alpha, gamma, c), rel_tol=1e-14)
        assert math.isclose(svl.ops_factor(alpha, gamma, c), O.ops_factor(alpha, gamma, c),
                            rel_tol=1e-14)
        if gamma >= 1:
            assert svl.optimal_gamma(alpha, c, gamma) == O.optimal_gamma(alpha, c, gamma)


def test_printed_values_and_bad_arguments(svl):
    assert abs(svl.walltime_speedup(0.9, 10, 0.0) - 6.86) < 0.005  # Leviathan App. E
    assert abs(svl.ops_factor(0.9, 10, 0.0) - 1.6) < 0.05
    assert math.isnan(svl.expected_tokens(1.5, 3))
    assert math.isnan(svl.walltime_speedup(0.5, 3, -1.0))
    assert svl.optimal_gamma(0.5, 0.1, 0) == -1
