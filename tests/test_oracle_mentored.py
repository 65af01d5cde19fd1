"""Pins of the oracle's mentored decoding (page "推测解码的一种最优有损变体", sections 导师解码 and
解决优化问题) against things other than itself: a general-purpose constrained optimiser on the
optimisation problem as the page states it, the lossless rule (D = 0), closed-form special
cases and the sampling law of the whole accept / replace process."""

import numpy as np
import pytest
from scipy.optimize import minimize

import oracle.spec_verify_oracle as O


def _emitted(p, r, s):
    """Law of the emitted token: draft accepted with r, else replacement s (page: pi_i =
    p_i r_i + s_i (1 - sum_j p_j r_j))."""
    acc = float(np.sum(p * r))
    return p * r + s * (1.0 - acc)


def _brute_force_optimum(q, p, D, starts=12, seed=0):
    """max sum p_i r_i over 0 <= r <= 1, s in the simplex, KL(q || pi) <= D, by SLSQP from
    several random starts (tiny vocabularies only)."""
    V = q.size
    rng = np.random.default_rng(seed)

    def unpack(x):
        return x[:V], x[V:]

    def objective(x):
        r, _ = unpack(x)
        return -float(np.sum(p * r))

    def kl_con(x):
        r, s = unpack(x)
        pi = np.maximum(_emitted(p, r, s), 1e-300)
        return D - float(np.sum(q * np.log(q / pi)))

    cons = [{"type": "ineq", "fun": kl_con},
            {"type": "eq", "fun": lambda x: float(np.sum(unpack(x)[1])) - 1.0}]
    bounds = [(0.0, 1.0)] * V + [(0.0, 1.0)] * V
    best = -np.inf
    for _ in range(starts):
        x0 = np.concatenate([rng.uniform(0, 1, V), rng.dirichlet(np.ones(V))])
        res = minimize(objective, x0, method="SLSQP", bounds=bounds, constraints=cons,
                       options={"maxiter": 500, "ftol": 1e-12})
        if res.success and kl_con(res.x) > -1e-7:
            best = max(best, -res.fun)
    return best


@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("D", [0.02, 0.1, 0.4])
def test_optimum_matches_general_optimiser(seed, D):
    rng = np.random.default_rng(100 + seed)
    V = 4
    q = rng.dirichlet(np.ones(V))
    p = rng.dirichlet(np.ones(V))
    sol = O.mentored_solve(q, p, D)
    ours = float(np.sum(p * sol["r"]))
    ref = _brute_force_optimum(q, p, D, seed=seed)
    assert ref > 0
    # the general optimiser finds a feasible point: ours must be at least as good (it is the
    # optimum) and not better than what the constraint allows (checked by feasibility below)
    assert ours >= ref - 2e-5, (ours, ref)
    acc = np.sum(p * sol["r"])
    s = sol["w"] / sol["w"].sum() if sol["w"].sum() > 0 else np.zeros(V)
    pi = _emitted(p, sol["r"], s)
    assert abs(pi.sum() - 1.0) < 1e-12
    assert O.kl_divergence(q, pi) <= D + 1e-9
    assert acc <= ref + 2e-5, (acc, ref)  # no feasible point does better than the optimiser


def test_zero_bound_is_the_lossless_rule():
    rng = np.random.default_rng(7)
    for _ in range(20):
        V = 50
        q = rng.dirichlet(np.full(V, 0.3))
        p = rng.dirichlet(np.full(V, 0.3))
        sol = O.mentored_solve(q, p, 0.0)
        assert sol["alpha"] == 1.0
        np.testing.assert_allclose(sol["r"][p > 0], np.minimum(1.0, q[p > 0] / p[p > 0]),
                                   rtol=1e-12)
        w_std, _ = O.residual_weights(q, p)
        np.testing.assert_allclose(sol["w"] / sol["w"].sum(), w_std / w_std.sum(), atol=1e-12)


def test_zero_bound_sequence_equals_lossless_verify():
    rng = np.random.default_rng(8)
    V, K = 40, 4
    for t in range(30):
        q_rows = [rng.dirichlet(np.full(V, 0.5)) for _ in range(K + 1)]
        p_rows = [rng.dirichlet(np.full(V, 0.5)) for _ in range(K)]
        drafts = [int(rng.choice(V, p=p_rows[k])) for k in range(K)]
        u = rng.uniform(0, 1, K + 1)
        a = O.verify_sequence(q_rows, p_rows, drafts, u)
        b = O.mentored_verify_sequence(q_rows, p_rows, drafts, u, 0.0)
        assert a["n"] == b["n"]
        np.testing.assert_array_equal(a["tokens"], b["tokens"])
        np.testing.assert_allclose(a["a"], b["a"], rtol=1e-12)


def test_trivial_case_accepts_everything():
    q = np.array([0.4, 0.3, 0.2, 0.1, 0.0])
    p = np.array([0.35, 0.3, 0.2, 0.1, 0.05])  # KL(q||p) = 0.4 ln(0.4/0.35) ~ 0.053
    sol = O.mentored_solve(q, p, 0.06)
    assert sol["trivial"] and np.all(sol["r"] == 1.0)
    # the draft token with q = 0 is accepted too: the emitted law is p itself
    r = O.mentored_verify_sequence([q, q], [p], [4], [0.999, 0.5], 0.06)
    assert r["n"] == 1 and r["tokens"][0] == 4
    assert not O.mentored_solve(q, p, 0.05)["trivial"]


def test_monotone_in_the_bound_and_tight():
    rng = np.random.default_rng(9)
    V = 30
    q = rng.dirichlet(np.full(V, 0.4))
    p = rng.dirichlet(np.full(V, 0.4))
    prev = -1.0
    for D in [0.0, 0.001, 0.01, 0.05, 0.1, 0.3]:
        sol = O.mentored_solve(q, p, D)
        acc = float(np.sum(p * sol["r"]))
        assert acc >= prev - 1e-15
        prev = acc
        if not sol["trivial"] and D > 0:
            # the divergence constraint is active at the optimum
            assert abs(sol["kl"] - D) < 1e-9


def test_sampling_law_of_the_whole_process():
    """Draft from p, accept with r, else draw from the replacement: the emitted token follows
    pi = min(p, q/alpha) + max(0, q/beta - p) (chi-square, 1e6 trials, V = 8)."""
    rng = np.random.default_rng(10)
    V, T = 8, 1_000_000
    q = rng.dirichlet(np.ones(V))
    p = rng.dirichlet(np.ones(V))
    sol = O.mentored_solve(q, p, 0.05)
    x = rng.choice(V, size=T, p=p)
    acc = rng.uniform(0, 1, T) < sol["r"][x]
    s = sol["w"] / sol["w"].sum()
    repl = rng.choice(V, size=T, p=s)
    out = np.where(acc, x, repl)
    pi = np.minimum(p, q / sol["alpha"]) + np.maximum(0.0, q / sol["beta"] - p)
    counts = np.bincount(out, minlength=V)
    chi2 = float(np.sum((counts - T * pi) ** 2 / (T * pi)))
    assert chi2 < 18.5  # df = 7, 1% critical value
    assert O.kl_divergence(q, pi) <= 0.05 + 1e-9


def test_batch_wrapper_matches_sequence():
    rng = np.random.default_rng(11)
    B, K, V = 3, 3, 200
    t = rng.normal(0, 2, (B, K + 1, V))
    d = t[:, :K] + rng.normal(0, 1, (B, K, V))
    drafts = rng.integers(0, V, (B, K))
    u = rng.uniform(0, 1, (B, K + 1))
    out = O.mentored_spec_verify(t, d, drafts, u, 0.8, 20, 1.0, 0.05)
    for b in range(B):
        q_rows = [O.row_distribution(t[b, k], 0.8, 20) for k in range(K + 1)]
        p_rows = [O.row_distribution(d[b, k], 0.8, 20) for k in range(K)]
        r = O.mentored_verify_sequence(q_rows, p_rows, drafts[b], u[b], 0.05)
        assert r["n"] == out["n"][b]
        np.testing.assert_array_equal(r["tokens"], out["tokens"][b])


def test_planted_mistakes_fail_a_pin(monkeypatch):
    """A replacement that ignores beta (the lossless residual) breaks the emitted law's
    normalisation; a divergence computed the other way round breaks the optimiser match."""
    rng = np.random.default_rng(12)
    V = 4
    q = rng.dirichlet(np.ones(V))
    p = rng.dirichlet(np.ones(V))
    good = O.mentored_solve(q, p, 0.1)

    orig = O._mentored_beta
    monkeypatch.setattr(O, "_mentored_beta", lambda q_, p_, R: 1.0)
    bad = O.mentored_solve(q, p, 0.1)
    s = bad["w"] / bad["w"].sum()
    pi_bad = _emitted(p, bad["r"], s)
    pi_formula = np.minimum(p, q / bad["alpha"]) + bad["w"]
    assert abs(pi_formula.sum() - 1.0) > 1e-6  # the pin on sum(pi) = 1 would fail
    monkeypatch.setattr(O, "_mentored_beta", orig)

    monkeypatch.setattr(O, "kl_divergence",
                        lambda a, b: float(np.sum(b[b > 0] * np.log(b[b > 0] / np.maximum(a[b > 0], 1e-300)))))
    swapped = O.mentored_solve(q, p, 0.1)
    assert abs(float(np.sum(p * swapped["r"])) - float(np.sum(p * good["r"]))) > 1e-4
    del pi_bad
