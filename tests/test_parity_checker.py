"""CPU tests of the GPU-vs-oracle checker (tests/parity.py), with the oracle standing in for the
GPU: the checker must accept the oracle's own results with no flip, reproduce the oracle's n and
tokens from its position-by-position steps, admit a different top-p cut, an accept decision or
a final token only inside the 1e-6 band (counting each), and reject planted mistakes."""

import numpy as np
import pytest

import oracle.spec_verify_oracle as O
from workloads import synthetic as S

import parity
from parity import FLIP_BAND, Lossless, check

F32 = np.float32


def _as_gpu(o):
    """Oracle batch results in the layout of the library's outputs."""
    g = {"tokens": np.asarray(o["tokens"]).astype(np.int32),
         "num_accepted": np.asarray(o["n"]).astype(np.int32)}
    if np.asarray(o["a"]).size:
        g.update(accept_prob=np.asarray(o["a"], dtype=np.float32),
                 q_draft=np.asarray(o["q_x"], dtype=np.float32),
                 p_draft=np.asarray(o["p_x"], dtype=np.float32))
    return g


def _one(r):
    """verify_sequence's result as a batch of one."""
    return {"tokens": r["tokens"][None], "n": np.array([r["n"]]), "a": r["a"][None],
            "q_x": r["q_x"][None], "p_x": r["p_x"][None]}


CASES = [
    ("dense fp32", dict(temperature=1.0), "normal", "f32", (6, 3, 700)),
    ("top-k bf16", dict(temperature=0.7, top_k=20), "zipf", "bf16", (5, 4, 3000)),
    ("top-p fp32 lenience 0.3", dict(temperature=1.0, top_p=0.9, lenience=0.3), "zipf", "f32",
     (5, 3, 2000)),
    ("top-k + top-p bf16", dict(temperature=1.2, top_k=60, top_p=0.8), "zipf", "bf16",
     (4, 2, 1500)),
    ("greedy", dict(temperature=0.0), "normal", "bf16", (6, 4, 500)),
    ("bonus only", dict(temperature=0.9, top_p=0.95), "zipf", "f32", (6, 0, 900)),
]


def _logits(gen, dtype, shape, seed):
    B, K, V = shape
    if gen == "zipf":
        return S.zipf_logits(B, K, V, 1.1, 1.5, dtype, seed=seed)
    return S.normal_logits(B, K, V, 2.0, 1.0, 0.5, dtype, seed=seed)


@pytest.mark.parametrize("name,params,gen,dtype,shape", CASES, ids=[c[0] for c in CASES])
def test_oracle_passes_with_no_flip(name, params, gen, dtype, shape):
    t, d = _logits(gen, dtype, shape, 3)
    drafts, u = parity.make_inputs(t, d, params, 3)
    o = parity.run_oracle(t, d, drafts, u, params)
    flips, summary = check(_as_gpu(o), t, d, drafts, u, params, max_flip_frac=0.0)
    assert flips == {"accept": 0, "draw": 0, "topp": 0}
    # the checker's position-by-position oracle steps reproduce the batch oracle
    np.testing.assert_array_equal(summary["n"], o["n"])
    np.testing.assert_array_equal(summary["tokens"], o["tokens"])


def test_mentored_oracle_passes_with_no_flip():
    params = dict(temperature=1.0, top_k=30, mentor_kl=0.1)
    t, d = S.zipf_logits(4, 3, 800, 1.1, 1.5, "f32", seed=4)
    drafts, u = parity.make_inputs(t, d, params, 4)
    o = parity.run_oracle_mentored(t, d, drafts, u, params)
    flips, summary = check(_as_gpu(o), t, d, drafts, u, params, max_flip_frac=0.0)
    assert flips == {"accept": 0, "draw": 0, "topp": 0}
    np.testing.assert_array_equal(summary["n"], o["n"])
    np.testing.assert_array_equal(summary["tokens"], o["tokens"])
    # and the lossless rule does not explain mentored results
    with pytest.raises(AssertionError):
        check(_as_gpu(o), t, d, drafts, u, params, rule=Lossless(1.0), max_flip_frac=0.0)


def _base_case(seed=5):
    params = dict(temperature=1.0, top_k=40)
    t, d = S.zipf_logits(6, 3, 1200, 1.1, 1.0, "f32", seed=seed)
    drafts, u = parity.make_inputs(t, d, params, seed)
    o = parity.run_oracle(t, d, drafts, u, params)
    return params, t, d, drafts, u, o


def _other_token(w, u, tok):
    """A token other than tok with positive weight whose CDF interval is far from u W."""
    for cand in np.nonzero(w > 0)[0]:
        if cand != tok and O.inverse_cdf_margin(w, u, int(cand)) > 1e-3:
            return int(cand)
    raise AssertionError("no such token")


def test_planted_mistakes_are_rejected():
    params, t, d, drafts, u, o = _base_case()
    g0 = _as_gpu(o)
    K = drafts.shape[1]
    b = int(np.argmax(o["n"] < K))  # a sequence that stopped at a rejection
    n = int(o["n"][b])
    tf, df = t.float().numpy(), d.float().numpy()
    q = O.row_distribution(tf[b, n], F32(1.0), 40)
    p = O.row_distribution(df[b, n], F32(1.0), 40)
    w, _ = O.residual_weights(q, p)

    def bad(mut):
        g = {k: v.copy() for k, v in g0.items()}
        mut(g)
        with pytest.raises(AssertionError):
            check(g, t, d, drafts, u, params)

    bad(lambda g: g["tokens"].__setitem__((b, n), _other_token(w, float(u[b, K]), o["tokens"][b, n])))
    bad(lambda g: g["accept_prob"].__setitem__((b, 0), g["accept_prob"][b, 0] + 1e-3))
    bad(lambda g: g["q_draft"].__setitem__((b, K - 1), g["q_draft"][b, K - 1] * 1.01 + 1e-4))
    bad(lambda g: g["tokens"].__setitem__((b, K), 7))  # padding
    bad(lambda g: (g["num_accepted"].__setitem__(b, n + 1),
                   g["tokens"].__setitem__((b, n), drafts[b, n])))
    b2 = int(np.argmax(o["n"] > 0))
    bad(lambda g: g["tokens"].__setitem__((b2, 0), (int(drafts[b2, 0]) + 1) % 1200))


def _near_boundary_row(rng, V=64):
    """A row and a float32 P lying 2e-7..4e-7 above a running sum c_j of its top-p order, with
    c_{j-1} and c_{j+1} far from P: the cut at j is admissible, the one at j - 1 is not."""
    while True:
        z = rng.normal(size=V).astype(np.float32)
        diag = {}
        O.row_distribution(z, F32(1.0), 0, F32(0.5), diag)
        c = diag["topp_cumsum"]
        j = int(np.searchsorted(c, 0.6))
        P = F32(c[j] + 3e-7)
        if not 2e-7 < float(P) - c[j] < 4e-7:
            continue
        if c[j + 1] - float(P) > 1e-3 and float(P) - c[j - 1] > 1e-3:
            return z, P, c, j


def test_topp_neighbouring_cut_admitted_only_inside_the_band():
    rng = np.random.default_rng(6)
    z, P, c, j = _near_boundary_row(rng)
    T = F32(1.0)
    diag = {}
    q_own = O.row_distribution(z, T, 0, P, diag)
    assert diag["topp_cut"] == j + 1 and diag["topp_margin"] < FLIP_BAND
    readings = parity.row_readings(z, T, 0, P)
    assert len(readings) == 2  # the oracle's cut (j + 1) and the one at j
    order = np.lexsort((np.arange(z.size), -O.row_distribution(z, T, 0, F32(1.0))))
    x = int(order[j])  # kept by both admissible cuts (renormalised differently), not below
    zd = rng.normal(size=z.size).astype(np.float32)
    p_row = O.row_distribution(zd, T, 0, P)
    t = np.stack([z, z])[None]  # target rows 0 and 1 (bonus)
    dr = zd[None, None]
    drafts = np.array([[x]])
    u = np.array([[0.999, 0.3]], dtype=np.float32)
    params = dict(temperature=1.0, top_p=float(P))

    def gpu_with(q0):
        return _as_gpu(_one(O.verify_sequence([q0, q_own], [p_row], [x], [0.999, 0.3])))

    # the cut at j (inside the band): explained, one top-p flip
    q_in = O.row_distribution(z, T, 0, float(c[j]))
    assert not parity._close(q_in[x], q_own[x])
    flips, _ = check(gpu_with(q_in), t, dr, drafts, u, params)
    assert flips["topp"] == 1
    # the cut at j - 1 (outside the band): rejected
    q_out = O.row_distribution(z, T, 0, float(c[j - 1]))
    assert q_out[x] == 0
    with pytest.raises(AssertionError):
        check(gpu_with(q_out), t, dr, drafts, u, params)


def test_accept_and_draw_flips_only_inside_the_band():
    params, t, d, drafts, u, o = _base_case(8)
    K = drafts.shape[1]
    inner = np.nonzero((o["a"][:, 0] > 1e-3) & (o["a"][:, 0] < 0.999))[0]
    assert inner.size, "no position with 0 < a < 1"
    b = int(inner[0])
    tf, df = t.float().numpy(), d.float().numpy()
    # accept flip: move u[b, 0] to a_0 - 5e-7 (then a_0 - 5e-6) and report a rejection
    a0 = float(o["a"][b, 0])
    for delta, ok in ((5e-7, True), (5e-6, False)):
        uu = u.copy()
        uu[b, 0] = F32(a0 - delta)  # the oracle accepts (u < a)
        r = O.verify_sequence(
            [O.row_distribution(tf[b, k], F32(1.0), 40) for k in range(K + 1)],
            [O.row_distribution(df[b, k], F32(1.0), 40) for k in range(K)],
            drafts[b], uu[b])
        assert r["n"] >= 1
        # a GPU that rejected at 0: n = 0 and the residual draw at position 0
        q = O.row_distribution(tf[b, 0], F32(1.0), 40)
        p = O.row_distribution(df[b, 0], F32(1.0), 40)
        w, _ = O.residual_weights(q, p)
        g = _as_gpu(o)
        g["num_accepted"][b] = 0
        g["tokens"][b] = -1
        g["tokens"][b, 0] = O.inverse_cdf(w, float(uu[b, K]))
        if ok:
            flips, _ = check(g, t, d, drafts, uu, params)
            assert flips["accept"] == 1
        else:
            with pytest.raises(AssertionError):
                check(g, t, d, drafts, uu, params)
    # draw flip: put u W 5e-7 W (then 5e-6 W) below the start of the drawn token's interval
    n = int(o["n"][b])
    q = O.row_distribution(tf[b, n], F32(1.0), 40)
    w = q if n == K else O.residual_weights(q, O.row_distribution(df[b, n], F32(1.0), 40))[0]
    C = np.cumsum(w)
    W = C[-1]
    pos = np.nonzero(w > 0)[0]
    tok = int(pos[len(pos) // 2])
    lo = C[tok - 1] / W
    for delta, ok in ((5e-7, True), (5e-6, False)):
        uu = u.copy()
        uu[b, K] = F32(lo - delta)
        assert (lo - 1e-6 < float(uu[b, K]) < lo) == ok
        oo = parity.run_oracle(t, d, drafts, uu, params)
        g = _as_gpu(oo)
        assert g["tokens"][b, n] != tok
        g["tokens"][b, n] = tok
        if ok:
            flips, _ = check(g, t, d, drafts, uu, params)
            assert flips["draw"] == 1
        else:
            with pytest.raises(AssertionError):
                check(g, t, d, drafts, uu, params)


def test_flip_cap():
    params, t, d, drafts, u, o = _base_case(9)
    g = _as_gpu(o)
    check(g, t, d, drafts, u, params, max_flips=0)
    assert parity.FLIP_LOG[-1][1] == {"accept": 0, "draw": 0, "topp": 0}
